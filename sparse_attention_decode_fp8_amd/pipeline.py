"""Sequencing of one decode step through the five library calls.

This only allocates output buffers once and issues the five calls in order on one
stream; all arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import _lib as L


class DecodeBuffers:
    """Per-step outputs and the split-KV workspace for a fixed geometry."""

    def __init__(self, num_rows, num_q_heads, max_blocks, k, num_splits, device="cuda"):
        self.k, self.num_splits = k, num_splits
        self.block_scores = torch.empty((num_rows, max_blocks), dtype=torch.float32, device=device)
        self.sel = torch.empty((num_rows, k), dtype=torch.int32, device=device)
        self.part_o = torch.empty((num_rows, num_q_heads, num_splits, L.HEAD_DIM),
                                  dtype=torch.float32, device=device)
        self.part_ml = torch.empty((num_rows, num_q_heads, num_splits, 2), dtype=torch.float32,
                                   device=device)
        self.out = torch.empty((num_rows, num_q_heads, L.HEAD_DIM), dtype=torch.bfloat16, device=device)


def run_step(pool, step, bufs: DecodeBuffers, q, q_idx, w, softmax_scale, slot=None, k_new=None,
             v_new=None, idx_k_new=None, n_init=0, n_local=1, stream=None):
    """append -> index score -> select -> sparse decode -> combine, on one stream."""
    if slot is not None and slot.numel() > 0:
        L.msa_kv_append(pool, slot, k_new, v_new, idx_k_new, stream)
    L.msa_index_score(pool, step, q_idx, w, bufs.block_scores, stream)
    L.msa_select_topk(step, bufs.block_scores, bufs.k, n_init, n_local, bufs.sel, stream)
    L.msa_sparse_decode(pool, step, q, bufs.sel, bufs.k, softmax_scale, bufs.num_splits,
                        bufs.part_o, bufs.part_ml, stream)
    L.msa_combine(step.num_rows, q.shape[1], L.HEAD_DIM, bufs.num_splits, bufs.part_o, bufs.part_ml,
                  bufs.out, stream)
    return bufs.out


def default_num_splits(k: int) -> int:
    """Split count used by the benchmark and the full-size parity tests: one split per
    four selected pages (each split is one workgroup of four waves, one page per wave)."""
    return max(1, (k + 3) // 4)
