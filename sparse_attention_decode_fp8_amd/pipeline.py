"""Sequencing of one decode step through the library calls.

This only allocates output buffers once and issues the calls in order on one stream;
all arithmetic happens in the HIP kernels.
"""
from __future__ import annotations

import torch

from . import _lib as L


def default_num_splits(k: int, pairs: int) -> int:
    """Split count used by the benchmark and the full-size parity tests, for `pairs`
    (query row, KV head) pairs: enough splits for about 256 decode workgroups (one per
    compute unit), a power of two, at most min(k, 16) (the fused merge takes at most 16
    splits). Few pairs (a small batch) are spread over many workgroups whose partials
    are merged, down to one block per split; many pairs fill the GPU on their own and
    skip the merge (one split writes its output directly)."""
    target = max(1, 256 // max(1, pairs))
    s = 1
    while s * 2 <= min(target, k, 16):
        s *= 2
    return s


class DecodeBuffers:
    """Per-step outputs and the split-KV workspaces for a fixed geometry: part_o /
    part_ml receive the partials of the separate msa_sparse_decode call; merge_o /
    merge_ml (two exchange buffers) and counters (one state word per row and KV head)
    are the fused entries' merge workspace, set up here for num_splits; score_x (idle
    words) and score_words (zeros) are the single-launch step's score exchange. With
    sel_tables > 1 (one selection per KV head) block_scores, sel and sel_pages have a
    table axis after the row."""

    def __init__(self, num_rows, num_q_heads, max_blocks, k, num_splits, device="cuda", sel_tables=1):
        self.k, self.num_splits = k, num_splits
        t = (sel_tables,) if sel_tables > 1 else ()
        self.block_scores = torch.empty((num_rows, *t, max_blocks), dtype=torch.float32, device=device)
        self.sel = torch.empty((num_rows, *t, k), dtype=torch.int32, device=device)
        self.sel_pages = torch.empty((num_rows, *t, k), dtype=torch.int32, device=device)
        self.part_o = torch.empty((num_rows, num_q_heads, num_splits, L.HEAD_DIM),
                                  dtype=torch.float32, device=device)
        self.part_ml = torch.empty((num_rows, num_q_heads, num_splits, 2), dtype=torch.float32,
                                   device=device)
        hkv = num_q_heads // 16   # pair-major: [rows][KV heads][2 buffers][16 heads][splits][...]
        self.merge_o = torch.empty((num_rows, hkv, 2, 16, num_splits, L.HEAD_DIM), dtype=torch.float32,
                                   device=device)
        self.merge_ml = torch.empty((num_rows, hkv, 2, 16, num_splits, 2), dtype=torch.float32, device=device)
        self.counters = torch.empty((num_rows, num_q_heads // 16), dtype=torch.int32, device=device)
        L.msa_merge_workspace_init(num_rows, num_q_heads, L.HEAD_DIM, num_splits, self.merge_o,
                                   self.merge_ml, self.counters)
        self.score_counters = torch.zeros(num_rows, dtype=torch.int32, device=device)
        self.score_x = torch.empty((num_rows, max_blocks), dtype=torch.float32, device=device)
        self.score_words = torch.empty(num_rows, dtype=torch.int32, device=device)
        L.msa_step_workspace_init(num_rows, max_blocks, self.score_x, self.score_words)
        self.out = torch.empty((num_rows, num_q_heads, L.HEAD_DIM), dtype=torch.bfloat16, device=device)


# New tokens per step up to which the append rides in the scoring launch: one slot per
# lane of a scoring wave; beyond it each wave would loop over the slots.
FUSED_APPEND_MAX = 64


def run_step(pool, step, bufs: DecodeBuffers, q, q_idx, w, softmax_scale, slot=None, k_new=None,
             v_new=None, idx_k_new=None, n_init=0, n_local=1, fused=True, stream=None,
             select_in="decode", single_launch=False):
    """One decode step on one stream: append -> index score -> select -> sparse decode
    -> combine. fused=True runs two launches (with single_launch, the whole step as one
    msa_decode_step launch where its shape allows, else the two): append + score, then
    select + decode + combine (select_in="decode":
    the selection is repeated by every decode workgroup, which measured faster on every
    workload than one selection per row at the end of the scoring launch), or append +
    score + select, then decode + combine (select_in="score"). With more than
    FUSED_APPEND_MAX new tokens the two-launch path appends in a launch of its own before
    scoring. fused=False issues the five separate calls. Returns the output tensor."""
    if fused and single_launch and select_in == "decode":
        if L.msa_decode_step(pool, step, q_idx, w, q, bufs.k, n_init, n_local, softmax_scale, bufs.num_splits,
                             bufs.score_x, bufs.score_words, bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                             block_scores=bufs.block_scores, sel=bufs.sel, sel_pages=bufs.sel_pages, slot=slot,
                             k_new=k_new, v_new=v_new, idx_k_new=idx_k_new, stream=stream, unsupported_ok=True):
            return bufs.out
    if fused:
        if select_in == "decode":
            if slot is not None and slot.numel() > FUSED_APPEND_MAX:
                # many new tokens: every scoring wave would scan them all for its page,
                # so the append runs first and the scorer without it
                L.msa_kv_append(pool, slot, k_new, v_new, idx_k_new, stream)
                L.msa_index_score(pool, step, q_idx, w, bufs.block_scores, stream)
            else:
                L.msa_append_score_select(pool, step, q_idx, w, bufs.k, n_init, n_local, bufs.block_scores,
                                          slot=slot, k_new=k_new, v_new=v_new, idx_k_new=idx_k_new,
                                          stream=stream)
            L.msa_select_decode_combine(pool, step, q, bufs.block_scores, bufs.k, n_init, n_local,
                                        softmax_scale, bufs.num_splits, bufs.merge_o, bufs.merge_ml,
                                        bufs.counters, bufs.out, sel=bufs.sel, sel_pages=bufs.sel_pages,
                                        stream=stream)
        elif select_in == "score":
            L.msa_append_score_select(pool, step, q_idx, w, bufs.k, n_init, n_local, bufs.block_scores,
                                      sel=bufs.sel, sel_pages=bufs.sel_pages, counters=bufs.score_counters,
                                      slot=slot, k_new=k_new, v_new=v_new, idx_k_new=idx_k_new,
                                      stream=stream)
            L.msa_sparse_decode_combine(pool, step, q, bufs.sel, bufs.k, softmax_scale, bufs.num_splits,
                                        bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                                        sel_pages=bufs.sel_pages, stream=stream)
        else:
            raise ValueError(f"select_in must be 'decode' or 'score', not {select_in!r}")
        return bufs.out
    if slot is not None and slot.numel() > 0:
        L.msa_kv_append(pool, slot, k_new, v_new, idx_k_new, stream)
    L.msa_index_score(pool, step, q_idx, w, bufs.block_scores, stream)
    L.msa_select_topk(step, bufs.block_scores, bufs.k, n_init, n_local, bufs.sel, bufs.sel_pages,
                      stream)
    L.msa_sparse_decode(pool, step, q, bufs.sel, bufs.k, softmax_scale, bufs.num_splits,
                        bufs.part_o, bufs.part_ml, sel_pages=bufs.sel_pages, stream=stream)
    L.msa_combine(step.num_rows, q.shape[1], L.HEAD_DIM, bufs.num_splits, bufs.part_o,
                  bufs.part_ml, bufs.out, stream)
    return bufs.out
