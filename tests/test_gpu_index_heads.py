"""Index scoring with 1, 2 and 4 index heads, one shared table or one per KV head, in
the plain scorer and in the fused append + score launch: block scores against the
oracle's on the same keys (the step's new tokens appended first by the oracle)."""
import numpy as np
import pytest
import torch

from oracle import msa_oracle as O
from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M


@pytest.mark.parametrize("hi,hkv,tables", [(1, 2, 1), (2, 2, 1), (2, 2, 2), (4, 1, 1), (4, 2, 2), (4, 4, 4),
                                           (4, 4, 1)])
@pytest.mark.parametrize("fused", [False, True])
def test_scores_for_index_head_counts(M, hi, hkv, tables, fused):
    wl = W.small(W.FMT_NVFP4, [1000, 2600, 130, 640], 3, num_kv_heads=hkv, k=5, seed=97 + hi)
    print("index heads", hi, "KV heads", hkv, "tables", tables, "fused", fused, flush=True)
    q_idx_bits = np.ascontiguousarray(wl.q_idx[:, :hi])
    w = np.ascontiguousarray(wl.w[:, :hi])
    pool = G.gpu_pool(M, wl)
    step, _, _, _, app = G.gpu_step_inputs(M, wl, tables)
    q_idx = G.dev_bf16(q_idx_bits)
    wt = torch.from_numpy(w).cuda()
    shape = (wl.num_rows, tables, wl.max_blocks) if tables > 1 else (wl.num_rows, wl.max_blocks)
    scores = torch.empty(shape, dtype=torch.float32, device="cuda")
    if fused:
        M.msa_append_score_select(pool, step, q_idx, wt, wl.k, 0, 1, scores, slot=app[0], k_new=app[1],
                                  v_new=app[2], idx_k_new=app[3])
    else:
        M.msa_kv_append(pool, *app)
        M.msa_index_score(pool, step, q_idx, wt, scores)
    torch.cuda.synchronize()
    ref = O.index_score(G.oracle_pool(wl, kv_blocks={}), wl.block_table, wl.row_seq, wl.row_pos, q_idx_bits, w,
                        wl.max_blocks, tables)
    G.assert_scores_close(scores.cpu().numpy().reshape(wl.num_rows * tables, -1),
                          ref.reshape(wl.num_rows * tables, -1))


@pytest.mark.parametrize("hi,hkv,tables", [(2, 2, 2), (4, 4, 4), (1, 2, 1)])
def test_scores_for_index_head_counts_nvfp4_keys(M, hi, hkv, tables):
    """The same with NVFP4 index keys (the fused launch encodes the new tokens' keys)."""
    wl = W.small(W.FMT_FP8, [1000, 2600, 130], 2, num_kv_heads=hkv, k=5, seed=98 + hi, index_fmt=W.IDX_NVFP4)
    print("NVFP4 index keys, index heads", hi, "tables", tables, flush=True)
    q_idx_bits = np.ascontiguousarray(wl.q_idx[:, :hi])
    w = np.ascontiguousarray(wl.w[:, :hi])
    pool = G.gpu_pool(M, wl)
    step, _, _, _, app = G.gpu_step_inputs(M, wl, tables)
    shape = (wl.num_rows, tables, wl.max_blocks) if tables > 1 else (wl.num_rows, wl.max_blocks)
    scores = torch.empty(shape, dtype=torch.float32, device="cuda")
    M.msa_append_score_select(pool, step, G.dev_bf16(q_idx_bits), torch.from_numpy(w).cuda(), wl.k, 0, 1, scores,
                              slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
    torch.cuda.synchronize()
    ref = O.index_score(G.oracle_pool(wl, kv_blocks={}), wl.block_table, wl.row_seq, wl.row_pos, q_idx_bits, w,
                        wl.max_blocks, tables)
    G.assert_scores_close(scores.cpu().numpy().reshape(wl.num_rows * tables, -1),
                          ref.reshape(wl.num_rows * tables, -1))
