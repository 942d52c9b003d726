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


@pytest.mark.parametrize("hi", [1, 2, 4])
@pytest.mark.parametrize("rows_per_req", [3, 5, 8])
def test_stated_rows_per_seq_gives_identical_scores(M, hi, rows_per_req):
    """With every request holding the same number of rows, stating it (msa_step_t
    rows_per_seq) launches one scoring workgroup row per group of a request's rows; the
    scores, and the fused launch's selections, are bit-identical to those of the
    one-row-per-grid-row launch (rows_per_seq = 0). Row counts of 3, 5 and 8 give whole
    and partial groups for 16 / hi rows per group."""
    wl = W.small(W.FMT_NVFP4, [1500, 2600, 700], rows_per_req, num_kv_heads=2, k=5, seed=96 + hi,
                 rows_per_req=rows_per_req)
    print("stated rows per request", rows_per_req, "index heads", hi, flush=True)
    q_idx = G.dev_bf16(np.ascontiguousarray(wl.q_idx[:, :hi]))
    wt = torch.from_numpy(np.ascontiguousarray(wl.w[:, :hi])).cuda()
    pool = G.gpu_pool(M, wl)
    sl, kb, vb, ib = wl.step_tokens()
    app = (torch.from_numpy(sl).cuda(), G.dev_bf16(kb), G.dev_bf16(vb), G.dev_bf16(ib))
    M.msa_kv_append(pool, *app)
    out = {}
    for stated in (0, None):
        step = M.Step(wl.block_table, wl.row_seq, wl.row_pos, rows_per_seq=stated)
        assert step.rows_per_seq == (0 if stated == 0 else rows_per_req)
        scores = torch.full((wl.num_rows, wl.max_blocks), 5.0, dtype=torch.float32, device="cuda")
        M.msa_index_score(pool, step, q_idx, wt, scores)
        fused = torch.full_like(scores, 5.0)
        sel = torch.full((wl.num_rows, wl.k), -7, dtype=torch.int32, device="cuda")
        pages = torch.full_like(sel, -7)
        counters = torch.zeros(wl.num_rows, dtype=torch.int32, device="cuda")
        M.msa_append_score_select(pool, step, q_idx, wt, wl.k, 0, 1, fused, sel=sel, sel_pages=pages,
                                  counters=counters)
        torch.cuda.synchronize()
        out[stated] = (scores, fused, sel, pages)
    for a, b in zip(out[0], out[None]):
        assert torch.equal(a, b)
    ref = O.index_score(G.oracle_pool(wl, kv_blocks={}), wl.block_table, wl.row_seq, wl.row_pos,
                        np.ascontiguousarray(wl.q_idx[:, :hi]), np.ascontiguousarray(wl.w[:, :hi]), wl.max_blocks, 1)
    G.assert_scores_close(out[None][0].cpu().numpy(), ref.reshape(wl.num_rows, -1))


def test_wrong_rows_per_seq_is_reported_by_the_debug_library(M):
    """A stated row count that matches num_rows / num_seqs but not row_seq (3 and 5 rows
    stated as 4 and 4) is reported as MSA_DEBUG_BAD_SEQ by the debug library; every
    access stays in bounds (the group's rows lie inside [0, num_rows))."""
    dbg = M.load_library(M.DEBUG_LIB_PATH)
    wl = W.small(W.FMT_NVFP4, [3000, 3000], 4, num_kv_heads=1, k=4, seed=91)
    row_seq = wl.row_seq.copy()
    row_seq[3] = 1                        # request 0: rows 0..2, request 1: rows 3..7
    pool = G.gpu_pool(M, wl)
    step = M.Step(wl.block_table, row_seq, wl.row_pos, rows_per_seq=4)
    scores = torch.empty((wl.num_rows, wl.max_blocks), dtype=torch.float32, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with M.use_library(dbg):
        M.msa_debug_set_error_word(err)
        try:
            M.msa_index_score(pool, step, G.dev_bf16(wl.q_idx), torch.from_numpy(wl.w).cuda(), scores)
            torch.cuda.synchronize()
        finally:
            M.msa_debug_set_error_word(None)
    assert int(err.item()) == 2            # MSA_DEBUG_BAD_SEQ
