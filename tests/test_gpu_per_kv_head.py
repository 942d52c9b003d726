"""Per-KV-head selection tables (one selection per query row and KV head, each scored
from its share of the index heads): scores, selections, outputs and partials of the HIP
path against the oracle, through every entry point that takes a selection."""
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


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("hkv,num_splits,fused", [(2, 2, False), (2, 2, True), (4, 1, True), (4, 3, False),
                                                  (4, 4, True)])
def test_per_kv_head_step_parity(M, fmt, hkv, num_splits, fused):
    wl = W.small(fmt, [1000, 2600, 130, 640], 3, num_kv_heads=hkv, k=5, seed=81 + hkv)
    _print("per-KV-head step", wl.name, "hkv", hkv, "splits", num_splits, "fused", fused)
    bufs = G.check_step_parity(M, wl, num_splits, fused, tables=hkv)
    sel = bufs.sel.cpu().numpy()
    # the tables really differ between KV heads somewhere (else the test shows nothing)
    assert any(not np.array_equal(sel[r, 0], sel[r, t]) for r in range(wl.num_rows) for t in range(1, hkv))


def test_per_kv_head_fused_score_select_matches_separate(M):
    """msa_append_score_select with a selection writes the same per-table scores and
    tables as msa_kv_append + msa_index_score + msa_select_topk."""
    wl = W.small(W.FMT_NVFP4, [3000, 700, 129], 2, num_kv_heads=4, k=6, seed=91)
    _print("per-KV-head fused score+select", wl.name)
    T = 4
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl, T)
    pa, pb = G.gpu_pool(M, wl), None
    pb = pa.clone()
    ra = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 1, sel_tables=T)
    rb = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 1, sel_tables=T)
    M.msa_kv_append(pa, *app)
    M.msa_index_score(pa, step, q_idx, w, ra.block_scores)
    M.msa_select_topk(step, ra.block_scores, wl.k, 0, 1, ra.sel, ra.sel_pages)
    M.msa_append_score_select(pb, step, q_idx, w, wl.k, 0, 1, rb.block_scores, rb.sel, rb.sel_pages,
                              rb.score_counters, slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
    torch.cuda.synchronize()
    assert np.array_equal(ra.block_scores.cpu().numpy(), rb.block_scores.cpu().numpy())
    assert np.array_equal(ra.sel.cpu().numpy(), rb.sel.cpu().numpy())
    assert np.array_equal(ra.sel_pages.cpu().numpy(), rb.sel_pages.cpu().numpy())
    assert int(rb.score_counters.abs().sum()) == 0
    bt = wl.block_table
    sel = ra.sel.cpu().numpy()
    pages = ra.sel_pages.cpu().numpy()
    for r in range(wl.num_rows):
        for t in range(T):
            exp = [bt[wl.row_seq[r], b] if b >= 0 else -1 for b in sel[r, t]]
            assert list(pages[r, t]) == exp


def test_per_kv_head_select_bit_exact_on_fp32_scores(M):
    """Same fp32 scores on both sides, heavy exact ties, rows both below and above the
    one-wave limit: per-(row, table) selections agree bit for bit."""
    rng = np.random.default_rng(92)
    for nb_max, k in ((257, 16), (3000, 32)):
        rows, T = 5, 4
        pos = rng.integers(0, nb_max * 128, rows).astype(np.int32)
        pos[0] = nb_max * 128 - 1
        S = np.full((rows, T, nb_max), -np.inf, np.float32)
        for r in range(rows):
            nb = pos[r] // 128 + 1
            S[r, :, :nb] = np.round(rng.standard_normal((T, nb)) * 4).astype(np.float32)
        _print("per-table select", nb_max, k)
        step = M.Step(np.zeros((1, nb_max), np.int32), np.zeros(rows, np.int32), pos, sel_tables=T)
        sel = torch.empty((rows, T, k), dtype=torch.int32, device="cuda")
        M.msa_select_topk(step, torch.from_numpy(S).cuda(), k, 0, 1, sel)
        ref = O.select_topk(S.astype(np.float64), pos, k)
        assert np.array_equal(sel.cpu().numpy(), ref)


def test_per_kv_head_step_parity_select_in_scoring_launch(M):
    wl = W.small(W.FMT_NVFP4, [1000, 2600, 130, 640], 3, num_kv_heads=4, k=5, seed=93)
    _print("per-KV-head step, select in scoring launch", wl.name)
    G.check_step_parity(M, wl, 2, True, tables=4, select_in="score")
