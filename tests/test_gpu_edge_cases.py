"""Edge cases of the HIP path against the oracle: calls with nothing to do, contexts of
a few tokens and exact page boundaries, and the largest top-k and split count."""
import numpy as np
import pytest
import torch

from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_splits,fused", [(1, False), (2, True)])
def test_page_boundary_contexts(M, fmt, num_splits, fused):
    # cached 0 / 1 / 127 / 128 / 255 / 383 / 1000 tokens + 1 appended: the new token is
    # the first, last or only token of its page; rows with nb <= k take the dense path
    wl = W.small(fmt, [0, 1, 127, 128, 255, 383, 1000], 1, num_kv_heads=1, k=2, seed=51)
    print("page boundary contexts", wl.name, "splits", num_splits, "fused", fused, flush=True)
    G.check_step_parity(M, wl, num_splits, fused)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_splits,fused", [(16, True), (3, False)])
def test_max_topk(M, fmt, num_splits, fused):
    # k = 64 (the largest supported), 16 splits (the most the fused merge takes);
    # 8191 + 1 = 64 blocks is dense, 8191 + 2 = 65 blocks selects
    wl = W.small(fmt, [9000, 8191, 300], 2, num_kv_heads=2, k=64, seed=52)
    print("max top-k", wl.name, "splits", num_splits, "fused", fused, flush=True)
    G.check_step_parity(M, wl, num_splits, fused)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("fused", [True, False])
def test_uneven_rows_per_request(M, fmt, fused):
    # requests with 1, 3, 0, 2 and 3 query rows: the row -> request map is not uniform
    full = W.small(fmt, [700, 2600, 900, 1300, 4000], 3, num_kv_heads=2, k=5, seed=54)
    wl = W.keep_rows(full, [2, 3, 4, 5, 10, 11, 12, 13, 14])
    assert list(wl.row_seq) == [0, 1, 1, 1, 3, 3, 4, 4, 4]
    print("uneven rows", wl.name, "fused", fused, flush=True)
    G.check_step_parity(M, wl, 2, fused)


def test_nothing_to_do_leaves_outputs_untouched(M):
    wl = W.small(W.FMT_NVFP4, [300], 1, num_kv_heads=1, k=2, seed=53)
    pool = G.gpu_pool(M, wl)
    before = {k: v.clone() for k, v in pool.arrays().items()}
    empty = M.Step(wl.block_table, np.zeros(0, np.int32), np.zeros(0, np.int32))
    bufs = M.DecodeBuffers(1, wl.num_heads, wl.max_blocks, wl.k, 2)
    for t in (bufs.block_scores, bufs.sel, bufs.sel_pages, bufs.part_o, bufs.part_ml):
        t.fill_(7)
    bufs.out.fill_(7.0)
    q = torch.zeros((1, wl.num_heads, 128), dtype=torch.bfloat16, device="cuda")
    q_idx = torch.zeros((1, 4, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((1, 4), dtype=torch.float32, device="cuda")
    no_slot = torch.zeros(0, dtype=torch.int64, device="cuda")
    M.msa_kv_append(pool, no_slot)
    M.msa_index_score(pool, empty, q_idx, w, bufs.block_scores)
    M.msa_select_topk(empty, bufs.block_scores, wl.k, 0, 1, bufs.sel, bufs.sel_pages)
    M.msa_sparse_decode(pool, empty, q, bufs.sel, wl.k, wl.softmax_scale, 2, bufs.part_o, bufs.part_ml)
    M.msa_combine(0, wl.num_heads, 128, 2, bufs.part_o, bufs.part_ml, bufs.out)
    M.msa_append_score_select(pool, empty, q_idx, w, wl.k, 0, 1, bufs.block_scores)
    M.msa_select_decode_combine(pool, empty, q, bufs.block_scores, wl.k, 0, 1, wl.softmax_scale, 2,
                                bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out)
    torch.cuda.synchronize()
    for k, v in pool.arrays().items():
        assert torch.equal(v, before[k]), k
    for t in (bufs.block_scores, bufs.sel, bufs.sel_pages, bufs.part_o, bufs.part_ml):
        assert bool((t == 7).all())
    assert bool((bufs.out.float() == 7.0).all())
    assert bool((bufs.counters == (2 << 26)).all())   # as set up for 2 splits
