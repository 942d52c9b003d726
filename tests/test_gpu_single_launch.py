"""msa_decode_step (the whole step in one launch) against the two fused launches and the
oracle: outputs, selections, block scores and the appended pool bytes bit for bit, over
consecutive calls that reuse the score exchange (which every call must leave idle)."""
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


def _print(*a):
    print(*a, flush=True)


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t


def _run(M, wl, pool, bufs, step, q, q_idx, w, app, single):
    kw = dict(slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3]) if app is not None else {}
    if single:
        M.msa_decode_step(pool, step, q_idx, w, q, wl.k, wl.n_init, wl.n_local, wl.softmax_scale, bufs.num_splits,
                          bufs.score_x, bufs.score_words, bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                          block_scores=bufs.block_scores, sel=bufs.sel, sel_pages=bufs.sel_pages, **kw)
    else:
        M.run_step(pool, step, bufs, q, q_idx, w, wl.softmax_scale, n_init=wl.n_init, n_local=wl.n_local,
                   single_launch=False, **kw)
    torch.cuda.synchronize()
    return [_bits(t).clone() for t in (bufs.out, bufs.sel, bufs.sel_pages, bufs.block_scores)]


SHAPES = [
    # fmt, ctx_lens, n_append (= rows per request), KV heads, k, splits, seed
    (W.FMT_NVFP4, [1000, 2600, 130, 640], 3, 2, 5, 2, 51),
    (W.FMT_FP8, [1000, 2600, 130, 640], 3, 2, 5, 3, 52),
    (W.FMT_NVFP4, [3000, 900], 1, 2, 2, 1, 60),                   # one split: direct output, 8 waves
    (W.FMT_FP8, [900, 300, 1000], 1, 2, 1, 1, 61),                # k = 1: direct output, 4 waves
    (W.FMT_NVFP4, [1500, 700, 2600], 4, 2, 4, 2, 53),            # groups of 4 rows
    (W.FMT_FP8, [4096], 0, 1, 8, 8, 54),                          # one split per block, no append
    (W.FMT_NVFP4, [4095, 4097, 8192, 300], 1, 4, 8, 4, 55),       # page-boundary contexts
    (W.FMT_NVFP4, [32768, 32768], 1, 4, 16, 8, 56),               # two requests of the 32k workload
    (W.FMT_FP8, [6000, 129], 2, 3, 6, 3, 57),                     # 3 KV heads, 3 splits
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"fmt{s[0]}_L{s[1][0]}_r{s[2]}_h{s[3]}_k{s[4]}_s{s[5]}")
def test_single_launch_equals_two_launches(M, shape):
    fmt, lens, n_app, hkv, k, ns, seed = shape
    wl = W.small(fmt, lens, n_app, num_kv_heads=hkv, k=k, seed=seed)
    _print("single launch vs two launches", wl.name, lens, "rows", wl.num_rows, "KV heads", hkv, "k", k,
           "splits", ns)
    pool_s = G.gpu_pool(M, wl)
    pool_t = pool_s.clone()
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    assert step.rows_per_seq == max(1, n_app)
    bufs_s = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    bufs_t = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    ref = _run(M, wl, pool_t, bufs_t, step, q, q_idx, w, app, single=False)
    for call in range(3):   # the same step again (the append rewrites the same bytes)
        got = _run(M, wl, pool_s, bufs_s, step, q, q_idx, w, app, single=True)
        for name, a, b in zip(("out", "sel", "sel_pages", "block_scores"), got, ref):
            assert torch.equal(a, b), (call, name)
        G.assert_score_exchange_idle(bufs_s)
        if ns > 1:
            G.assert_merge_ready(bufs_s)
    for name, a in pool_s.arrays().items():
        assert torch.equal(a, pool_t.arrays()[name]), f"pool array {name} differs after the append"


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_single_launch_rows_that_grow_and_shrink(M, fmt):
    """Consecutive calls on one exchange with different row lengths (fewer visible
    blocks, then more, then fewer): each equals the two-launch step on its own inputs."""
    wl = W.small(fmt, [3000, 5200, 2600, 4100], 1, num_kv_heads=2, k=6, seed=58)
    _print("single launch, changing row lengths", wl.name)
    pool = G.gpu_pool(M, wl)
    step_full, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    bufs_s = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 2)
    bufs_t = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 2)
    for cut in (900, 0, 2000, 0):
        pos = np.maximum(wl.row_pos - cut, 0)
        step = M.Step(wl.block_table, wl.row_seq, pos)
        # no append (its slots belong to the full positions); the same inputs for both paths
        ref = _run(M, wl, pool, bufs_t, step, q, q_idx, w, None, single=False)
        got = _run(M, wl, pool, bufs_s, step, q, q_idx, w, None, single=True)
        for name, a, b in zip(("out", "sel", "sel_pages", "block_scores"), got, ref):
            assert torch.equal(a, b), (cut, name)
        G.assert_score_exchange_idle(bufs_s)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_single_launch_against_the_oracle(M, fmt):
    """Scores, selection and outputs of the single launch against the oracle (verify
    rows: three rows per request, causal among the new tokens)."""
    wl = W.small(fmt, [1000, 2600, 130, 640], 3, num_kv_heads=2, k=5, seed=59)
    _print("single launch vs oracle", wl.name)
    G.check_step_parity(M, wl, 2, "single")
