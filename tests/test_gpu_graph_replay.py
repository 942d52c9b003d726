"""Calls captured once in a HIP graph and replayed several times, with eager work and
synchronisations between the replays: every replay equals the eager call bit for bit.
Covers the fused step (whose merge workspace alternates its exchange buffers from call
to call, so the replays use both), the step with the selection in the scoring launch
(its per-row counters must return to zero), the five separate calls, the allocation-
free decode (its fixed scratch shared with an eager call of another size in between)
and the union decode."""
import numpy as np
import pytest
import torch

from sparse_attention_decode_fp8_amd.pipeline import default_num_splits
from synth import workloads as W
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def M():
    import sparse_attention_decode_fp8_amd as M
    return M


def _print(*a):
    print(*a, flush=True)


def _capture(fn):
    """A graph of fn's launches (fn is run eagerly once first, on a side stream)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def _replay_and_check(g, outputs, spoil, reps=4):
    """Replay g `reps` times; before each replay spoil the outputs eagerly (fill
    kernels) and synchronise; after it compare every output bit for bit with `outputs`'
    reference values."""
    ref = [t.clone() for t in outputs]
    for rep in range(reps):
        spoil()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (t, r) in enumerate(zip(outputs, ref)):
            assert torch.equal(t.view(torch.int8) if t.dtype == torch.bfloat16 else t,
                               r.view(torch.int8) if r.dtype == torch.bfloat16 else r), (rep, i)


@pytest.mark.parametrize("cfg,fused,select_in", [(1, True, "decode"), (1, "single", "decode"), (0, "single", "decode"),
                                                 (3, True, "decode"), (1, True, "score"), (0, False, "decode")])
def test_step_graph_replays_equal_the_eager_step(M, cfg, fused, select_in):
    wl = W.config(cfg)
    ns = default_num_splits(wl.k, wl.num_rows * wl.num_kv_heads)
    _print("graph replay", wl.name, "fused", fused, "select in", select_in, "splits", ns)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    kw = dict(slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3]) if app is not None else {}

    def step_fn():
        M.run_step(pool, step, bufs, q, q_idx, w, wl.softmax_scale, n_init=wl.n_init, n_local=wl.n_local,
                   fused=bool(fused), select_in=select_in, single_launch=fused == "single", **kw)

    step_fn()                                  # the eager reference
    torch.cuda.synchronize()
    outs = [bufs.block_scores, bufs.sel, bufs.out] + ([bufs.sel_pages] if fused else [])
    ref = [t.clone() for t in outs]
    g = _capture(step_fn)

    def spoil():
        bufs.out.fill_(7.0)
        bufs.sel.fill_(-3)
        bufs.block_scores.fill_(1.0)

    # the capture's own eager run and the graph's replays must all equal the reference
    for t, r in zip(outs, ref):
        assert torch.equal(t, r)
    _replay_and_check(g, outs, spoil)
    if select_in == "score":
        assert int(bufs.score_counters.abs().sum().item()) == 0
    if fused and ns > 1:
        G.assert_merge_ready(bufs)
    if fused == "single":   # the single launch's score exchange is idle again
        G.assert_score_exchange_idle(bufs)


def test_no_alloc_and_union_graph_replays(M):
    wl = W.small(W.FMT_NVFP4, [3000, 5200, 2600, 4100], 2, num_kv_heads=4, k=8, seed=71)
    _print("graph replay: allocation-free decode and union decode", wl.name)
    pool = G.gpu_pool(M, wl)
    sl, kb, vb, ib = wl.step_tokens()
    M.msa_kv_append(pool, torch.from_numpy(sl).cuda(), G.dev_bf16(kb), G.dev_bf16(vb), G.dev_bf16(ib))
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
    q = G.dev_bf16(wl.q)
    sel = torch.from_numpy(W.verify_tables(wl, 0.6)).cuda()
    out_na = torch.empty(wl.num_rows, wl.num_heads, 128, dtype=torch.bfloat16, device="cuda")
    out_un = torch.empty_like(out_na)
    groups = torch.from_numpy(M.group_rows_of(wl.row_seq, 2)).cuda()
    ns = 4
    po = torch.empty(wl.num_rows, wl.num_heads, ns, 128, device="cuda")
    pm = torch.empty(wl.num_rows, wl.num_heads, ns, 2, device="cuda")
    # a second, smaller call of the allocation-free entry between replays (same scratch)
    small = W.keep_rows(wl, [1, 2, 5])
    step_s = M.Step(small.block_table, small.row_seq, small.row_pos)
    q_s, sel_s = G.dev_bf16(small.q), sel[[1, 2, 5]].contiguous()
    out_s = torch.empty(small.num_rows, small.num_heads, 128, dtype=torch.bfloat16, device="cuda")

    def calls():
        M.msa_sparse_decode_combine_noalloc(pool, step, q, sel, wl.k, wl.softmax_scale, ns, out_na)
        M.msa_sparse_decode_union(pool, step, q, sel, wl.k, groups, 2, wl.softmax_scale, ns, part_o=po,
                                  part_ml=pm)
        M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, po, pm, out_un)

    calls()
    torch.cuda.synchronize()
    outs = [out_na, out_un]
    g = _capture(calls)

    def spoil():
        out_na.fill_(3.0)
        out_un.fill_(3.0)
        M.msa_sparse_decode_combine_noalloc(pool, step_s, q_s, sel_s, wl.k, wl.softmax_scale, 2, out_s)

    _replay_and_check(g, outs, spoil)
    # the allocation-free decode equals the workspace entry
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    M.msa_sparse_decode_combine(pool, step, q, sel, wl.k, wl.softmax_scale, ns, bufs.merge_o, bufs.merge_ml,
                                bufs.counters, bufs.out)
    torch.cuda.synchronize()
    assert torch.equal(bufs.out.view(torch.int16), out_na.view(torch.int16))
