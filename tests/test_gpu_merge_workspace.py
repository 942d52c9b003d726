"""The fused entries' split-merge workspace: msa_merge_workspace_init sets it up for one
split count; successive fused calls (alternating exchange buffers) equal the separate
decode + combine calls bit for bit and leave it ready for the next call; a call with
another split count touches no workspace word and writes NaN; a fresh set-up serves
the new split count."""
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


def test_workspace_init_sets_up_state(M):
    rows, hq, S = 3, 32, 5
    po = torch.full((rows, hq // 16, 2, 16, S, 128), 1.5, dtype=torch.float32, device="cuda")
    pm = torch.full((rows, hq // 16, 2, 16, S, 2), -2.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((rows, hq // 16), 9, dtype=torch.int32, device="cuda")
    guard = torch.full((64,), 3.0, dtype=torch.float32, device="cuda")
    M.msa_merge_workspace_init(rows, hq, 128, S, po, pm, cnt)
    torch.cuda.synchronize()
    assert bool((po.view(torch.int32) == M.MERGE_IDLE_BITS).all())
    assert bool((pm.view(torch.int32) == M.MERGE_IDLE_BITS).all())
    assert bool((cnt == (S << 26)).all())
    assert bool((guard == 3.0).all())


def _reference(M, wl, pool, step, q, scores, ns):
    ref = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    M.msa_select_topk(step, scores, wl.k, wl.n_init, wl.n_local, ref.sel, ref.sel_pages)
    M.msa_sparse_decode(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns, ref.part_o, ref.part_ml,
                        sel_pages=ref.sel_pages)
    M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, ref.part_o, ref.part_ml, ref.out)
    return ref


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_successive_calls_and_split_changes(M, fmt):
    wl = W.small(fmt, [3000, 700, 5000, 9000], 2, num_kv_heads=2, k=16, seed=81)
    print("merge workspace", wl.name, flush=True)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    kw = dict(slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
    scores = torch.empty((wl.num_rows, wl.max_blocks), dtype=torch.float32, device="cuda")
    M.msa_append_score_select(pool, step, q_idx, w, wl.k, wl.n_init, wl.n_local, scores, **kw)
    # one workspace sized for 16 splits, set up in turn for each split count used
    ws = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 16)
    for ns in (8, 2, 16, 3):
        print("  splits", ns, flush=True)
        ref = _reference(M, wl, pool, step, q, scores, ns)
        M.msa_merge_workspace_init(wl.num_rows, wl.num_heads, 128, ns, ws.merge_o, ws.merge_ml, ws.counters)
        ws.num_splits = ns
        for call in range(5):   # both buffers, twice over, alternating the two entries
            ws.out.fill_(0)
            if call % 2 == 0:
                M.msa_select_decode_combine(pool, step, q, scores, wl.k, wl.n_init, wl.n_local,
                                            wl.softmax_scale, ns, ws.merge_o, ws.merge_ml, ws.counters,
                                            ws.out, sel=ws.sel, sel_pages=ws.sel_pages)
            else:
                M.msa_sparse_decode_combine(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns, ws.merge_o,
                                            ws.merge_ml, ws.counters, ws.out, sel_pages=ref.sel_pages)
            torch.cuda.synchronize()
            assert torch.equal(ws.out.view(torch.int16), ref.out.view(torch.int16)), (ns, call)
            G.assert_merge_ready(ws)
            if call % 2 == 0:
                assert torch.equal(ws.sel, ref.sel)
        epoch = (ws.counters.cpu().numpy().view(np.uint32) >> 31)
        assert (epoch == 1).all()   # five calls: buffer 0, 1, 0, 1, 0 -> next is 1
        # a call with another split count (within the allocation): workspace untouched,
        # NaN outputs
        other = 4 if ns != 4 else 2
        before = [t.clone() for t in (ws.merge_o, ws.merge_ml, ws.counters)]
        M.msa_select_decode_combine(pool, step, q, scores, wl.k, wl.n_init, wl.n_local, wl.softmax_scale,
                                    other, ws.merge_o, ws.merge_ml, ws.counters, ws.out)
        torch.cuda.synchronize()
        for t0, t in zip(before, (ws.merge_o, ws.merge_ml, ws.counters)):
            assert torch.equal(t0.view(torch.int32), t.view(torch.int32))
        assert bool(torch.isnan(ws.out.float()).all())
        # after a fresh set-up the new split count works
        M.msa_merge_workspace_init(wl.num_rows, wl.num_heads, 128, other, ws.merge_o, ws.merge_ml, ws.counters)
        ref2 = _reference(M, wl, pool, step, q, scores, other)
        M.msa_select_decode_combine(pool, step, q, scores, wl.k, wl.n_init, wl.n_local, wl.softmax_scale,
                                    other, ws.merge_o, ws.merge_ml, ws.counters, ws.out)
        torch.cuda.synchronize()
        assert torch.equal(ws.out.view(torch.int16), ref2.out.view(torch.int16)), ns


def test_calls_with_fewer_rows_share_the_workspace(M):
    """The workspace is pair-major: calls with fewer rows (a different batch) use the
    first rows' slots and state words and leave the others as they were."""
    full = W.small(W.FMT_NVFP4, [3000, 700, 5000, 9000], 2, num_kv_heads=2, k=16, seed=82)
    part = W.keep_rows(full, [0, 1, 4, 5])
    pool = G.gpu_pool(M, full)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, full)
    M.msa_kv_append(pool, app[0], app[1], app[2], app[3])
    ns = 4
    ws = M.DecodeBuffers(full.num_rows, full.num_heads, full.max_blocks, full.k, ns)
    for call, wl in enumerate([full, part, full, part, part, full]):
        st, qq, qi, ww, _ = G.gpu_step_inputs(M, wl)
        scores = torch.empty((wl.num_rows, wl.max_blocks), dtype=torch.float32, device="cuda")
        M.msa_index_score(pool, st, qi, ww, scores)
        ref = _reference(M, wl, pool, st, qq, scores, ns)
        out = torch.zeros_like(ref.out)
        M.msa_select_decode_combine(pool, st, qq, scores, wl.k, wl.n_init, wl.n_local, wl.softmax_scale, ns,
                                    ws.merge_o, ws.merge_ml, ws.counters, out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.out.view(torch.int16)), call
        G.assert_merge_ready(ws)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("k,ctx", [(16, [3000, 9000]), (16, [2500 + 37 * i for i in range(70)]), (5, [3000, 9000])])
def test_one_split_direct_output_equals_partials_and_combine(M, fmt, k, ctx):
    """With one split the combining entries write the output themselves (no workspace);
    it equals msa_sparse_decode + msa_combine bit for bit, in both wave layouts the
    decode picks by launch size (4 or 280 workgroups, against 256 compute units)."""
    wl = W.small(fmt, ctx, 2, num_kv_heads=2, k=k, seed=85)
    print("one split", wl.name, "k", k, "rows", wl.num_rows, flush=True)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    scores = torch.empty((wl.num_rows, wl.max_blocks), dtype=torch.float32, device="cuda")
    M.msa_append_score_select(pool, step, q_idx, w, wl.k, wl.n_init, wl.n_local, scores, slot=app[0],
                              k_new=app[1], v_new=app[2], idx_k_new=app[3])
    ref = _reference(M, wl, pool, step, q, scores, 1)
    ws = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 1)
    M.msa_select_decode_combine(pool, step, q, scores, wl.k, wl.n_init, wl.n_local, wl.softmax_scale, 1,
                                ws.merge_o, ws.merge_ml, ws.counters, ws.out, sel=ws.sel, sel_pages=ws.sel_pages)
    torch.cuda.synchronize()
    assert torch.equal(ws.sel, ref.sel) and torch.equal(ws.sel_pages, ref.sel_pages)
    assert torch.equal(ws.out.view(torch.int16), ref.out.view(torch.int16))
    ws.out.fill_(0)
    M.msa_sparse_decode_combine(pool, step, q, ref.sel, wl.k, wl.softmax_scale, 1, ws.merge_o, ws.merge_ml,
                                ws.counters, ws.out, sel_pages=ref.sel_pages)
    torch.cuda.synchronize()
    assert torch.equal(ws.out.view(torch.int16), ref.out.view(torch.int16))
