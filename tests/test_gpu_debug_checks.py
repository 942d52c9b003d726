"""The debug build (libmsadecode_debug.so, MSA_DEBUG_CHECKS): on valid inputs it reports
nothing and computes exactly what the release build does; each kind of bad device-side
metadata is reported in the caller's error word by the kernels' own checks, which skip
or redirect the access they guard (so these cases stay in bounds by construction)."""
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


@pytest.fixture(scope="module")
def dbg(M):
    lib = M.load_library(M.DEBUG_LIB_PATH)
    assert lib.msa_debug_checks_enabled() == 1
    return lib


def _print(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("fused", [True, False, "single"])
def test_valid_step_reports_nothing_and_matches_release(M, dbg, fmt, fused):
    wl = W.small(fmt, [1000, 2600, 130], 2, num_kv_heads=2, k=5, seed=95)
    _print("debug build, valid step", wl.name, "fused", fused)
    pool = G.gpu_pool(M, wl)
    ref = G.run_gpu_step(M, wl, pool.clone(), 2, fused=fused)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with M.use_library(dbg):
        M.msa_debug_set_error_word(err)
        try:
            got = G.run_gpu_step(M, wl, pool.clone(), 2, fused=fused)
        finally:
            M.msa_debug_set_error_word(None)
    assert int(err.item()) == 0
    assert torch.equal(got.block_scores, ref.block_scores)
    assert torch.equal(got.sel, ref.sel)
    assert torch.equal(got.out.view(torch.int16), ref.out.view(torch.int16))


def _bad_case_setup(M, fmt):
    wl = W.small(fmt, [1000, 2600], 1, num_kv_heads=2, k=4, seed=96)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 2)
    M.msa_index_score(pool, step, q_idx, w, bufs.block_scores)
    M.msa_select_topk(step, bufs.block_scores, wl.k, 0, 1, bufs.sel, bufs.sel_pages)
    torch.cuda.synchronize()
    return wl, pool, step, q, q_idx, w, app, bufs


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_bad_metadata_is_reported(M, dbg, fmt):
    wl, pool, step, q, q_idx, w, app, bufs = _bad_case_setup(M, fmt)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with M.use_library(dbg):
        M.msa_debug_set_error_word(err)
        try:
            def expect(code, what):
                torch.cuda.synchronize()
                assert int(err.item()) == code, (what, int(err.item()))
                err.zero_()

            # a page id past the pool in sel_pages: the decode reads page 0 instead
            _print("debug: page id past the pool (sel_pages)")
            sp = bufs.sel_pages.clone()
            sp[0, 0] = wl.num_pages + 7
            M.msa_sparse_decode(pool, step, q, bufs.sel, wl.k, wl.softmax_scale, 2, bufs.part_o, bufs.part_ml,
                                sel_pages=sp)
            expect(1, "page")
            # a selection entry past the row's visible blocks: dropped
            _print("debug: selection entry past the row")
            sl = bufs.sel.clone()
            sl[1, 0] = wl.max_blocks + 3
            M.msa_sparse_decode(pool, step, q, sl, wl.k, wl.softmax_scale, 2, bufs.part_o, bufs.part_ml)
            expect(4, "sel")
            # a request id past num_seqs: the selection reads request 0's table
            _print("debug: request id past num_seqs")
            bad_seq = M.Step(wl.block_table, np.where(np.arange(wl.num_rows) == 0, len(wl.ctx_lens) + 3,
                                                      wl.row_seq).astype(np.int32), wl.row_pos)
            M.msa_select_topk(bad_seq, bufs.block_scores, wl.k, 0, 1, bufs.sel, bufs.sel_pages)
            expect(2, "seq")
            # a position past the block table: the selection clamps to the table
            _print("debug: position past the table")
            bad_pos = M.Step(wl.block_table, wl.row_seq,
                             np.where(np.arange(wl.num_rows) == 1, wl.max_blocks * 128 + 5, wl.row_pos).astype(np.int32))
            M.msa_select_topk(bad_pos, bufs.block_scores, wl.k, 0, 1, bufs.sel, bufs.sel_pages)
            expect(3, "pos")
            # a block-table page past the pool: the scorer reads page 0's keys instead
            _print("debug: block-table page past the pool")
            bt = wl.block_table.copy()
            bt[1, 2] = wl.num_pages + 11
            M.msa_index_score(pool, M.Step(bt, wl.row_seq, wl.row_pos), q_idx, w, bufs.block_scores)
            expect(1, "table page")
            # an append slot whose page lies past the pool: the token is not written
            _print("debug: append slot past the pool")
            slot = app[0].clone()
            slot[0] = (wl.num_pages + 2) * 128 + 5
            before = {k: v.clone() for k, v in pool.arrays().items()}
            M.msa_kv_append(pool, slot[:1], app[1][:1].contiguous(), app[2][:1].contiguous(),
                            app[3][:1].contiguous())
            expect(5, "slot")
            for k, v in pool.arrays().items():
                assert torch.equal(v, before[k]), k
        finally:
            M.msa_debug_set_error_word(None)


def test_bad_union_groups_are_reported_and_stay_in_bounds(M, dbg):
    """msa_sparse_decode_union with malformed row groups (longer than max_group_rows,
    mixing two requests, past num_rows): the debug library reports
    MSA_DEBUG_BAD_GROUP and the kernel clamps the group to its first rows inside the
    call, so every access stays in bounds; a valid grouping reports nothing."""
    wl = W.small(W.FMT_NVFP4, [1500, 2200], 4, num_kv_heads=2, k=5, seed=98)
    pool = G.gpu_pool(M, wl)
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
    q = G.dev_bf16(wl.q)
    sel = torch.from_numpy(W.verify_tables(wl, 0.5)).cuda()
    out = torch.zeros(wl.num_rows, wl.num_heads, 128, dtype=torch.bfloat16, device="cuda")
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with M.use_library(dbg):
        M.msa_debug_set_error_word(err)
        try:
            for groups, want in (([0, 4, 8], 0), ([0, 8], 7), ([2, 6], 7), ([4, 12], 7), ([0, 3, 4, 8], 0)):
                _print("debug: union groups", groups)
                gr = torch.tensor(groups, dtype=torch.int32, device="cuda")
                M.msa_sparse_decode_union(pool, step, q, sel, wl.k, gr, 4, wl.softmax_scale, 1, out=out)
                torch.cuda.synchronize()
                assert int(err.item()) == want, (groups, int(err.item()))
                err.zero_()
        finally:
            M.msa_debug_set_error_word(None)


@pytest.mark.parametrize("entry", ["select_decode_combine", "sparse_decode_combine"])
def test_merge_give_up_is_reported_and_sticky(M, dbg, entry):
    """A merging split that gives up waiting (forced from the host: a poll limit of 0,
    so the merger never reads and every kernel still exits normally) writes NaN, sets
    the pair's failure bit, and the debug library reports MSA_DEBUG_MERGE_TIMEOUT. Later
    calls keep writing NaN and touch no workspace word until the workspace is set up
    again; then the merge equals msa_sparse_decode + msa_combine bit for bit."""
    wl = W.small(W.FMT_NVFP4, [3000, 2000], 1, num_kv_heads=2, k=8, seed=97)
    ns = 4
    _print("forced merge give-up", entry, wl.name, "splits", ns)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
    M.msa_kv_append(pool, *app)
    M.msa_index_score(pool, step, q_idx, w, bufs.block_scores)
    M.msa_select_topk(step, bufs.block_scores, wl.k, 0, 1, bufs.sel, bufs.sel_pages)
    M.msa_sparse_decode(pool, step, q, bufs.sel, wl.k, wl.softmax_scale, ns, bufs.part_o, bufs.part_ml,
                        sel_pages=bufs.sel_pages)
    ref = torch.empty_like(bufs.out)
    M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, bufs.part_o, bufs.part_ml, ref)

    def call():
        if entry == "select_decode_combine":
            M.msa_select_decode_combine(pool, step, q, bufs.block_scores, wl.k, 0, 1, wl.softmax_scale, ns,
                                        bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out)
        else:
            M.msa_sparse_decode_combine(pool, step, q, bufs.sel, wl.k, wl.softmax_scale, ns, bufs.merge_o,
                                        bufs.merge_ml, bufs.counters, bufs.out, sel_pages=bufs.sel_pages)
        torch.cuda.synchronize()

    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    with M.use_library(dbg):
        M.msa_debug_set_error_word(err)
        try:
            M.msa_debug_set_merge_poll_limit(0)
            call()
            assert int(err.item()) == 6                      # MSA_DEBUG_MERGE_TIMEOUT
            assert torch.isnan(bufs.out.float()).all()
            c = bufs.counters.cpu().numpy().view(np.uint32)
            assert ((c & (1 << 25)) != 0).all() and (((c >> 26) & 0x1f) == ns).all()
            M.msa_debug_set_merge_poll_limit(-1)             # the release bound again
            err.zero_()
            words = [t.clone() for t in (bufs.counters, bufs.merge_o, bufs.merge_ml)]
            bufs.out.zero_()
            call()                                           # still failed: NaN, nothing touched
            assert torch.isnan(bufs.out.float()).all() and int(err.item()) == 0
            for a, b in zip(words, (bufs.counters, bufs.merge_o, bufs.merge_ml)):
                assert torch.equal(a.view(torch.int32), b.view(torch.int32))
        finally:
            M.msa_debug_set_merge_poll_limit(-1)
            M.msa_debug_set_error_word(None)
    M.msa_merge_workspace_init(wl.num_rows, wl.num_heads, 128, ns, bufs.merge_o, bufs.merge_ml, bufs.counters)
    call()
    assert torch.equal(bufs.out.view(torch.int16), ref.view(torch.int16))
    G.assert_merge_ready(bufs)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_forced_merge_handoffs_give_the_same_outputs(M, dbg, fmt):
    """The split merge of a (row, KV head) is shared by its last splits to arrive, each
    merging a slice of the heads; one that is not the last hands its slice to the last
    split when its bounded wait runs out. With the debug library's bound set to 0 every
    such split hands over at once unless the last split has already arrived: the
    outputs stay those of msa_sparse_decode + msa_combine bit for bit, nothing is
    reported and the workspace is left ready, for split counts with 2 and 4 slices."""
    wl = W.small(fmt, [3000, 2000, 5100, 700], 2, num_kv_heads=2, k=16, seed=99)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    M.msa_kv_append(pool, *app)
    scores = torch.empty((wl.num_rows, wl.max_blocks), dtype=torch.float32, device="cuda")
    M.msa_index_score(pool, step, q_idx, w, scores)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    for ns in (2, 3, 4, 5, 8, 16):
        _print("forced merge handoffs", wl.name, "splits", ns)
        ref = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
        M.msa_select_topk(step, scores, wl.k, wl.n_init, wl.n_local, ref.sel, ref.sel_pages)
        M.msa_sparse_decode(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns, ref.part_o, ref.part_ml,
                            sel_pages=ref.sel_pages)
        M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, ref.part_o, ref.part_ml, ref.out)
        bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, ns)
        with M.use_library(dbg):
            M.msa_debug_set_error_word(err)
            try:
                M.msa_debug_set_merge_helper_poll_limit(0)
                for call in range(4):   # both exchange buffers, both fused entries
                    bufs.out.fill_(0)
                    if call % 2 == 0:
                        M.msa_select_decode_combine(pool, step, q, scores, wl.k, wl.n_init, wl.n_local,
                                                    wl.softmax_scale, ns, bufs.merge_o, bufs.merge_ml,
                                                    bufs.counters, bufs.out)
                    else:
                        M.msa_sparse_decode_combine(pool, step, q, ref.sel, wl.k, wl.softmax_scale, ns,
                                                    bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                                                    sel_pages=ref.sel_pages)
                    torch.cuda.synchronize()
                    assert int(err.item()) == 0, (ns, call)
                    assert torch.equal(bufs.out.view(torch.int16), ref.out.view(torch.int16)), (ns, call)
                    G.assert_merge_ready(bufs)
            finally:
                M.msa_debug_set_merge_helper_poll_limit(-1)
                M.msa_debug_set_error_word(None)
