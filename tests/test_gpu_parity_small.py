"""Element-by-element parity of the HIP path with the oracle at small sizes that
still span several pages, ragged last pages, identity rows and several splits."""
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
def test_append_bytes_bit_exact(M, fmt):
    wl = W.small(fmt, [1000, 300, 129], 2, num_kv_heads=2, k=4, seed=41)
    _print("append parity", wl.name, wl.num_pages)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
    M.msa_kv_append(pool, *app)
    # a negative slot is skipped
    M.msa_kv_append(pool, torch.tensor([-1, -5], dtype=torch.int64, device="cuda"),
                    app[1][:2].contiguous(), app[2][:2].contiguous(), app[3][:2].contiguous())
    torch.cuda.synchronize()
    ref = G.oracle_pool(wl)
    for name, arr in pool.arrays().items():
        g = arr.cpu().numpy()
        e = ref[name]
        if name in ("k_scales", "v_scales") and fmt == W.FMT_FP8:
            assert np.array_equal(g, e.astype(np.float32))
        else:
            assert np.array_equal(g.reshape(-1), e.reshape(-1).view(np.uint8)), name


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_splits,fused", [(1, True), (2, False), (2, True), (5, True), (2, "single"),
                                              (5, "single")])
def test_full_step_parity(M, fmt, num_splits, fused):
    wl = W.small(fmt, [1000, 2600, 130, 640], 3, num_kv_heads=2, k=5, seed=31)
    _print("step parity", wl.name, "splits", num_splits, "fused", fused)
    G.check_step_parity(M, wl, num_splits, fused)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_kv_heads,num_splits,fused", [(8, 1, True), (8, 4, True), (8, 2, False), (3, 2, True),
                                                           (8, 4, "single"), (3, 2, "single")])
def test_step_parity_other_kv_head_counts(M, fmt, num_kv_heads, num_splits, fused):
    """8 KV heads (128 query heads) and 3 KV heads: the (row, KV head) grid, the query
    and output strides and the per-KV-head page regions at head counts other than the
    workloads' 1 and 4."""
    wl = W.small(fmt, [1500, 700, 2600], 2, num_kv_heads=num_kv_heads, k=4, seed=33)
    _print("step parity", wl.name, "KV heads", num_kv_heads, "splits", num_splits, "fused", fused)
    G.check_step_parity(M, wl, num_splits, fused)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
@pytest.mark.parametrize("num_splits", [1, 4])
def test_full_step_parity_select_in_scoring_launch(M, fmt, num_splits):
    """The fused step with the selection at the end of the scoring launch (one-wave
    search per row) and the table-driven combining decode."""
    wl = W.small(fmt, [1000, 2600, 130, 640], 3, num_kv_heads=2, k=5, seed=32)
    _print("step parity, select in scoring launch", wl.name, "splits", num_splits)
    G.check_step_parity(M, wl, num_splits, True, select_in="score")


def test_num_splits_agree(M):
    wl = W.small(W.FMT_NVFP4, [3000, 2000], 1, num_kv_heads=1, k=16, seed=43)
    pool = G.gpu_pool(M, wl)
    outs = []
    for ns in (1, 2, 4, 8, 16):
        _print("splits", ns)
        bufs = G.run_gpu_step(M, wl, pool.clone(), ns)
        outs.append(bufs.out.float().cpu().numpy())
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 2 ** -7   # one bf16 ulp at |x| < 2


def _select_case(rng, rows, nb_max, k, quantum):
    S = np.full((rows, nb_max), -np.inf, np.float32)
    pos = rng.integers(0, nb_max * 128, size=rows).astype(np.int32)
    pos[0] = nb_max * 128 - 1
    for r in range(rows):
        nb = pos[r] // 128 + 1
        S[r, :nb] = (np.round(rng.standard_normal(nb) * 8 / quantum) * quantum).astype(np.float32)
    return S, pos


@pytest.mark.parametrize("nb_max,k,n_init,n_local,quantum", [
    (40, 8, 0, 1, 1.0), (257, 16, 0, 1, 0.5), (2048, 32, 0, 1, 4.0), (1025, 16, 2, 2, 2.0),
    (5000, 64, 1, 1, 0.25), (300, 7, 0, 0, 1.0)])
def test_select_bit_exact_on_fp32_scores_with_ties(M, nb_max, k, n_init, n_local, quantum):
    """Same fp32 scores on both sides (heavy exact ties): the tables must agree bit for bit."""
    rng = np.random.default_rng(nb_max + k)
    rows = 12
    S, pos = _select_case(rng, rows, nb_max, k, quantum)
    _print("select", nb_max, k, n_init, n_local)
    step = M.Step(np.zeros((1, nb_max), np.int32), np.zeros(rows, np.int32), pos)
    sel = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    M.msa_select_topk(step, torch.from_numpy(S).cuda(), k, n_init, n_local, sel)
    ref = O.select_topk(S.astype(np.float64), pos, k, n_init, n_local)
    assert np.array_equal(sel.cpu().numpy(), ref)


def test_select_over_1024_way_tie(M):
    nb = 2048
    S = np.full((1, nb), 1.0, np.float32)
    tied = np.sort(np.random.default_rng(5).choice(nb - 1, 1500, replace=False))
    S[0, tied] = 3.5
    step = M.Step(np.zeros((1, nb), np.int32), np.zeros(1, np.int32), np.array([nb * 128 - 1], np.int32))
    sel = torch.empty((1, 32), dtype=torch.int32, device="cuda")
    M.msa_select_topk(step, torch.from_numpy(S).cuda(), 32, 0, 1, sel)
    assert list(sel.cpu().numpy()[0]) == sorted(list(tied[:31]) + [nb - 1])


def test_index_scores_tie_exactly_for_identical_keys(M):
    wl = W.small(W.FMT_FP8, [128 * 40], 0, num_kv_heads=1, k=8, seed=44)
    W.inject_ties(wl, 20)
    pool = G.gpu_pool(M, wl)
    step, q, q_idx, w, _ = G.gpu_step_inputs(M, wl)
    S = torch.empty((1, wl.max_blocks), dtype=torch.float32, device="cuda")
    M.msa_index_score(pool, step, q_idx, w, S)
    S = S.cpu().numpy()[0]
    tied = wl.tie_blocks[0]
    assert len(set(S[tied].tolist())) == 1
    others = np.setdiff1d(np.arange(wl.max_blocks), tied)
    assert S[tied[0]] > S[others].max()


def test_decode_on_oracle_selection_matches_attention(M):
    """msa_sparse_decode + msa_combine given the oracle's selection table."""
    for fmt in (W.FMT_FP8, W.FMT_NVFP4):
        wl = W.small(fmt, [700, 5000, 64], 1, num_kv_heads=3, k=6, seed=45)
        _print("decode given selection", wl.name)
        pool = G.gpu_pool(M, wl)
        step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
        M.msa_kv_append(pool, *app)
        ref_pool = G.oracle_pool(wl)
        S_ref = O.index_score(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q_idx, wl.w,
                              wl.max_blocks)
        sel_ref = O.select_topk(S_ref, wl.row_pos, wl.k)
        out_ref = O.attend(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel_ref,
                           wl.softmax_scale)
        sel = torch.from_numpy(sel_ref).cuda()
        for ns in (1, 3, 6):
            po = torch.empty((wl.num_rows, wl.num_heads, ns, 128), dtype=torch.float32, device="cuda")
            pm = torch.empty((wl.num_rows, wl.num_heads, ns, 2), dtype=torch.float32, device="cuda")
            out = torch.empty((wl.num_rows, wl.num_heads, 128), dtype=torch.bfloat16, device="cuda")
            M.msa_sparse_decode(pool, step, q, sel, wl.k, wl.softmax_scale, ns, po, pm)
            M.msa_combine(wl.num_rows, wl.num_heads, 128, ns, po, pm, out)
            G.assert_out_close(G.bf16_to_np(out), out_ref, f"{wl.name} splits {ns}")


def test_combine_matches_oracle_combine(M):
    rng = np.random.default_rng(8)
    rows, H, S = 3, 32, 5
    m = rng.standard_normal((rows, H, S)) * 4
    m[0, 0, 2] = -np.inf
    l = rng.random((rows, H, S)) * 10 + 0.5
    l[0, 0, 2] = 0.0
    Op = rng.standard_normal((rows, H, S, 128)) * l[..., None]
    Op[0, 0, 2] = 0.0
    ml = np.stack([m, l], -1).astype(np.float32)
    out = torch.empty((rows, H, 128), dtype=torch.bfloat16, device="cuda")
    M.msa_combine(rows, H, 128, S, torch.from_numpy(Op.astype(np.float32)).cuda(),
                  torch.from_numpy(ml).cuda(), out)
    ref = O.combine(ml[..., 0].astype(np.float64), ml[..., 1].astype(np.float64),
                    Op.astype(np.float32).astype(np.float64))
    got = G.bf16_to_np(out)
    # one bf16 rounding of the exact merge
    assert np.all(np.abs(got - ref) <= np.abs(ref) * 2 ** -8 + 1e-6)


def test_sel_pages_and_fused_combine(M):
    """sel_pages is the block-table image of sel; the two fused launches (append + score +
    select, decode + combine) equal the five separate calls bit for bit and leave their
    counters at zero."""
    wl = W.small(W.FMT_NVFP4, [3000, 700, 5000], 2, num_kv_heads=2, k=8, seed=46)
    pool = G.gpu_pool(M, wl)
    for ns in (1, 3, 4, 8):
        _print("fused vs separate, splits", ns)
        pa = pool.clone()
        a = G.run_gpu_step(M, wl, pa, ns, fused=True)
        b = G.run_gpu_step(M, wl, pool.clone(), ns, fused=False)
        sel, sp = a.sel.cpu().numpy(), a.sel_pages.cpu().numpy()
        exp = np.where(sel >= 0, wl.block_table[wl.row_seq[:, None], np.maximum(sel, 0)], -1)
        assert np.array_equal(sp, exp)
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))
        assert torch.equal(a.sel, b.sel)
        nb = torch.from_numpy(wl.row_pos // 128 + 1).cuda()
        vis = torch.arange(wl.max_blocks, device="cuda")[None] < nb[:, None]
        assert torch.equal(a.block_scores[vis], b.block_scores[vis])
        G.assert_merge_ready(a)
        assert int(a.score_counters.abs().sum()) == 0
        # the scoring launch can also select (last workgroup per row group)
        pc = pool.clone()
        step, q, q_idx, w, app = G.gpu_step_inputs(M, wl)
        bs = torch.empty_like(a.block_scores)
        sel2 = torch.full_like(a.sel, -7)
        sp2 = torch.full_like(a.sel, -7)
        M.msa_append_score_select(pc, step, q_idx, w, wl.k, 0, 1, bs, sel2, sp2, a.score_counters,
                                  slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
        torch.cuda.synchronize()
        assert torch.equal(sel2, b.sel) and torch.equal(sp2, b.sel_pages)
        assert int(a.score_counters.abs().sum()) == 0
        for name, arr in pa.arrays().items():
            assert torch.equal(arr, pc.arrays()[name]), name
        # a second call with the same counters still merges correctly
        step, q, q_idx, w, _ = G.gpu_step_inputs(M, wl)
        M.msa_sparse_decode_combine(pa, step, q, a.sel, wl.k, wl.softmax_scale, ns, a.merge_o,
                                    a.merge_ml, a.counters, a.out, sel_pages=a.sel_pages)
        torch.cuda.synchronize()
        assert torch.equal(a.out.view(torch.int16), b.out.view(torch.int16))


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_fused_step_many_rows_per_request(M, fmt):
    """Verify-style step (4 rows per request, appended tokens spanning a page boundary):
    fused and separate launches agree bit for bit, repeatedly."""
    wl = W.small(fmt, [126, 1022, 3000, 9000], 4, num_kv_heads=2, k=6, seed=47)
    pool = G.gpu_pool(M, wl)
    ref = G.run_gpu_step(M, wl, pool.clone(), 3, fused=False)
    for rep in range(3):
        got = G.run_gpu_step(M, wl, pool.clone(), 3, fused=True)
        assert torch.equal(got.sel, ref.sel)
        assert torch.equal(got.out.view(torch.int16), ref.out.view(torch.int16)), rep


@pytest.mark.parametrize("nb_max,k,n_init,n_local,quantum,tie_max,ns", [
    (40, 8, 0, 1, 1.0, 0, 2), (257, 16, 0, 1, 0.5, 5, 2), (257, 16, 0, 1, 0.5, 40, 2), (600, 16, 1, 1, 2.0, 0, 2),
    (1025, 16, 2, 2, 2.0, 9, 2), (2048, 32, 0, 1, 4.0, 0, 2), (2048, 32, 0, 1, 0.25, 1200, 2),
    (300, 7, 0, 0, 1.0, 3, 2), (3000, 64, 0, 1, 1.0, 100, 4), (5000, 16, 0, 1, 1.0, 0, 2),
    (1500, 8, 0, 1, 1.0, 20, 8), (257, 4, 0, 1, 0.5, 10, 1), (700, 16, 0, 1, 1.0, 0, 1)])
def test_fused_select_bit_exact_with_ties(M, nb_max, k, n_init, n_local, quantum, tie_max, ns):
    """The selection inside the fused decode on the same fp32 scores as the oracle, with
    heavy exact ties and `tie_max` extra blocks tied at each row's maximum: tables
    identical. The cases span every shape of the two-level selection (1, 2, 4 and 8 keys
    per lane, one to eight first-level waves, in workgroups of 4, 8 and 16 waves) and the
    block radix select that takes rows too long for it (5000 blocks)."""
    rng = np.random.default_rng(7 * nb_max + k + tie_max)
    rows = 6
    S, pos = _select_case(rng, rows, nb_max, k, quantum)
    for r in range(rows):
        nb = pos[r] // 128 + 1
        if tie_max and nb > 2:
            top = S[r, :nb].max()
            S[r, rng.choice(nb - 1, min(tie_max, nb - 1), replace=False)] = top
    _print("fused select", nb_max, k, n_init, n_local, tie_max, "splits", ns)
    wl = W.small(W.FMT_NVFP4, [300], 1, num_kv_heads=1, k=k, seed=91)
    pool = G.gpu_pool(M, wl)
    bt = rng.integers(0, wl.num_pages, size=(1, nb_max)).astype(np.int32)
    step = M.Step(bt, np.zeros(rows, np.int32), pos)
    q = torch.from_numpy(rng.standard_normal((rows, wl.num_heads, 128)).astype(np.float32)).to(torch.bfloat16).cuda()
    bufs = M.DecodeBuffers(rows, wl.num_heads, nb_max, k, ns)
    M.msa_select_decode_combine(pool, step, q, torch.from_numpy(S).cuda(), k, n_init, n_local,
                                wl.softmax_scale, ns, bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                                sel=bufs.sel, sel_pages=bufs.sel_pages)
    torch.cuda.synchronize()
    ref = O.select_topk(S.astype(np.float64), pos, k, n_init, n_local)
    sel = bufs.sel.cpu().numpy()
    assert np.array_equal(sel, ref)
    assert np.array_equal(bufs.sel_pages.cpu().numpy(), np.where(ref >= 0, bt[0][np.maximum(ref, 0)], -1))
    G.assert_merge_ready(bufs)
