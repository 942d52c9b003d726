"""msa_sparse_decode_union (query pairing: the rows of a request decoded together over
the union of their selected pages) against the oracle: each row's output against its
own attention (oracle.attend), and the split partials against oracle.union_partials,
on verify-style tables with chosen overlap between the rows of a request, rows that
cross a page boundary, ragged groups, per-KV-head tables, sel_pages, and config 2's
40 x 4 verify rows (sampled requests) on the GPU's own selection."""
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


def _full_gpu_pool(M, wl):
    """Every cached token and the step's appended tokens (the verify rows' own)."""
    pool = G.gpu_pool(M, wl)
    sl, kb, vb, ib = wl.step_tokens()
    if len(sl):
        M.msa_kv_append(pool, torch.from_numpy(sl).cuda(), G.dev_bf16(kb), G.dev_bf16(vb), G.dev_bf16(ib))
    return pool


def _union(M, wl, pool, sel, groups, max_rows, ns, tables=1, sel_pages=None):
    """One union decode; num_splits > 1 also runs msa_combine. Returns the bf16 output
    as float64 and, for ns > 1, the partials (part_ml, part_o) as written."""
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos, sel_tables=tables)
    q = G.dev_bf16(wl.q)
    sel_d = torch.from_numpy(np.ascontiguousarray(sel, dtype=np.int32)).cuda()
    sp = None if sel_pages is None else torch.from_numpy(np.ascontiguousarray(sel_pages, dtype=np.int32)).cuda()
    gr = torch.from_numpy(np.asarray(groups, dtype=np.int32)).cuda()
    rows, hq = wl.num_rows, wl.num_heads
    out = torch.zeros(rows, hq, 128, dtype=torch.bfloat16, device="cuda")
    if ns == 1:
        M.msa_sparse_decode_union(pool, step, q, sel_d, wl.k, gr, max_rows, wl.softmax_scale, 1, out=out,
                                  sel_pages=sp)
        torch.cuda.synchronize()
        return G.bf16_to_np(out), None
    po = torch.full((rows, hq, ns, 128), float("nan"), device="cuda")
    pm = torch.full((rows, hq, ns, 2), float("nan"), device="cuda")
    M.msa_sparse_decode_union(pool, step, q, sel_d, wl.k, gr, max_rows, wl.softmax_scale, ns, part_o=po,
                              part_ml=pm, sel_pages=sp)
    M.msa_combine(rows, hq, 128, ns, po, pm, out)
    torch.cuda.synchronize()
    return G.bf16_to_np(out), (pm.cpu().numpy(), po.cpu().numpy())


def _check_partials(parts, ref, rows):
    """Partials to the bars of the one-row decode's partials (base-2 m, l; O relative to
    its weight sum); the empty ones exactly (-inf, 0, 0)."""
    ml, po = parts
    m, l, Op = ref
    for r in rows:
        fin = np.isfinite(m[r])
        assert np.array_equal(np.isneginf(ml[r, :, :, 0]), ~fin), f"row {r}: empty-split pattern"
        assert np.allclose(ml[r, :, :, 0][fin], m[r][fin], rtol=1e-4, atol=1e-3)
        lr = np.where(fin, l[r], 0)
        assert np.allclose(ml[r, :, :, 1], lr, rtol=2e-2, atol=1e-3)
        assert (po[r][~fin] == 0).all()
        den = np.maximum(lr, 1e-30)[..., None]
        assert np.max(np.abs(po[r] / den - Op[r] / den)[fin]) < 1e-2


def _oracle_pool_all(wl):
    return G.oracle_pool(wl)


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_FP8])
@pytest.mark.parametrize("overlap", [0.0, 0.6, 1.0])
@pytest.mark.parametrize("size,ns", [(4, 1), (4, 3), (2, 2), (3, 1), (1, 2)])
def test_union_matches_oracle_small_verify(M, fmt, overlap, size, ns):
    # 4 verify rows per request; requests at 1022 and 126 cross a page boundary
    wl = W.small(fmt, [1022, 1500, 126, 2600], 4, num_kv_heads=2, k=5, seed=41)
    _print("union small verify", wl.name, "overlap", overlap, "group size", size, "splits", ns)
    pool = _full_gpu_pool(M, wl)
    sel = W.verify_tables(wl, overlap)
    groups = M.group_rows_of(wl.row_seq, size)
    out, parts = _union(M, wl, pool, sel, groups, size, ns)
    opool = _oracle_pool_all(wl)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    G.assert_out_close(out, ref, "union outputs")
    if parts is not None:
        up = O.union_partials(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale, ns,
                              groups)
        _check_partials(parts, up, range(wl.num_rows))


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_FP8])
def test_union_many_chunks_ragged_groups_and_sel_pages(M, fmt):
    # k = 24 over 4 rows: up to 96 union entries (many rounds of 8 chunks); requests
    # with 1, 2, 3 and 4 rows (a request's rows stay together); sel_pages given
    full = W.small(fmt, [5000, 3100, 4000, 7000], 4, num_kv_heads=1, k=24, seed=42)
    keep = [0, 4, 5, 8, 9, 10, 12, 13, 14, 15]
    wl = W.keep_rows(full, keep)
    _print("union ragged groups", wl.name, "rows", wl.num_rows)
    pool = _full_gpu_pool(M, full)
    sel = W.verify_tables(wl, 0.5)
    pages = np.where(sel >= 0, full.block_table[wl.row_seq[:, None], np.maximum(sel, 0)], -1)
    opool = _oracle_pool_all(full)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    for size, ns in ((4, 1), (4, 7), (2, 4)):
        groups = M.group_rows_of(wl.row_seq, size)
        out, parts = _union(M, wl, pool, sel, groups, size, ns, sel_pages=pages)
        G.assert_out_close(out, ref, f"ragged groups of {size}, {ns} splits")
        if parts is not None:
            up = O.union_partials(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale,
                                  ns, groups)
            _check_partials(parts, up, range(wl.num_rows))


def test_union_per_kv_head_tables(M):
    wl = W.small(W.FMT_NVFP4, [1500, 2200], 4, num_kv_heads=2, k=6, seed=43)
    _print("union per-KV-head tables", wl.name)
    pool = _full_gpu_pool(M, wl)
    sel = np.stack([W.verify_tables(wl, 0.7, seed_tag=5), W.verify_tables(wl, 0.3, seed_tag=6)], axis=1)
    groups = M.group_rows_of(wl.row_seq, 4)
    opool = _oracle_pool_all(wl)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    for ns in (1, 3):
        out, parts = _union(M, wl, pool, sel, groups, 4, ns, tables=2)
        G.assert_out_close(out, ref, f"per-KV-head tables, {ns} splits")
        if parts is not None:
            up = O.union_partials(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale,
                                  ns, groups)
            _check_partials(parts, up, range(wl.num_rows))


def test_union_groups_of_one_row_equal_sparse_decode_partials(M):
    # one-row groups with full tables split their tables as msa_sparse_decode does; the
    # chunk-to-wave assignment and the arithmetic are the same, so the partials agree
    # bit for bit
    wl = W.small(W.FMT_NVFP4, [1500, 2200, 3000], 1, num_kv_heads=2, k=6, seed=44)
    pool = _full_gpu_pool(M, wl)
    sel = W.verify_tables(wl, 0.0)
    assert (sel >= 0).all()
    groups = np.arange(wl.num_rows + 1, dtype=np.int32)
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
    q = G.dev_bf16(wl.q)
    sel_d = torch.from_numpy(sel).cuda()
    rows, hq, ns = wl.num_rows, wl.num_heads, 3
    po = torch.zeros(rows, hq, ns, 128, device="cuda")
    pm = torch.zeros(rows, hq, ns, 2, device="cuda")
    M.msa_sparse_decode(pool, step, q, sel_d, wl.k, wl.softmax_scale, ns, po, pm)
    _, parts = _union(M, wl, pool, sel, groups, 1, ns)
    assert np.array_equal(parts[0], pm.cpu().numpy())
    assert np.array_equal(parts[1], po.cpu().numpy())


@pytest.mark.parametrize("shared", [False, True])
def test_union_config2_sampled_requests(M, shared):
    """Config 2 (40 requests x 4 verify rows, NVFP4, k 16) on the GPU's own selection
    (shared: every row of a request takes its first row's table, the full-overlap
    case); 8 seeded requests and the longest one against the oracle, and every row
    against the one-row decode of the same table."""
    wl = W.config(2)
    _print("union config 2, shared tables", shared)
    pool = G.gpu_pool(M, wl)
    bufs = G.run_gpu_step(M, wl, pool, 1)      # appends the step's tokens, selects
    sel = bufs.sel.cpu().numpy()
    if shared:
        first = {}
        for r in range(wl.num_rows):
            first.setdefault(int(wl.row_seq[r]), r)
        sel = np.stack([sel[first[int(s)]] for s in wl.row_seq])
    groups = M.group_rows_of(wl.row_seq, 4)
    assert len(groups) == 41
    out, _ = _union(M, wl, pool, sel, groups, 4, 1)
    # the one-row decode of the same tables (GPU against GPU, each within the bar of the truth)
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
    one = torch.zeros(wl.num_rows, wl.num_heads, 128, dtype=torch.bfloat16, device="cuda")
    ws = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, 1)
    M.msa_sparse_decode_combine(pool, step, G.dev_bf16(wl.q), torch.from_numpy(sel).cuda(), wl.k,
                                wl.softmax_scale, 1, ws.merge_o, ws.merge_ml, ws.counters, one)
    torch.cuda.synchronize()
    assert np.max(np.abs(out - G.bf16_to_np(one))) <= 2 * G.OUT_ATOL
    _out2, parts = _union(M, wl, pool, sel, groups, 4, 2)
    rng = np.random.default_rng(2024)
    reqs = set(int(s) for s in rng.choice(len(wl.ctx_lens), size=8, replace=False))
    reqs.add(int(np.argmax(wl.ctx_lens)))
    rows = [r for r in range(wl.num_rows) if int(wl.row_seq[r]) in reqs]
    blocks = {s: sorted(set(int(b) for r in rows if wl.row_seq[r] == s for b in sel[r] if b >= 0)) for s in reqs}
    opool = G.oracle_pool(wl, seqs=sorted(reqs), kv_blocks=blocks)
    sub = np.asarray(rows)
    ref = O.attend(opool, wl.block_table, wl.row_seq[sub], wl.row_pos[sub], wl.q[sub], sel[sub], wl.softmax_scale)
    G.assert_out_close(out[sub], ref, "config 2 union outputs")
    G.assert_out_close(_out2[sub], ref, "config 2 union outputs, 2 splits")
    # the partials of the sampled groups against the oracle's union split
    sub_groups = M.group_rows_of(wl.row_seq[sub], 4)
    up = O.union_partials(opool, wl.block_table, wl.row_seq[sub], wl.row_pos[sub], wl.q[sub], sel[sub],
                          wl.softmax_scale, 2, sub_groups)
    _check_partials((parts[0][sub], parts[1][sub]), up, range(len(rows)))


def test_union_edge_cases(M):
    """k = 64 over 4 rows (256 picks), more splits than union entries, zero-row groups,
    and rows in no group (left untouched)."""
    wl = W.small(W.FMT_NVFP4, [9000, 12000], 4, num_kv_heads=1, k=64, seed=45)
    _print("union edge cases", wl.name)
    pool = _full_gpu_pool(M, wl)
    opool = _oracle_pool_all(wl)
    sel = W.verify_tables(wl, 0.4)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    groups = M.group_rows_of(wl.row_seq, 4)
    for ns in (1, 5):
        out, parts = _union(M, wl, pool, sel, groups, 4, ns)
        G.assert_out_close(out, ref, f"k 64, {ns} splits")
        if parts is not None:
            up = O.union_partials(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale,
                                  ns, groups)
            _check_partials(parts, up, range(wl.num_rows))
    # full overlap at k = 5: 5 union entries per group over 20 splits, so most splits
    # hold nothing
    wl5 = W.small(W.FMT_FP8, [1022, 2600], 4, num_kv_heads=1, k=5, seed=46)
    pool5, opool5 = _full_gpu_pool(M, wl5), _oracle_pool_all(wl5)
    sel5 = W.verify_tables(wl5, 1.0)
    groups5 = M.group_rows_of(wl5.row_seq, 4)
    ref5 = O.attend(opool5, wl5.block_table, wl5.row_seq, wl5.row_pos, wl5.q, sel5, wl5.softmax_scale)
    out, parts = _union(M, wl5, pool5, sel5, groups5, 4, 20)
    G.assert_out_close(out, ref5, "20 splits over 5 or 6 entries")
    up = O.union_partials(opool5, wl5.block_table, wl5.row_seq, wl5.row_pos, wl5.q, sel5, wl5.softmax_scale, 20,
                          groups5)
    _check_partials(parts, up, range(wl5.num_rows))
    # zero-row groups and rows in no group: rows 4..7 are not in any group
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos)
    q = G.dev_bf16(wl.q)
    sel_d = torch.from_numpy(sel).cuda()
    gr = torch.tensor([0, 0, 2, 2, 4], dtype=torch.int32, device="cuda")
    o = torch.full((wl.num_rows, wl.num_heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    M.msa_sparse_decode_union(pool, step, q, sel_d, wl.k, gr, 4, wl.softmax_scale, 1, out=o)
    torch.cuda.synchronize()
    got = G.bf16_to_np(o)
    G.assert_out_close(got[:4], ref[:4], "groups [0,0) [0,2) [2,2) [2,4)")
    assert np.isnan(got[4:]).all(), "rows in no group were written"


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_FP8])
def test_union_eight_kv_heads(M, fmt):
    wl = W.small(fmt, [1022, 2600], 4, num_kv_heads=8, k=5, seed=47)
    _print("union, 8 KV heads", wl.name)
    pool = _full_gpu_pool(M, wl)
    opool = _oracle_pool_all(wl)
    sel = W.verify_tables(wl, 0.7)
    ref = O.attend(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    groups = M.group_rows_of(wl.row_seq, 4)
    for ns in (1, 3):
        out, parts = _union(M, wl, pool, sel, groups, 4, ns)
        G.assert_out_close(out, ref, f"8 KV heads, {ns} splits")
        if parts is not None:
            up = O.union_partials(opool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale,
                                  ns, groups)
            _check_partials(parts, up, range(wl.num_rows))
