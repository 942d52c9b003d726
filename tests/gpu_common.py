"""Helpers shared by the GPU parity tests: move seeded workloads to the GPU, run the
HIP path through the C ABI, build the oracle's side independently on the CPU, and
compare to the stated bars."""
from __future__ import annotations

import numpy as np
import torch

from oracle import msa_oracle as O
from synth import workloads as W

SCORE_RTOL = 1e-5      # |S_gpu - S_ref| <= 1e-5 * max(|S_ref|, 1)
OUT_ATOL = 1e-2        # bf16 outputs vs float64 attention
GAP_RTOL = 1e-4        # rows whose k-th / (k+1)-th score gap exceeds this must match bit for bit


def dev_bf16(bits) -> torch.Tensor:
    a = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16)).view(np.int16)
    return torch.from_numpy(a).cuda().view(torch.bfloat16)


def bf16_to_np(t: torch.Tensor) -> np.ndarray:
    return W.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)


def gpu_pool(M, wl: W.Workload):
    """A device pool holding every cached token, written by msa_kv_append."""
    pool = M.KVPool(wl.fmt, wl.num_pages, wl.num_kv_heads, k_tensor_scale=wl.k_tensor_scale,
                    v_tensor_scale=wl.v_tensor_scale, k_page_scale=wl.k_page_scale,
                    v_page_scale=wl.v_page_scale, index_fmt=wl.index_fmt,
                    index_tensor_scale=wl.index_tensor_scale)
    for s in range(len(wl.ctx_lens)):
        L = int(wl.ctx_lens[s])
        if L == 0:
            continue
        slot = torch.from_numpy(wl.slots(s, np.arange(L))).cuda()
        M.msa_kv_append(pool, slot, dev_bf16(wl.k_src[s][:L]), dev_bf16(wl.v_src[s][:L]),
                        dev_bf16(wl.idx_src[s][:L]))
    return pool


def gpu_step_inputs(M, wl: W.Workload, tables=1):
    step = M.Step(wl.block_table, wl.row_seq, wl.row_pos, sel_tables=tables)
    q = dev_bf16(wl.q)
    q_idx = dev_bf16(wl.q_idx)
    w = torch.from_numpy(wl.w).cuda()
    sl, kb, vb, ib = wl.step_tokens()
    app = None
    if len(sl):
        app = (torch.from_numpy(sl).cuda(), dev_bf16(kb), dev_bf16(vb), dev_bf16(ib))
    return step, q, q_idx, w, app


def run_gpu_step(M, wl, pool, num_splits, fused=True, tables=1, select_in="decode"):
    """One step. fused: True (the two fused launches, run_step's default), "single"
    (msa_decode_step, the whole step in one launch, which must accept the shape), False
    (the five separate calls)."""
    step, q, q_idx, w, app = gpu_step_inputs(M, wl, tables)
    bufs = M.DecodeBuffers(wl.num_rows, wl.num_heads, wl.max_blocks, wl.k, num_splits, sel_tables=tables)
    kw = {}
    if app is not None:
        kw = dict(slot=app[0], k_new=app[1], v_new=app[2], idx_k_new=app[3])
    if fused == "single":
        M.msa_decode_step(pool, step, q_idx, w, q, wl.k, wl.n_init, wl.n_local, wl.softmax_scale, num_splits,
                          bufs.score_x, bufs.score_words, bufs.merge_o, bufs.merge_ml, bufs.counters, bufs.out,
                          block_scores=bufs.block_scores, sel=bufs.sel, sel_pages=bufs.sel_pages, **kw)
    else:
        M.run_step(pool, step, bufs, q, q_idx, w, wl.softmax_scale, n_init=wl.n_init,
                   n_local=wl.n_local, fused=bool(fused), select_in=select_in, **kw)
    torch.cuda.synchronize()
    return bufs


def oracle_pool(wl: W.Workload, seqs=None, kv_blocks=None):
    """The oracle's own pool: index keys of every token of `seqs` (all requests if
    None) and K/V of every token, or only of the (seq -> blocks) given in kv_blocks."""
    pool = O.new_pool(wl.fmt, wl.num_pages, wl.num_kv_heads, k_tensor_scale=wl.k_tensor_scale,
                      v_tensor_scale=wl.v_tensor_scale, k_page_scale=wl.k_page_scale,
                      v_page_scale=wl.v_page_scale, index_fmt=wl.index_fmt,
                      index_tensor_scale=wl.index_tensor_scale)
    seqs = range(len(wl.ctx_lens)) if seqs is None else seqs
    for s in seqs:
        T = wl.total_len(s)
        pos = np.arange(T)
        O.kv_append(pool, wl.slots(s, pos), None, None, wl.idx_src[s])
        if kv_blocks is None:
            kv_pos = pos
        else:
            bl = sorted(set(int(b) for b in kv_blocks.get(s, []) if b >= 0))
            kv_pos = np.concatenate([np.arange(b * 128, min((b + 1) * 128, T)) for b in bl]) if bl else \
                np.zeros(0, np.int64)
        if len(kv_pos):
            O.kv_append(pool, wl.slots(s, kv_pos), wl.k_src[s][kv_pos], wl.v_src[s][kv_pos], None)
    return pool


def assert_scores_close(S_gpu, S_ref, rows=None):
    rows = range(S_ref.shape[0]) if rows is None else rows
    for r in rows:
        g, e = S_gpu[r].astype(np.float64), S_ref[r]
        ninf = np.isneginf(e)
        assert np.array_equal(np.isneginf(g), ninf), f"row {r}: -inf pattern differs"
        err = np.abs(g[~ninf] - e[~ninf]) / np.maximum(np.abs(e[~ninf]), 1.0)
        assert err.size == 0 or err.max() <= SCORE_RTOL, f"row {r}: score rel err {err.max():.3g}"


def gap_qualified(S_row, nb, k, n_init=0, n_local=1) -> bool:
    if nb <= k:
        return True
    free = np.asarray([S_row[b] for b in range(n_init, nb - n_local)])
    kk = k - n_init - n_local
    if kk <= 0 or kk >= len(free):
        return True
    srt = np.sort(free)[::-1]
    a, b = srt[kk - 1], srt[kk]
    return (a - b) > GAP_RTOL * abs(a)


def check_selection_valid(sel_row, S_ref_row, nb, k, n_init=0, n_local=1):
    """Where the boundary is too close to call, the GPU's choice must still be a valid
    top-k: min(nb, k) entries of visible blocks in strictly ascending order (so no
    block twice), then only -1 padding, the forced blocks present, and every chosen
    free block's reference score within tolerance of the boundary."""
    row = [int(b) for b in sel_row]
    n = min(nb, k)
    assert len(row) == k and all(b == -1 for b in row[n:]), f"padding {row}"
    chosen = row[:n]
    assert all(0 <= b < nb for b in chosen), f"entries outside the visible blocks {row}"
    assert all(a < b for a, b in zip(chosen, chosen[1:])), f"not strictly ascending {row}"
    forced = set(range(min(n_init, nb))) | set(range(nb - n_local, nb))
    assert forced <= set(chosen)
    if nb <= k:
        return
    free = [b for b in range(n_init, nb - n_local)]
    kk = k - len(forced)
    thr = np.sort([S_ref_row[b] for b in free])[::-1][kk - 1]
    tol = 2 * SCORE_RTOL * max(abs(thr), 1.0)
    for b in chosen:
        if b not in forced:
            assert S_ref_row[b] >= thr - tol


def assert_out_close(out_gpu, out_ref, what=""):
    err = np.abs(out_gpu - out_ref).max()
    assert err <= OUT_ATOL, f"{what} max abs err {err:.4g}"
    return err


def oracle_rows(wl: W.Workload, rows, tables=1, also_sel=None):
    """Index scores, selection and attention of the given rows, computed by the oracle
    from the seeded source alone (it encodes only the pages those rows need). With
    tables > 1, one selection per (row, KV head). also_sel (the rows' selection from
    the GPU, [len(rows)][k] or [len(rows)][T][k]) adds the attention over that table as
    a fifth result, for rows where several selections are valid: the output for a given
    table is unique."""
    rows = list(rows)
    seqs = sorted(set(int(wl.row_seq[r]) for r in rows))
    pool = oracle_pool(wl, seqs=seqs, kv_blocks={s: [] for s in seqs})
    sub = np.asarray(rows)
    S = O.index_score(pool, wl.block_table, wl.row_seq[sub], wl.row_pos[sub], wl.q_idx[sub],
                      wl.w[sub], wl.max_blocks, tables)
    sel = O.select_topk(S, wl.row_pos[sub], wl.k, wl.n_init, wl.n_local)
    for s in seqs:
        mine = [i for i, r in enumerate(rows) if wl.row_seq[r] == s]
        blocks = set(int(b) for i in mine for b in np.ravel(sel[i]) if b >= 0)
        if also_sel is not None:
            blocks |= set(int(b) for i in mine for b in np.ravel(also_sel[i]) if b >= 0)
        blocks = sorted(blocks)
        T = wl.total_len(s)
        pos = np.concatenate([np.arange(b * 128, min((b + 1) * 128, T)) for b in blocks])
        O.kv_append(pool, wl.slots(s, pos), wl.k_src[s][pos], wl.v_src[s][pos], None)
    out = O.attend(pool, wl.block_table, wl.row_seq[sub], wl.row_pos[sub], wl.q[sub], sel,
                   wl.softmax_scale)
    if also_sel is None:
        return S, sel, out, pool
    out_also = O.attend(pool, wl.block_table, wl.row_seq[sub], wl.row_pos[sub], wl.q[sub],
                        np.asarray(also_sel, dtype=np.int32), wl.softmax_scale)
    return S, sel, out, pool, out_also


def assert_merge_ready(bufs):
    """A fused call leaves its merge workspace ready for the next one: every state word
    names the workspace's split count with no arrivals, and the exchange buffer it
    selects holds the idle pattern in that (row, KV head)'s region."""
    import sparse_attention_decode_fp8_amd as M
    S = bufs.num_splits
    c = bufs.counters.cpu().numpy().view(np.uint32)
    assert ((c & ((1 << 26) - 1)) == 0).all(), "arrivals, handoffs or a failure left in a state word"
    assert (((c >> 26) & 0x1f) == S).all(), "state word names another split count"
    rows, hkv = c.shape
    # pair-major, laid out for S splits (a workspace may be allocated for more)
    mo = bufs.merge_o.view(torch.int32).reshape(-1)[:rows * hkv * 2 * 16 * S * 128]
    mm = bufs.merge_ml.view(torch.int32).reshape(-1)[:rows * hkv * 2 * 16 * S * 2]
    mo = mo.reshape(rows, hkv, 2, 16, S, 128).cpu().numpy()
    mm = mm.reshape(rows, hkv, 2, 16, S, 2).cpu().numpy()
    for r in range(rows):
        for g in range(hkv):
            e = int(c[r, g] >> 31)
            assert (mo[r, g, e] == M.MERGE_IDLE_BITS).all(), (r, g)
            assert (mm[r, g, e] == M.MERGE_IDLE_BITS).all(), (r, g)


def assert_score_exchange_idle(bufs):
    """msa_decode_step leaves its score exchange as it found it: every word idle, every
    reader count zero."""
    import sparse_attention_decode_fp8_amd as M
    x = bufs.score_x.view(torch.int32).cpu().numpy().view(np.uint32)
    assert (x == M.MERGE_IDLE_BITS).all(), "score exchange words left written"
    assert int(bufs.score_words.abs().sum().item()) == 0, "reader counts left"


def check_step_parity(M, wl: W.Workload, num_splits: int, fused: bool, tables: int = 1,
                      select_in: str = "decode"):
    """Run one whole step on the GPU and compare scores, selection, outputs and the
    split partials with the oracle, computed from the same seeded source. tables > 1:
    one selection per (row, KV head)."""
    pool = gpu_pool(M, wl)
    bufs = run_gpu_step(M, wl, pool, num_splits, fused=fused, tables=tables, select_in=select_in)
    ref_pool = oracle_pool(wl)
    S_ref = O.index_score(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q_idx, wl.w, wl.max_blocks,
                          tables)
    sel_ref = O.select_topk(S_ref, wl.row_pos, wl.k, wl.n_init, wl.n_local)
    out_ref = O.attend(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel_ref, wl.softmax_scale)
    # per-(row, table) views: table rows r * T + t
    S = bufs.block_scores.cpu().numpy().reshape(wl.num_rows * tables, -1)
    S_flat = S_ref.reshape(wl.num_rows * tables, -1)
    assert_scores_close(S, S_flat)
    sel = bufs.sel.cpu().numpy().reshape(wl.num_rows * tables, -1)
    sel_flat = sel_ref.reshape(wl.num_rows * tables, -1)
    nb = np.repeat(wl.row_pos // 128 + 1, tables)
    same_t = np.ones(wl.num_rows * tables, bool)
    for r in range(wl.num_rows * tables):
        if gap_qualified(S_flat[r], nb[r], wl.k, wl.n_init, wl.n_local):
            assert np.array_equal(sel[r], sel_flat[r]), r
        else:
            check_selection_valid(sel[r], S_flat[r], nb[r], wl.k, wl.n_init, wl.n_local)
            same_t[r] = np.array_equal(sel[r], sel_flat[r])
    same = same_t.reshape(wl.num_rows, tables).all(axis=1)
    out = bf16_to_np(bufs.out)
    assert_out_close(out[same], out_ref[same], "outputs")
    if not same.all():
        # rows where another selection is valid too: the output on the GPU's own
        # (validated) table is unique
        sel_gpu = bufs.sel.cpu().numpy()
        out_gsel = O.attend(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel_gpu,
                            wl.softmax_scale)
        assert_out_close(out[~same], out_gsel[~same], "outputs on the GPU's selection")
    if fused:   # the partials passed through the merge workspace, ready for the next call
        assert_merge_ready(bufs)
        if fused == "single":
            assert_score_exchange_idle(bufs)
        return bufs
    # the split partials the kernel wrote
    m, l, Op = O.split_partials(ref_pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel_ref,
                                wl.softmax_scale, num_splits)
    ml = bufs.part_ml.cpu().numpy()
    po = bufs.part_o.cpu().numpy()
    for r in np.nonzero(same)[0]:
        fin = np.isfinite(m[r])
        assert np.array_equal(np.isneginf(ml[r, :, :, 0]), ~fin)
        assert np.allclose(ml[r, :, :, 0][fin], m[r][fin], rtol=1e-4, atol=1e-3)
        lr = np.where(fin, l[r], 0)
        assert np.allclose(ml[r, :, :, 1], lr, rtol=2e-2, atol=1e-3)
        # O is unnormalised: compare relative to its sum of weights
        den = np.maximum(lr, 1e-30)[..., None]
        assert np.max(np.abs(po[r] / den - Op[r] / den)[fin]) < 1e-2
    return bufs
