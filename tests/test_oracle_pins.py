"""Pins of the float64 oracle against things other than itself: library decode
tables, exact-rational brute force, closed forms, invariants and a library
attention routine. CPU only."""
from fractions import Fraction
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import msa_oracle as O
from synth import workloads as W


# ------------------------------------------------------------------ format tables
def test_e4m3_table_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    tab = O.e4m3_table()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(tab), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(tab[~nan], ref[~nan])


def test_e4m3_table_anchors():
    t = O.E4M3
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert t[0x08] == 2.0 ** -6 and t[0x01] == 2.0 ** -9 and t[0x07] == 7 * 2.0 ** -9
    assert t[0x38] == 1.0 and t[0x40] == 2.0 and t[0xC0] == -2.0 and t[0x00] == 0.0
    finite = t[~np.isnan(t)]
    assert np.nanmax(np.abs(finite)) == 448.0
    # codes 0..126 are strictly increasing (used by the encoder as a grid)
    assert np.all(np.diff(t[:127]) > 0)


def test_e2m1_table_anchors():
    t = O.E2M1
    assert list(t[:8]) == [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(t[8:]) == [-0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0]


# ------------------------------------------------------------------ encoders
def _fr(x):
    return Fraction(float(x))


def _brute_nearest(x, values_by_code, codes, lsb_even):
    """Nearest code by exact rational distance; ties to the code with even LSB."""
    fx = _fr(x)
    best, bestd = None, None
    for c in codes:
        d = abs(fx - _fr(values_by_code[c]))
        if bestd is None or d < bestd or (d == bestd and lsb_even(c) and not lsb_even(best)):
            best, bestd = c, d
    return best


def _brute_e4m3(x):
    ref = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    neg = math.copysign(1.0, float(x)) < 0
    codes = [c for c in range(256) if not np.isnan(ref[c]) and ((c >= 0x80) == neg)]
    if abs(float(x)) >= 448.0:
        return 0xFE if neg else 0x7E
    return _brute_nearest(x, ref, codes, lambda c: c % 2 == 0)


def _e4m3_probe_values():
    t = O.E4M3[:127]
    mids = (t[:-1] + t[1:]) / 2            # exact ties
    rng = np.random.default_rng(11)
    rnd = rng.standard_normal(300) * np.exp2(rng.integers(-12, 10, 300))
    v = np.concatenate([t, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9), rnd,
                        [450.0, 463.9, 464.0, 1e6, 2.0 ** -10, 2.0 ** -11, 3 * 2.0 ** -11]])
    v = np.concatenate([v, -v]).astype(np.float32).astype(np.float64)
    return v


def test_e4m3_encode_brute_force_and_torch():
    v = _e4m3_probe_values()
    got = O.e4m3_encode(v)
    for x, c in zip(v, got):
        assert c == _brute_e4m3(x), (x, c)
    inr = np.abs(v) < 448.0
    tor = torch.tensor(v[inr], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of values that round to zero, as we do
    assert np.array_equal(tor, got[inr])


def _brute_e2m1(x):
    neg = math.copysign(1.0, float(x)) < 0
    codes = list(range(8, 16)) if neg else list(range(8))
    if abs(float(x)) >= 6.0:
        return 15 if neg else 7
    return _brute_nearest(x, O.E2M1, codes, lambda c: c % 2 == 0)


def test_e2m1_encode_brute_force_with_ties():
    grid = O.E2M1[:8]
    mids = (grid[:-1] + grid[1:]) / 2
    v = np.concatenate([grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
                        [6.5, 7.0, 100.0, 0.1, 0.3]])
    v = np.concatenate([v, -v])
    got = O.e2m1_encode(v)
    for x, c in zip(v, got):
        assert c == _brute_e2m1(x), (x, c)
    # explicit tie outcomes (round half to even code)
    exp = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in exp.items():
        assert O.e2m1_encode(np.array([x]))[0] == c


def _f32(fr):
    return Fraction(float(np.float32(float(fr))))


def _brute_nvfp4_group(x16, t):
    """The stated NVFP4 recipe computed with exact rationals and brute-force rounding."""
    t = _f32(Fraction(float(t)))
    amax = max(abs(_fr(v)) for v in x16)
    y = _f32(amax / _f32(6 * t))
    sc = _brute_e4m3(float(y))
    dec = _fr(O.E4M3[sc])
    if dec == 0:
        return [0] * 16, sc
    d = _f32(dec * t)
    return [_brute_e2m1(float(_f32(_fr(v) / d))) for v in x16], sc


def test_nvfp4_encode_matches_exact_rational_recipe():
    rng = np.random.default_rng(5)
    x = W.bf16_bits_to_f32(W.to_bf16_bits(rng.standard_normal((40, 32), dtype=np.float32)))
    x[3, :16] *= 1e-4          # tiny group: scale rounds low
    x[4, :16] = 0.0            # all-zero group
    x[5, 16:] *= 60.0          # group above the tensor amax: saturating scale
    t = float(np.float32(4.0 / (6 * 448)))
    codes, sc = O.nvfp4_encode(x.astype(np.float64), t)
    for r in range(x.shape[0]):
        for g in range(2):
            bc, bs = _brute_nvfp4_group(x[r, 16 * g:16 * g + 16], t)
            assert sc[r, g] == bs
            assert list(codes[r, 16 * g:16 * g + 16]) == bc


def test_nvfp4_reconstruction_bound():
    """Every element decodes to within half an E2M1 step (times the group scale)
    unless it saturates; the group amax lands in the top binade."""
    rng = np.random.default_rng(6)
    x = W.bf16_bits_to_f32(W.to_bf16_bits(rng.standard_normal((500, 128), dtype=np.float32))).astype(np.float64)
    t = float(np.float32(np.abs(x).max() / (6 * 448)))
    codes, sc = O.nvfp4_encode(x, t)
    d = np.repeat(O.E4M3[sc] * t, 16, axis=1)
    rec = O.E2M1[codes] * d
    step = np.where(np.abs(x / d) < 2, 0.5, np.where(np.abs(x / d) < 4, 1.0, 2.0)) * d
    assert np.all(np.abs(rec - x) <= step / 2 * (1 + 1e-6) + 1e-30)
    g = np.abs(x).reshape(500, 8, 16).max(-1) / O.E4M3[sc] / t
    assert np.all((g > 5.0) & (g < 6.5))


def test_pack_nibbles_low_is_even():
    assert O.pack_nibbles(np.array([1, 2], np.uint8))[0] == 0x21
    assert list(O.unpack_nibbles(np.array([0xA5], np.uint8))) == [5, 10]


def test_fp8_kv_encode_is_scaled_e4m3():
    x = np.array([1.0, -3.0, 0.0, 1000.0])
    s = 0.5
    assert list(O.fp8_kv_encode(x, s)) == [0x40, 0xCC, 0x00, 0x7E]  # 2.0, -6.0 (1.5*2^2), 0, sat


# ------------------------------------------------------------------ append
def test_kv_append_writes_only_its_slot_and_skips_negative():
    pool = O.new_pool(O.FMT_NVFP4, 4, 2, k_tensor_scale=0.01, v_tensor_scale=0.01)
    rng = np.random.default_rng(1)
    kb = W.to_bf16_bits(rng.standard_normal((2, 2, 128), dtype=np.float32))
    ib = W.to_bf16_bits(rng.standard_normal((2, 64), dtype=np.float32))
    O.kv_append(pool, np.array([2 * 128 + 5, -1]), kb, kb, ib)
    nz = np.argwhere(pool["k_codes"] != 0)
    assert set(map(tuple, nz[:, [0, 2]])) == {(2, 5)}
    assert np.argwhere(pool["index_k"] != 0)[:, :2].tolist() == [[2, 5]] * int((pool["index_k"] != 0).sum())
    assert np.array_equal(pool["index_k"][2, 5], O.e4m3_encode(W.bf16_bits_to_f32(ib[0])))


# ------------------------------------------------------------------ index score
def _tiny_pool_with_keys(keys, Hkv=1):
    """keys: float array [n_tok][64] of E4M3-representable values at positions 0.."""
    n = keys.shape[0]
    pages = (n + 127) // 128
    pool = O.new_pool(O.FMT_FP8, pages + 1, Hkv)
    bt = np.array([list(range(pages, 0, -1))], dtype=np.int32)   # reversed physical order
    for p in range(n):
        b, off = divmod(p, 128)
        pool["index_k"][bt[0, b], off] = O.e4m3_encode(keys[p])
    return pool, bt


def test_index_score_unit_key_closed_form():
    keys = np.zeros((130, 64))
    keys[7, 13] = 1.0          # block 0, a unit key along dim 13
    keys[129, 2] = 1.0         # block 1
    pool, bt = _tiny_pool_with_keys(keys)
    rng = np.random.default_rng(3)
    q = W.to_bf16_bits(rng.standard_normal((1, 4, 64), dtype=np.float32))
    w = np.array([[0.25, 0.5, 0.75, 1.0]], np.float32)
    S = O.index_score(pool, bt, [0], [129], q, w, 3)
    qf = W.bf16_bits_to_f32(q[0]).astype(np.float64)
    exp0 = (w[0] * np.maximum(qf[:, 13], 0)).sum()
    exp1 = (w[0] * np.maximum(qf[:, 2], 0)).sum()
    assert S[0, 0] == pytest.approx(max(exp0, 0.0), abs=0, rel=1e-15)
    assert S[0, 1] == pytest.approx(max(exp1, 0.0), abs=0, rel=1e-15)
    assert S[0, 2] == -np.inf


def test_index_score_negative_dots_give_zero_and_mask_hides_future():
    keys = np.zeros((256, 64))
    keys[:, 0] = -1.0                     # every dot negative when q[:,0] > 0
    keys[200, 0] = 8.0                    # a strong key after row_pos
    pool, bt = _tiny_pool_with_keys(keys)
    q = np.zeros((1, 4, 64), np.float32)
    q[0, :, 0] = 1.0
    S = O.index_score(pool, bt, [0], [150], W.to_bf16_bits(q), np.ones((1, 4), np.float32), 2)
    assert S[0, 0] == 0.0 and S[0, 1] == 0.0          # masked token 200 not seen
    S2 = O.index_score(pool, bt, [0], [200], W.to_bf16_bits(q), np.ones((1, 4), np.float32), 2)
    assert S2[0, 1] == 32.0                            # 4 heads * 1 * 8


def test_index_score_invariant_to_physical_page_order():
    wl = W.small(W.FMT_FP8, [700, 300], 0, num_kv_heads=1, k=2, seed=9)
    pool = _oracle_pool(wl)
    S = O.index_score(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q_idx, wl.w, wl.max_blocks)
    # move every page to a new physical slot
    perm = np.random.default_rng(2).permutation(wl.num_pages)
    pool2 = dict(pool)
    pool2["index_k"] = np.empty_like(pool["index_k"])
    pool2["index_k"][perm] = pool["index_k"]
    bt2 = np.where(wl.block_table >= 0, perm[np.maximum(wl.block_table, 0)], -1)
    S2 = O.index_score(pool2, bt2, wl.row_seq, wl.row_pos, wl.q_idx, wl.w, wl.max_blocks)
    assert np.array_equal(S, S2)


# ------------------------------------------------------------------ select
def _dominance_select(S_row, nb, k, n_init, n_local):
    """The unique k-subset containing the forced blocks in which every chosen
    free block beats every unchosen free block (higher score, then smaller index)."""
    forced = set(range(min(n_init, nb))) | set(range(nb - n_local, nb))
    free = [b for b in range(nb) if b not in forced]
    beats = lambda a, b: (S_row[a] > S_row[b]) or (S_row[a] == S_row[b] and a < b)
    found = []
    for comb in itertools.combinations(free, k - len(forced)):
        cs = set(comb)
        if all(beats(a, b) for a in cs for b in free if b not in cs):
            found.append(sorted(cs | forced))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("seed", range(6))
def test_select_matches_dominance_brute_force(seed):
    rng = np.random.default_rng(seed)
    nb, k = 9, 4
    S = np.round(rng.standard_normal((3, nb + 2)), 1)     # coarse values: many ties
    S[:, nb:] = -np.inf
    pos = np.full(3, (nb - 1) * 128 + 17)
    for n_init in (0, 1):
        sel = O.select_topk(S, pos, k, n_init=n_init, n_local=1)
        for r in range(3):
            assert list(sel[r]) == _dominance_select(S[r], nb, k, n_init, 1)


def test_select_tie_break_over_1024_ties():
    nb, k = 2048, 32
    S = np.full((1, nb), -5.0)
    tied = np.sort(np.random.default_rng(4).choice(nb - 1, 1100, replace=False))
    S[0, tied] = 7.25
    sel = O.select_topk(S, [nb * 128 - 1], k)
    assert list(sel[0]) == sorted(list(tied[:k - 1]) + [nb - 1])


def test_select_identity_and_padding_and_forced_last():
    S = np.array([[3.0, 2.0, 1.0, -np.inf, -np.inf]])
    assert list(O.select_topk(S, [2 * 128 + 5], 5)[0]) == [0, 1, 2, -1, -1]
    S = np.array([[9.0, 8.0, 7.0, 6.0, -1.0]])   # last block is the worst but forced
    assert list(O.select_topk(S, [4 * 128], 3)[0]) == [0, 1, 4]


# ------------------------------------------------------------------ attention
def _oracle_pool(wl, with_step=True):
    pool = O.new_pool(wl.fmt, wl.num_pages, wl.num_kv_heads, k_tensor_scale=wl.k_tensor_scale,
                      v_tensor_scale=wl.v_tensor_scale, k_page_scale=wl.k_page_scale,
                      v_page_scale=wl.v_page_scale)
    sl, kb, vb, ib = wl.prefill_tokens()
    O.kv_append(pool, sl, kb, vb, ib)
    if with_step:
        sl, kb, vb, ib = wl.step_tokens()
        O.kv_append(pool, sl, kb, vb, ib)
    return pool


def _exact_nvfp4_vectors(rng, shape, t):
    """Vectors (last axis a multiple of 16) that NVFP4 holds exactly at tensor scale t (a
    power of two): each 16-group is E2M1 values times one E4M3 scale times t, with the
    group's largest magnitude exactly 6 * scale * t, so the recipe picks that scale and
    codes every element exactly. The scales of one vector's groups are all different
    (some with a mantissa, 1.25 = 0x3A, 1.75 = 0x3E, ...), so a scale applied to the
    wrong group changes the value."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    n = shape[-1] // 16
    scale_set = np.array([2.0 ** e * m for e in range(-4, 3) for m in (1.0, 1.25, 1.5, 1.75)])
    out = np.empty(shape)
    flat = out.reshape(-1, n, 16)
    for i in range(flat.shape[0]):
        scales = rng.choice(scale_set, n, replace=False)
        for g in range(n):
            v = rng.choice(grid, 16) * rng.choice([-1, 1], 16)
            v[rng.integers(16)] = 6.0 * rng.choice([-1, 1])
            flat[i, g] = v * scales[g] * t
    return out


def _exact_fp8_values(rng, shape, page_scale):
    """Values E4M3(code) * page_scale for random non-NaN codes (subnormals, both signs
    of zero and 448 included), exactly representable in bf16 for a power-of-two scale.
    The code values come from torch's float8_e4m3fn, not from the oracle's table."""
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    codes = rng.choice(np.array([c for c in range(256) if c not in (0x7F, 0xFF)]), shape)
    return lib[codes] * page_scale, codes


def _exact_kv(wl, rng):
    """Rewrite a workload's K/V source with values its KV format holds exactly, and its
    scales with distinct powers of two: NVFP4 tensor scales 2^-5 (K) and 2^-3 (V);
    FP8 page scales 2^(page % 7 - 3) for K and 2^(2 - page % 5) for V. The source
    is then the exact value of every appended token, independently of the oracle's
    decoding."""
    if wl.fmt == W.FMT_NVFP4:
        wl.k_tensor_scale, wl.v_tensor_scale = 2.0 ** -5, 2.0 ** -3
        for s in range(len(wl.ctx_lens)):
            T = wl.total_len(s)
            shp = (T, wl.num_kv_heads, wl.head_dim)
            wl.k_src[s] = W.to_bf16_bits(_exact_nvfp4_vectors(rng, shp, wl.k_tensor_scale).astype(np.float32))
            wl.v_src[s] = W.to_bf16_bits(_exact_nvfp4_vectors(rng, shp, wl.v_tensor_scale).astype(np.float32))
    else:
        pages = np.arange(wl.num_pages)
        wl.k_page_scale = (2.0 ** (pages % 7 - 3)).astype(np.float32)
        wl.v_page_scale = (2.0 ** (2 - pages % 5)).astype(np.float32)
        for s in range(len(wl.ctx_lens)):
            T = wl.total_len(s)
            page = wl.block_table[s][np.arange(T) // 128]
            shp = (T, wl.num_kv_heads, wl.head_dim)
            kv, _ = _exact_fp8_values(rng, shp, wl.k_page_scale[page][:, None, None].astype(np.float64))
            vv, _ = _exact_fp8_values(rng, shp, wl.v_page_scale[page][:, None, None].astype(np.float64))
            wl.k_src[s] = W.to_bf16_bits(kv.astype(np.float32))
            wl.v_src[s] = W.to_bf16_bits(vv.astype(np.float32))
    return wl


def _dense_sdpa(wl, r):
    """torch scaled_dot_product_attention (float64, CPU) over all visible tokens, on the
    workload's exact K/V source values (see _exact_kv): it never decodes the pool."""
    seq, pos = int(wl.row_seq[r]), int(wl.row_pos[r])
    outs = []
    q = torch.tensor(W.bf16_bits_to_f32(wl.q[r]).astype(np.float64))
    K_all = W.bf16_bits_to_f32(wl.k_src[seq][:pos + 1]).astype(np.float64)   # [T][Hkv][D]
    V_all = W.bf16_bits_to_f32(wl.v_src[seq][:pos + 1]).astype(np.float64)
    for g in range(wl.num_kv_heads):
        K, V = K_all[:, g], V_all[:, g]
        qg = q[16 * g:16 * g + 16][None]                       # [1, 16, D]
        o = torch.nn.functional.scaled_dot_product_attention(
            qg, torch.tensor(K)[None].contiguous(), torch.tensor(V)[None].contiguous(),
            scale=wl.softmax_scale)
        outs.append(o[0].numpy())
    return np.concatenate(outs)


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_sparse_equals_dense_when_all_blocks_selected(fmt):
    wl = _exact_kv(W.small(fmt, [300, 129], 2, num_kv_heads=2, k=4, seed=21), np.random.default_rng(24))
    pool = _oracle_pool(wl)
    sel = np.tile(np.arange(4, dtype=np.int32), (wl.num_rows, 1))
    nb = wl.row_pos // 128 + 1
    sel = np.where(np.arange(4)[None] < nb[:, None], sel, -1).astype(np.int32)
    out = O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    for r in range(wl.num_rows):
        ref = _dense_sdpa(wl, r)
        # fp64 rounding only (the FP8 source reaches 448 * 8, so the bound is relative)
        assert np.max(np.abs(out[r] - ref)) <= 1e-13 * max(1.0, np.max(np.abs(ref)))


@pytest.mark.parametrize("fmt", [W.FMT_FP8, W.FMT_NVFP4])
def test_kv_round_trips_exactly_through_append_and_dequant(fmt):
    """K and V values the format holds exactly come back bit for bit from kv_append +
    dequant_page, for every page and KV head, with NVFP4 group scales that differ
    inside each token and non-unit tensor scales that differ between K and V, and FP8
    page scales that differ from page to page and between K and V. A scale broadcast
    that tiles instead of repeating, a dropped tensor scale, the other tensor's scale,
    or the scale of a neighbouring page fails here. Slots never written decode to 0."""
    rng = np.random.default_rng(25)
    wl = _exact_kv(W.small(fmt, [200, 300], 1, num_kv_heads=2, k=4, seed=26), rng)
    pool = _oracle_pool(wl)
    written = np.zeros((wl.num_pages, 128), bool)
    for s in range(len(wl.ctx_lens)):
        T = wl.total_len(s)
        for p in range(T):
            page = int(wl.block_table[s][p // 128])
            written[page, p % 128] = True
            for kv, src in (("k", wl.k_src[s]), ("v", wl.v_src[s])):
                exact = W.bf16_bits_to_f32(src[p]).astype(np.float64)          # [Hkv][D]
                for g in range(wl.num_kv_heads):
                    got = O.dequant_page(pool, page, g, kv)[p % 128]
                    assert np.array_equal(got, exact[g]), (fmt, kv, s, p, g)
    for page in range(wl.num_pages):
        for g in range(wl.num_kv_heads):
            for kv in ("k", "v"):
                assert not O.dequant_page(pool, page, g, kv)[~written[page]].any()


def test_fp8_kv_append_codes_use_each_pages_own_scales():
    """FP8 append: the code written for x on page p is the E4M3 code c with
    x = E4M3[c] * scale_p, for K with the K scale and for V with the V scale of that
    page (closed form: the codes the values were made from)."""
    rng = np.random.default_rng(27)
    k_sc = np.array([0.25, 8.0, 2.0 ** -5, 2.0], np.float32)
    v_sc = np.array([4.0, 0.125, 1.0, 2.0 ** -4], np.float32)
    pool = O.new_pool(O.FMT_FP8, 4, 2, k_page_scale=k_sc, v_page_scale=v_sc)
    slots = np.array([0 * 128 + 3, 1 * 128 + 0, 2 * 128 + 127, 3 * 128 + 64, 1 * 128 + 5])
    page = slots // 128
    kx, kc = _exact_fp8_values(rng, (5, 2, 128), k_sc[page][:, None, None].astype(np.float64))
    vx, vc = _exact_fp8_values(rng, (5, 2, 128), v_sc[page][:, None, None].astype(np.float64))
    O.kv_append(pool, slots, W.to_bf16_bits(kx.astype(np.float32)), W.to_bf16_bits(vx.astype(np.float32)), None)
    for i, sl in enumerate(slots):
        assert np.array_equal(pool["k_codes"][sl // 128, :, sl % 128], kc[i])
        assert np.array_equal(pool["v_codes"][sl // 128, :, sl % 128], vc[i])
    assert np.array_equal(pool["k_scales"], k_sc) and np.array_equal(pool["v_scales"], v_sc)   # read, not written


def test_split_combine_identity():
    wl = W.small(W.FMT_NVFP4, [900, 400], 1, num_kv_heads=2, k=5, seed=22)
    pool = _oracle_pool(wl)
    S = O.index_score(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q_idx, wl.w, wl.max_blocks)
    sel = O.select_topk(S, wl.row_pos, wl.k)
    ref = O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
    for ns in (1, 2, 3, 5):
        m, l, Op = O.split_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel,
                                    wl.softmax_scale, ns)
        assert np.max(np.abs(O.combine(m, l, Op) - ref)) < 1e-12


def test_attend_single_token_and_equal_logits():
    pool = O.new_pool(O.FMT_FP8, 2, 1, k_page_scale=[1.0, 1.0], v_page_scale=[1.0, 1.0])
    pool["v_codes"][1, 0, 0] = O.e4m3_encode(np.full(128, 1.5))
    pool["v_codes"][1, 0, 1] = O.e4m3_encode(np.full(128, -0.5))
    bt = np.array([[1]], np.int32)
    q = W.to_bf16_bits(np.ones((1, 16, 128), np.float32))
    out = O.attend(pool, bt, [0], [0], q, np.array([[0]], np.int32), 0.1)
    assert np.all(out == 1.5)                  # one visible token: its V
    out = O.attend(pool, bt, [0], [1], q, np.array([[0]], np.int32), 0.1)
    assert np.allclose(out, 0.5, atol=0, rtol=1e-15)   # K = 0: equal logits, mean of V


def test_partials_single_token_closed_form():
    pool = O.new_pool(O.FMT_FP8, 1, 1, k_page_scale=[1.0], v_page_scale=[1.0])
    pool["k_codes"][0, 0, 0] = O.e4m3_encode(np.full(128, 0.5))
    pool["v_codes"][0, 0, 0] = O.e4m3_encode(np.full(128, 2.0))
    q = W.to_bf16_bits(np.ones((1, 16, 128), np.float32))
    m, l, Op = O.split_partials(pool, np.array([[0]], np.int32), [0], [0], q,
                                np.array([[0, -1]], np.int32), 0.125, 2)
    assert np.allclose(m[0, :, 0], 0.125 * 64 * oracle.LOG2E, rtol=1e-15)
    assert np.all(l[0, :, 0] == 1.0) and np.all(Op[0, :, 0] == 2.0)
    assert np.all(np.isneginf(m[0, :, 1])) and np.all(l[0, :, 1] == 0)


def test_decode_step_small_verify_workload_runs():
    wl = W.small(W.FMT_NVFP4, [1000, 2600, 130], 3, num_kv_heads=1, k=4, seed=23)
    pool = _oracle_pool(wl, with_step=False)
    sl, kb, vb, ib = wl.step_tokens()
    S, sel, out = O.decode_step(pool, wl.block_table, wl.row_seq, wl.row_pos, sl, kb, vb, ib,
                                wl.q_idx, wl.w, wl.q, wl.k, wl.softmax_scale, wl.max_blocks)
    nb = wl.row_pos // 128 + 1
    for r in range(wl.num_rows):
        assert sel[r, min(nb[r], wl.k) - 1] == nb[r] - 1 if nb[r] > wl.k else True
        assert np.all(np.isfinite(S[r, :nb[r]])) and np.all(np.isneginf(S[r, nb[r]:]))
    assert np.all(np.isfinite(out))


# ---- NVFP4 index keys (reading: the KV's NVFP4 recipe applied to the 64-d index key)
def _nvfp4_exact_keys(rng, n, t, pow2_scales=False):
    """Keys that NVFP4 holds exactly: each 16-group is E2M1 values times one E4M3 scale
    times t, with the group's largest magnitude 6 * scale * t (so the encoder picks
    exactly that scale: amax / (6 t) is an E4M3 value). With power-of-two scales the
    values have at most 2 significant bits, so E4M3 holds them exactly too."""
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6])
    keys = np.empty((n, 64))
    for i in range(n):
        for g in range(4):
            sc = 2.0 ** rng.integers(-3, 4) * (1.0 if pow2_scales else rng.choice([1.0, 1.25, 1.5, 1.75]))
            v = rng.choice(grid, 16) * rng.choice([-1, 1], 16)
            v[rng.integers(16)] = 6.0 * rng.choice([-1, 1])        # the group's amax
            keys[i, 16 * g:16 * g + 16] = v * sc * t
    return keys


def test_nvfp4_index_keys_round_trip_exactly():
    rng = np.random.default_rng(61)
    t = 0.0625                                   # a power of two keeps every product exact
    keys = _nvfp4_exact_keys(rng, 40, t)
    bits = W.to_bf16_bits(keys.astype(np.float32))
    assert np.array_equal(W.bf16_bits_to_f32(bits), keys)       # exact in bf16 too
    pool = O.new_pool(O.FMT_FP8, 2, 1, index_fmt=O.IDX_NVFP4, index_tensor_scale=t)
    slots = np.concatenate([np.arange(3, 23), 128 + np.arange(100, 120)])
    O.kv_append(pool, slots, None, None, bits)
    got = np.concatenate([O.index_keys(pool, 0, 23)[3:], O.index_keys(pool, 1, 120)[100:]])
    assert np.array_equal(got, keys)
    # untouched slots stay zero; token p = 16 t + n of group g sits at [g][n][t]; the
    # low nibble holds the even element
    written = np.zeros((2, 16, 8), bool)
    for pg, p in [(0, p) for p in range(3, 23)] + [(1, p) for p in range(100, 120)]:
        written[pg, p % 16, p // 16] = True
    for pg in range(2):
        assert not pool["index_scales"][pg][:, ~written[pg]].any()
        assert not pool["index_k"][pg][:, ~written[pg]].any()
    c = O.unpack_nibbles(pool["index_k"][0, 1, 3 % 16, 3 // 16])           # token 3, group 1
    assert np.array_equal(O.E2M1[c] * O.E4M3[pool["index_scales"][0, 1, 3, 0]] * t, keys[0, 16:32])


def test_index_score_same_for_nvfp4_and_e4m3_keys_that_both_hold_exactly():
    rng = np.random.default_rng(62)
    t = 1.0
    L = 300
    keys = _nvfp4_exact_keys(rng, L, t, pow2_scales=True)   # |keys| <= 6 * 8 < 448
    bits = W.to_bf16_bits(keys.astype(np.float32))
    bt = np.array([[2, 0, 1]], np.int32)
    slots = bt[0][np.arange(L) // 128].astype(np.int64) * 128 + np.arange(L) % 128
    pools = []
    for fmt in (O.IDX_E4M3, O.IDX_NVFP4):
        p = O.new_pool(O.FMT_FP8, 3, 1, index_fmt=fmt, index_tensor_scale=t)
        O.kv_append(p, slots, None, None, bits)
        pools.append(p)
    assert np.array_equal(O.index_keys(pools[0], 2, 128), O.index_keys(pools[1], 2, 128))
    q = W.to_bf16_bits(rng.standard_normal((2, 4, 64)).astype(np.float32))
    w = rng.random((2, 4)).astype(np.float32)
    S0 = O.index_score(pools[0], bt, [0, 0], [L - 1, 200], q, w, 3)
    S1 = O.index_score(pools[1], bt, [0, 0], [L - 1, 200], q, w, 3)
    assert np.array_equal(S0, S1) and np.isfinite(S0[0]).all() and np.isneginf(S0[1, 2])


# ---- per-KV-head selection tables (reading: T tables per row, index heads split into
# T consecutive equal groups; KV head g attends the blocks of table g)
def test_index_score_per_table_unit_key_closed_form():
    keys = np.zeros((130, 64))
    keys[7, 13] = 1.0          # block 0: a unit key along dim 13
    keys[129, 2] = 1.0         # block 1: along dim 2
    pool, bt = _tiny_pool_with_keys(keys)
    q = np.zeros((1, 4, 64), np.float32)
    q[0, :, 13] = [1.0, -2.0, 3.0, 0.5]
    q[0, :, 2] = [-1.0, 4.0, 0.25, 2.0]
    w = np.array([[0.5, 0.25, 2.0, 1.0]], np.float32)
    qb = W.to_bf16_bits(q)
    S4 = O.index_score(pool, bt, [0], [129], qb, w, 3, tables=4)
    # table t holds index head t alone: w_t * relu(q_t[d])
    assert list(S4[0, :, 0]) == [0.5, 0.0, 6.0, 0.5]
    assert list(S4[0, :, 1]) == [0.0, 1.0, 0.5, 2.0]
    S2 = O.index_score(pool, bt, [0], [129], qb, w, 3, tables=2)
    # table 0: heads 0, 1; table 1: heads 2, 3
    assert list(S2[0, :, 0]) == [0.5, 6.5]
    assert list(S2[0, :, 1]) == [1.0, 2.5]
    assert np.all(np.isneginf(S4[0, :, 2])) and np.all(np.isneginf(S2[0, :, 2]))
    S1 = O.index_score(pool, bt, [0], [129], qb, w, 3)
    assert list(S1[0, :2]) == [7.0, 3.5]


def test_index_score_tables_partition_the_heads():
    """Every token's score is the sum of its per-table terms: with one token per block
    the shared block score is the sum of the table scores."""
    rng = np.random.default_rng(71)
    keys = np.zeros((128 * 3, 64))
    for b in range(3):
        keys[128 * b + 5] = O.e4m3_table()[O.e4m3_encode(rng.standard_normal(64))]
    pool, bt = _tiny_pool_with_keys(keys)
    for p in range(128 * 3):
        if p % 128 != 5:
            pool["index_k"][bt[0, p // 128], p % 128] = 0      # zero keys score 0
    q = W.to_bf16_bits(rng.standard_normal((1, 4, 64), dtype=np.float32))
    w = rng.uniform(0, 1, (1, 4)).astype(np.float32)
    S1 = O.index_score(pool, bt, [0], [3 * 128 - 1], q, w, 3)
    for T in (2, 4):
        ST = O.index_score(pool, bt, [0], [3 * 128 - 1], q, w, 3, tables=T)
        assert np.allclose(ST[0].sum(axis=0), S1[0], rtol=1e-15, atol=0)


def test_select_per_table_matches_dominance_brute_force():
    rng = np.random.default_rng(72)
    nb, k, T = 9, 4, 3
    S = np.round(rng.standard_normal((2, T, nb + 1)), 1)
    S[:, :, nb:] = -np.inf
    pos = np.full(2, (nb - 1) * 128 + 3)
    sel = O.select_topk(S, pos, k)
    assert sel.shape == (2, T, k)
    for r in range(2):
        for t in range(T):
            assert list(sel[r, t]) == _dominance_select(S[r, t], nb, k, 0, 1)


def test_attend_per_kv_head_tables_reduce_to_shared_tables():
    """KV head g with table g gives the heads of g exactly what a shared table equal
    to table g gives them (and equal tables give the shared result everywhere)."""
    wl = W.small(W.FMT_NVFP4, [900, 700], 1, num_kv_heads=2, k=3, seed=73)
    pool = _oracle_pool(wl)
    rng = np.random.default_rng(74)
    nb = wl.row_pos // 128 + 1
    sel3 = np.full((wl.num_rows, 2, wl.k), -1, np.int32)
    for r in range(wl.num_rows):
        for g in range(2):
            pick = np.sort(rng.choice(nb[r] - 1, wl.k - 1, replace=False))
            sel3[r, g] = list(pick) + [nb[r] - 1]
    out3 = O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel3, wl.softmax_scale)
    for g in range(2):
        shared = O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel3[:, g],
                          wl.softmax_scale)
        assert np.array_equal(out3[:, 16 * g:16 * g + 16], shared[:, 16 * g:16 * g + 16])
    same = np.repeat(sel3[:, :1], 2, axis=1)
    assert np.array_equal(O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, same, wl.softmax_scale),
                          O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel3[:, 0], wl.softmax_scale))
    for ns in (1, 2, 3):
        m, l, Op = O.split_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel3,
                                    wl.softmax_scale, ns)
        assert np.max(np.abs(O.combine(m, l, Op) - out3)) < 1e-12


# ---- union partials (query pairing: groups of rows over the union of their tables)
def _groups(row_seq, size):
    starts = [0]
    for i in range(1, len(row_seq) + 1):
        if i == len(row_seq) or row_seq[i] != row_seq[i - 1] or i - starts[-1] == size:
            starts.append(i)
    return starts


@pytest.mark.parametrize("fmt", [W.FMT_NVFP4, W.FMT_FP8])
def test_union_partials_combine_to_each_rows_attention(fmt):
    # verify rows that cross a page boundary (1022..1025, 126..129), so rows of a group
    # see different numbers of tokens of a shared block
    wl = W.small(fmt, [1022, 1500, 126], 4, num_kv_heads=2, k=5, seed=31)
    pool = _oracle_pool(wl)
    for overlap in (0.0, 0.6, 1.0):
        sel = W.verify_tables(wl, overlap)
        ref = O.attend(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale)
        for size in (4, 2, 3):
            groups = _groups(wl.row_seq, size)
            for ns in (1, 2, 3, 7):
                m, l, Op = O.union_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel,
                                            wl.softmax_scale, ns, groups)
                err = np.max(np.abs(O.combine(m, l, Op) - ref))
                assert err < 1e-12 * max(1.0, np.max(np.abs(ref))), (overlap, size, ns, err)


def test_union_partials_of_one_row_groups_are_split_partials():
    # a group of one row whose table has k distinct blocks: its union is its table, so
    # the union split is the table split
    wl = W.small(W.FMT_NVFP4, [1500, 2200], 1, num_kv_heads=2, k=6, seed=32)
    pool = _oracle_pool(wl)
    sel = W.verify_tables(wl, 0.0)
    assert (sel >= 0).all()
    groups = list(range(wl.num_rows + 1))
    for ns in (1, 2, 4, 6):
        a = O.union_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale, ns, groups)
        b = O.split_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale, ns)
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_union_split_follows_first_pick_order_and_row_masks():
    # two rows of one request at positions 300 and 301; tables [0, 2] and [1, 2]: the
    # union is [0, 2, 1] (first picks, rows in order), so with 3 splits block 0 is split 0
    # (row 0 only), block 2 split 1 (both rows; row 0 sees 45 of its tokens, row 1 46)
    # and block 1 split 2 (row 1 only)
    wl = W.small(W.FMT_FP8, [300], 2, num_kv_heads=1, k=2, seed=33)
    assert list(wl.row_pos) == [300, 301]
    pool = _oracle_pool(wl)
    sel = np.array([[0, 2], [1, 2]], np.int32)
    m, l, Op = O.union_partials(pool, wl.block_table, wl.row_seq, wl.row_pos, wl.q, sel, wl.softmax_scale, 3, [0, 2])
    assert np.isneginf(m[0, :, 2]).all() and (l[0, :, 2] == 0).all() and (Op[0, :, 2] == 0).all()
    assert np.isneginf(m[1, :, 0]).all() and (l[1, :, 0] == 0).all()
    assert np.isfinite(m[0, :, :2]).all() and np.isfinite(m[1, :, 1:]).all()
    for r, b, s in ((0, 0, 0), (0, 2, 1), (1, 2, 1), (1, 1, 2)):
        one = O.split_partials(pool, wl.block_table, wl.row_seq[r:r + 1], wl.row_pos[r:r + 1], wl.q[r:r + 1],
                               np.array([[b]], np.int32), wl.softmax_scale, 1)
        assert np.array_equal(m[r, :, s], one[0][0, :, 0]) and np.array_equal(l[r, :, s], one[1][0, :, 0])
        assert np.array_equal(Op[r, :, s], one[2][0, :, 0])
    # the rows' masks differ on the shared block: row 1 sees token 301, row 0 does not
    assert not np.array_equal(l[0, :, 1], l[1, :, 1])
