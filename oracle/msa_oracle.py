"""Plain, slow, float64 CPU oracle for block-sparse (MSA-style) attention decode.

TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may import, call or
execute this module; only the tests, the package smoke check and the benchmark's
CPU-baseline leg do. It shares no code, tables or helpers with the HIP kernels.

What it computes is taken from three public pull-request pages of TensorRT-LLM,
cited below by title and section:

  [Rubin]  "[None][feat] Add Rubin (sm_107) MiniMax-M3.1 low-latency decode
           targets" (PR #21136)
  [GB300]  "MiniMax-M3 NVFP4 low-latency decode megakernel for modeling_v2 for
           Blackwell" (PR #20306)
  [P128]   "[None][perf] MiniMax-M3: native P128 draft KV view for the NVFP4
           hybrid cache" (PR #19731)

The pages give contracts, not formulas. Where they are silent this oracle takes
the plainest reading and says so ("reading:" in the docstrings); every reading is
listed in the design notes. Each function is the definition written out in
numpy float64, in the order the method runs it:

  kv_append      quantise new K/V/index-K into their 128-token page slots
  index_keys     exact value of a page's index keys (E4M3 or NVFP4)
  index_score    per-token index score, max-pooled into 128-token blocks (one
                 table per row, or one per KV head over its share of index heads)
  select_topk    top-k blocks, ties to the smaller block, ascending, -1 padded
  split_partials split-KV online-softmax partials (m, l, O) per split
  union_partials the same partials for groups of rows decoded over the union
                 of their tables (query pairing)
  combine        fixed-order log-sum-exp merge with one divide per output
  attend         the whole attention for a row as one softmax (definition)

Floating-point decisions that produce integers (quantised codes) are taken in
fp32, the precision the kernels use: each fp32 operation is computed in fp64
and rounded once to fp32, which equals the correctly rounded fp32 result
because 53 >= 2*24 + 2 (Figueroa, "When is double rounding innocuous?",
SIGNUM Newsletter 1995).
"""
from __future__ import annotations

import numpy as np

PAGE = 128          # tokens per page: [P128] Description ("native P128")
GROUP = 16          # NVFP4: one e4m3 scale per 16 contiguous elements (reading)
HEADS_PER_KV = 16   # [Rubin] Description: "16 query heads per KV head"
FMT_FP8 = 1
FMT_NVFP4 = 2
IDX_E4M3 = 1        # index-key formats
IDX_NVFP4 = 2


# --------------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------------
def e4m3_table() -> np.ndarray:
    """Value of every 8-bit E4M3 code, float64 [256].

    Reading: the pages say only "E4M3" ([Rubin] commit adding the NVFP4 index-K
    mirror) and "saturating FP8 casts" ([Rubin] Description, shared changes). We
    take OCP E4M3FN: sign bit 7, exponent bits 6..3 with bias 7, mantissa bits
    2..0; exponent 0 is subnormal (m * 2^-9); 0x7F/0xFF are NaN; no infinities;
    largest finite magnitude 448.
    """
    t = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        m = c & 0x7
        if e == 0xF and m == 0x7:
            t[c] = np.nan
        elif e == 0:
            t[c] = s * m * 2.0 ** -9
        else:
            t[c] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


def e2m1_table() -> np.ndarray:
    """Value of every 4-bit E2M1 code, float64 [16].

    Reading: NVFP4 element format E2M1 (sign bit 3, exponent bits 2..1 with bias 1,
    mantissa bit 0; exponent 0 is subnormal m * 0.5). Magnitudes
    {0, 0.5, 1, 1.5, 2, 3, 4, 6}.
    """
    t = np.empty(16, dtype=np.float64)
    for c in range(16):
        s = -1.0 if c & 0x8 else 1.0
        e = (c >> 1) & 0x3
        m = c & 0x1
        t[c] = s * (m * 0.5 if e == 0 else (1.0 + m / 2.0) * 2.0 ** (e - 1))
    return t


E4M3 = e4m3_table()
E2M1 = e2m1_table()
E4M3_MAX = 448.0
E2M1_MAX = 6.0


def _encode_to_grid(x: np.ndarray, grid: np.ndarray, max_code: int) -> np.ndarray:
    """Round |x| to the nearest value of an ascending non-negative grid whose index
    is the code; ties go to the even code; |x| >= grid[max_code] saturates.

    Returns unsigned magnitude codes. The codes of both formats are monotonic in
    magnitude, and adjacent codes alternate mantissa parity, so "even code" is
    IEEE round-half-to-even.
    """
    a = np.abs(np.asarray(x, dtype=np.float64))
    hi = np.searchsorted(grid, a, side="left")          # grid[hi-1] < a <= grid[hi]
    hi = np.clip(hi, 1, max_code)
    lo = hi - 1
    d_lo = a - grid[lo]
    d_hi = grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a >= grid[max_code], max_code, code)
    code = np.where(a == 0.0, 0, code)
    return code.astype(np.uint8)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even E4M3 encode of fp32-representable values.

    [Rubin] Description: the KV path uses "saturating FP8 casts": magnitudes at or
    above 448 become 448, never NaN. The sign bit follows the input's sign bit.
    """
    x = np.asarray(x, dtype=np.float64)
    grid = E4M3[:127]                      # codes 0x00..0x7E, ascending
    mag = _encode_to_grid(x, grid, 126)
    sign = np.signbit(x).astype(np.uint8) << 7
    return (mag | sign).astype(np.uint8)


def e2m1_encode(x: np.ndarray) -> np.ndarray:
    """Saturating round-to-nearest-even E2M1 encode (codes 0..15, sign bit 3)."""
    x = np.asarray(x, dtype=np.float64)
    grid = E2M1[:8]
    mag = _encode_to_grid(x, grid, 7)
    sign = np.signbit(x).astype(np.uint8) << 3
    return (mag | sign).astype(np.uint8)


def f32(x):
    """Round float64 values to the nearest fp32 (ties to even), returned as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------------
# Token encoders (the arithmetic of the KV append)
# --------------------------------------------------------------------------------
def nvfp4_encode(x: np.ndarray, tensor_scale: float):
    """NVFP4-encode vectors along the last axis (length a multiple of 16).

    Reading (the pages name the NVFP4 KV pool but not its recipe): per group of 16
    contiguous elements, amax = max|x|; y = fl32(amax / fl32(6 * t));
    scale code sc = E4M3(y); if the decoded scale is 0 every code is +0; else
    d = fl32(dec(sc) * t) and each element is E2M1(fl32(x / d)). t is the fp32
    tensor scale. Returns (nibble codes uint8 [..., n], scale codes uint8 [..., n/16]).
    """
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (n // GROUP, GROUP))
    t = f32(tensor_scale)
    amax = np.abs(g).max(axis=-1)
    y = f32(amax / f32(6.0 * t))
    sc = e4m3_encode(y)
    dec = E4M3[sc]
    d = f32(dec * t)
    safe_d = np.where(dec == 0.0, 1.0, d)
    q = f32(g / safe_d[..., None])
    codes = e2m1_encode(q)
    codes = np.where((dec == 0.0)[..., None], 0, codes).astype(np.uint8)
    return codes.reshape(x.shape), sc


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Pack 4-bit codes pairwise: byte j = code[2j] | code[2j+1] << 4 (reading:
    low nibble holds the even element)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def fp8_kv_encode(x: np.ndarray, page_scale: float) -> np.ndarray:
    """FP8 KV element: E4M3(fl32(x / s)) with s the fp32 scale of the page
    (reading: one fp32 scale per page for K and one for V, all heads)."""
    return e4m3_encode(f32(np.asarray(x, dtype=np.float64) / f32(page_scale)))


# --------------------------------------------------------------------------------
# The paged pool (numpy mirror of the device layout)
# --------------------------------------------------------------------------------
def new_pool(fmt: int, num_pages: int, num_kv_heads: int, head_dim: int = 128,
             index_dim: int = 64, k_tensor_scale: float = 1.0,
             v_tensor_scale: float = 1.0, k_page_scale=None, v_page_scale=None,
             index_fmt: int = IDX_E4M3, index_tensor_scale: float = 1.0) -> dict:
    """A zero-filled pool. Layout per page, head-major inside the page
    ([Rubin] commit messages name the HND storage of the main KV pool):

      NVFP4: codes u8 [pages][Hkv][128][D/2], scales u8 (e4m3) [pages][Hkv][128][D/16]
      FP8:   codes u8 [pages][Hkv][128][D],   scales fp32 [pages]
      index-K, E4M3:  u8 [pages][128][index_dim], one unscaled key per token
      index-K, NVFP4: token p of a page = 16 t + n (t = p // 16, n = p % 16), key
                      group g = 16 elements: codes u8 [pages][g 4][n 16][t 8][8],
                      scales u8 (e4m3) [pages][g 4][n 16][t 8], one fp32 tensor scale
                      (group-major so that one group of 8 token rows is contiguous)
    """
    p = {"fmt": fmt, "num_pages": num_pages, "Hkv": num_kv_heads, "D": head_dim,
         "di": index_dim, "index_fmt": index_fmt}
    if index_fmt == IDX_E4M3:
        p["index_k"] = np.zeros((num_pages, PAGE, index_dim), np.uint8)
    elif index_fmt == IDX_NVFP4:
        G = index_dim // GROUP
        p["index_k"] = np.zeros((num_pages, G, 16, PAGE // 16, GROUP // 2), np.uint8)
        p["index_scales"] = np.zeros((num_pages, G, 16, PAGE // 16), np.uint8)
        p["index_tensor_scale"] = float(np.float32(index_tensor_scale))
    else:
        raise ValueError("unknown index-key format")
    if fmt == FMT_NVFP4:
        for kv in ("k", "v"):
            p[kv + "_codes"] = np.zeros((num_pages, num_kv_heads, PAGE, head_dim // 2), np.uint8)
            p[kv + "_scales"] = np.zeros((num_pages, num_kv_heads, PAGE, head_dim // GROUP), np.uint8)
        p["k_tensor_scale"] = float(np.float32(k_tensor_scale))
        p["v_tensor_scale"] = float(np.float32(v_tensor_scale))
    elif fmt == FMT_FP8:
        for kv, ps in (("k", k_page_scale), ("v", v_page_scale)):
            p[kv + "_codes"] = np.zeros((num_pages, num_kv_heads, PAGE, head_dim), np.uint8)
            p[kv + "_scales"] = (np.ones(num_pages, np.float32) if ps is None
                                 else np.asarray(ps, np.float32).copy())
    else:
        raise ValueError("unknown KV format")
    return p


def kv_append(pool: dict, slot: np.ndarray, k_new=None, v_new=None, idx_new=None) -> None:
    """Quantise new tokens into their page slots (in place).

    [GB300] "Step-loop runtime hooks" lists "a hook for the KV update"; [Rubin]
    Description lists "saturating FP8 casts". slot = page * 128 + offset; a
    negative slot is skipped and nothing is written (reading, after the [Rubin]
    guard-page item: writes through unallocated entries must not land anywhere).
    k_new / v_new: bf16 bit patterns [n][Hkv][D]; idx_new: bf16 bits [n][index_dim].
    Any of the three may be None to skip that part.
    """
    slot = np.asarray(slot, dtype=np.int64)
    keep = np.nonzero(slot >= 0)[0]
    page, off = slot[keep] // PAGE, slot[keep] % PAGE
    if idx_new is not None:
        xi = bf16_bits_to_f64(np.asarray(idx_new)[keep])         # [n][index_dim]
        if pool["index_fmt"] == IDX_NVFP4:
            # reading: [Rubin] Description lists NVFP4 index-K pages
            # (indexer_kv_dtype='nvfp4') without a recipe; they take the KV's NVFP4
            # recipe, encoded from the bf16 key with the pool's index tensor scale
            codes, sc = nvfp4_encode(xi, pool["index_tensor_scale"])
            packed = pack_nibbles(codes)                            # [n][index_dim / 2]
            for g in range(sc.shape[1]):
                pool["index_k"][page, g, off % 16, off // 16] = packed[:, 8 * g:8 * g + 8]
                pool["index_scales"][page, g, off % 16, off // 16] = sc[:, g]
        else:
            pool["index_k"][page, off] = e4m3_encode(xi)
    for kv, src in (("k", k_new), ("v", v_new)):
        if src is None:
            continue
        x = bf16_bits_to_f64(np.asarray(src)[keep])          # [n][Hkv][D]
        if pool["fmt"] == FMT_NVFP4:
            codes, sc = nvfp4_encode(x, pool[kv + "_tensor_scale"])
            pool[kv + "_codes"][page, :, off] = pack_nibbles(codes)
            pool[kv + "_scales"][page, :, off] = sc
        else:
            s = pool[kv + "_scales"][page].astype(np.float64)[:, None, None]
            pool[kv + "_codes"][page, :, off] = e4m3_encode(f32(x / f32(s)))


def index_keys(pool: dict, page: int, n: int) -> np.ndarray:
    """Exact value of the first n index keys of a page, float64 [n][index_dim]."""
    if pool["index_fmt"] == IDX_NVFP4:
        p = np.arange(n)
        codes = pool["index_k"][page][:, p % 16, p // 16]                  # [G][n][8]
        vals = E2M1[unpack_nibbles(codes)]                                 # [G][n][16]
        sc = E4M3[pool["index_scales"][page][:, p % 16, p // 16]]          # [G][n]
        keys = vals * sc[:, :, None] * pool["index_tensor_scale"]
        return np.concatenate(list(keys), axis=1)                          # [n][index_dim]
    return E4M3[pool["index_k"][page, :n]]


def dequant_page(pool: dict, page: int, head: int, kv: str) -> np.ndarray:
    """Exact value of one page of K or V for one KV head, float64 [128][D]."""
    codes = pool[kv + "_codes"][page, head]
    if pool["fmt"] == FMT_NVFP4:
        vals = E2M1[unpack_nibbles(codes)]                               # [128][D]
        sc = E4M3[pool[kv + "_scales"][page, head]]                       # [128][D/16]
        return vals * np.repeat(sc, GROUP, axis=1) * pool[kv + "_tensor_scale"]
    return E4M3[codes] * float(pool[kv + "_scales"][page])


# --------------------------------------------------------------------------------
# Step a2: index score and block max-pool
# --------------------------------------------------------------------------------
def index_score(pool: dict, block_table, row_seq, row_pos, q_idx_bits, w,
                max_blocks: int, tables: int = 1) -> np.ndarray:
    """Block scores S [rows][max_blocks] (float64), or S [rows][tables][max_blocks]
    when tables > 1.

    The pages name the scorer ([GB300] "The TP4 decode target": "an index scorer
    that prefetches older index-K pages"; [Rubin] commits: a CuTe DSL scorer and
    an indexer proxy max-score pass) but not its formula. Reading: for a query
    row r and a visible token p (p <= row_pos[r]) with index key k_p (E4M3, or
    NVFP4 decoded exactly),
        s_p = sum_h w[r,h] * max(0, q_idx[r,h] . k_p)
    and the block score is the max of s_p over the block's visible tokens.
    Blocks past the row's last visible block are -inf; so is nothing else.

    Per-KV-head tables ([Rubin] commits: the indexer hands "KV-head-reduced
    scores" to its selector, and the prefill tile select runs one CTA per KV head
    and writes a head-major table). Reading: with `tables` = T tables per row,
    the Hi index heads are split into T equal consecutive groups and table t
    sums only over its group, h in [t*Hi/T, (t+1)*Hi/T); T = 1 is the shared
    score above.
    """
    rows = len(row_pos)
    Hi = np.asarray(w).shape[1]
    assert tables >= 1 and Hi % tables == 0, "index heads must split evenly into the tables"
    per = Hi // tables
    S = np.full((rows, tables, max_blocks), -np.inf)
    for r in range(rows):
        seq, pos = int(row_seq[r]), int(row_pos[r])
        q = bf16_bits_to_f64(q_idx_bits[r])                     # [Hi][di]
        wr = np.asarray(w[r], dtype=np.float64)                 # [Hi]
        for b in range(pos // PAGE + 1):
            page = int(block_table[seq][b])
            n_vis = min(PAGE, pos - PAGE * b + 1)
            K = index_keys(pool, page, n_vis)                   # [n_vis][di]
            dots = K @ q.T                                       # [n_vis][Hi]
            terms = np.maximum(dots, 0.0) * wr                   # [n_vis][Hi]
            for t in range(tables):
                S[r, t, b] = terms[:, t * per:(t + 1) * per].sum(axis=1).max()
    return S[:, 0] if tables == 1 else S


# --------------------------------------------------------------------------------
# Step a3: top-k block selection
# --------------------------------------------------------------------------------
def select_topk(S: np.ndarray, row_pos, k: int, n_init: int = 0, n_local: int = 1) -> np.ndarray:
    """Selection table sel [rows][k] int32, ascending logical block ids, -1 padded.

    [Rubin] commits (NVFP4 index-K mirror): the table is "ascending, -1-padded";
    (prefill tile select): the same table "including tie order and init / local
    forcing". [GB300] "The TP4 decode target", Numerics: score ties go to the
    smaller block, at any tie width. [GB300] "Step-loop runtime hooks": an
    identity block table for short sequences.
    Reading: with nb = row_pos // 128 + 1 visible blocks, a row with nb <= k
    selects 0..nb-1. Otherwise the first n_init and last n_local blocks are
    forced and count inside k; the other k - |forced| slots go to the best
    remaining blocks by (higher score, then smaller index).
    Per-KV-head scores S [rows][T][max_blocks] give one table per (row, KV head),
    sel [rows][T][k], each selected by the same rule from its own scores.
    """
    if S.ndim == 3:
        rows, T = S.shape[:2]
        flat = select_topk(S.reshape(rows * T, -1), np.repeat(np.asarray(row_pos), T), k, n_init, n_local)
        return flat.reshape(rows, T, k)
    rows = S.shape[0]
    sel = np.full((rows, k), -1, dtype=np.int32)
    for r in range(rows):
        nb = int(row_pos[r]) // PAGE + 1
        if nb <= k:
            sel[r, :nb] = np.arange(nb)
            continue
        forced = set(range(min(n_init, nb))) | set(range(max(nb - n_local, 0), nb))
        rest = [b for b in range(nb) if b not in forced]
        rest.sort(key=lambda b: (-S[r, b], b))
        chosen = sorted(forced | set(rest[: k - len(forced)]))
        sel[r, : len(chosen)] = chosen
    return sel


# --------------------------------------------------------------------------------
# Steps a4 + a5: sparse GQA attention over the selected pages
# --------------------------------------------------------------------------------
def _row_tokens(sel_entries, pos: int):
    """Absolute positions of the visible tokens of the given selected blocks."""
    toks = []
    for b in sel_entries:
        if b < 0:
            continue
        hi = min(PAGE * (int(b) + 1), pos + 1)
        toks.extend(range(PAGE * int(b), hi))
    return np.asarray(toks, dtype=np.int64)


def _gather_kv(pool, block_table, seq, tokens, head):
    K = np.empty((len(tokens), pool["D"]))
    V = np.empty((len(tokens), pool["D"]))
    cache = {}
    for i, t in enumerate(tokens):
        b, off = divmod(int(t), PAGE)
        page = int(block_table[seq][b])
        if page not in cache:
            cache[page] = (dequant_page(pool, page, head, "k"), dequant_page(pool, page, head, "v"))
        K[i] = cache[page][0][off]
        V[i] = cache[page][1][off]
    return K, V


LOG2E = 1.0 / np.log(2.0)


def split_partials(pool: dict, block_table, row_seq, row_pos, q_bits, sel, softmax_scale: float,
                   num_splits: int):
    """Split-KV partials in base-2 units: m = max_p x_p, l = sum_p 2^(x_p - m),
    O = sum_p 2^(x_p - m) V_p, where x_p = softmax_scale * (q . K_p) * log2(e).

    [Rubin] commits (CuTe sparse decode): work is split per "(top-k split, KV
    head, query row)". Reading: split s of S takes the selection entries
    [floor(s*k/S), floor((s+1)*k/S)); a split with no visible token has
    m = -inf, l = 0, O = 0. Returns m, l [rows][Hq][S] and O [rows][Hq][S][D].
    sel is [rows][k] (one table per row) or [rows][Hkv][k] (KV head g reads
    table g).
    """
    rows, k = sel.shape[0], sel.shape[-1]
    Hq = q_bits.shape[1]
    D = pool["D"]
    m = np.full((rows, Hq, num_splits), -np.inf)
    l = np.zeros((rows, Hq, num_splits))
    O = np.zeros((rows, Hq, num_splits, D))
    for r in range(rows):
        seq, pos = int(row_seq[r]), int(row_pos[r])
        q = bf16_bits_to_f64(q_bits[r])                           # [Hq][D]
        for s in range(num_splits):
            lo, hi = (s * k) // num_splits, ((s + 1) * k) // num_splits
            for g in range(pool["Hkv"]):
                table = sel[r] if sel.ndim == 2 else sel[r, g]
                toks = _row_tokens(table[lo:hi], pos)
                if len(toks) == 0:
                    continue
                K, V = _gather_kv(pool, block_table, seq, toks, g)
                for h in range(g * HEADS_PER_KV, (g + 1) * HEADS_PER_KV):
                    x = softmax_scale * (K @ q[h]) * LOG2E
                    mx = x.max()
                    p = np.exp2(x - mx)
                    m[r, h, s], l[r, h, s], O[r, h, s] = mx, p.sum(), p @ V
    return m, l, O


def union_blocks(tables) -> list:
    """The union of a row group's selection tables: every selected block once, in
    the order of its first pick, rows in order and each table in order."""
    seen, out = set(), []
    for table in tables:
        for b in table:
            b = int(b)
            if b >= 0 and b not in seen:
                seen.add(b)
                out.append(b)
    return out


def union_partials(pool: dict, block_table, row_seq, row_pos, q_bits, sel, softmax_scale: float,
                   num_splits: int, group_rows):
    """Split partials (m, l, O in base-2 units, as split_partials) of rows decoded in
    groups over the union of their tables.

    [Rubin] commit messages: the tuned NVFP4 sparse decode at a verify length of 4
    query rows per request includes "query pairing". Reading: the rows of one
    request (a group: rows group_rows[i] .. group_rows[i+1]-1) read each page of the
    union of their selections once; each row keeps its own softmax over its own
    selected blocks and its own visible tokens. Split s of S takes the union
    entries [floor(s*N/S), floor((s+1)*N/S)) of the N entries (union_blocks order);
    row r's partial of split s covers the blocks of that range that r selected (none:
    m = -inf, l = 0, O = 0). KV head g reads table g when sel is [rows][Hkv][k].
    Returns m, l [rows][Hq][S] and O [rows][Hq][S][D]; rows in no group stay empty.
    """
    rows = sel.shape[0]
    Hq = q_bits.shape[1]
    D = pool["D"]
    m = np.full((rows, Hq, num_splits), -np.inf)
    l = np.zeros((rows, Hq, num_splits))
    O = np.zeros((rows, Hq, num_splits, D))
    for gi in range(len(group_rows) - 1):
        r0, r1 = int(group_rows[gi]), int(group_rows[gi + 1])
        for g in range(pool["Hkv"]):
            tables = [sel[r] if sel.ndim == 2 else sel[r, g] for r in range(r0, r1)]
            U = union_blocks(tables)
            N = len(U)
            for s in range(num_splits):
                part = U[(s * N) // num_splits:((s + 1) * N) // num_splits]
                for r in range(r0, r1):
                    mine = set(int(b) for b in tables[r - r0])
                    toks = _row_tokens([b for b in part if b in mine], int(row_pos[r]))
                    if len(toks) == 0:
                        continue
                    K, V = _gather_kv(pool, block_table, int(row_seq[r]), toks, g)
                    q = bf16_bits_to_f64(q_bits[r])
                    for h in range(g * HEADS_PER_KV, (g + 1) * HEADS_PER_KV):
                        x = softmax_scale * (K @ q[h]) * LOG2E
                        mx = x.max()
                        p = np.exp2(x - mx)
                        m[r, h, s], l[r, h, s], O[r, h, s] = mx, p.sum(), p @ V
    return m, l, O


def combine(m: np.ndarray, l: np.ndarray, O: np.ndarray) -> np.ndarray:
    """Merge split partials: M = max_s m_s, out = (sum_s 2^(m_s-M) O_s) /
    (sum_s 2^(m_s-M) l_s), summed over s in ascending order with one divide.

    [Rubin] "Items and numerics", row LC_ONEDIV: the split-K merge "divides once
    per output (fixed order, no atomics)".
    """
    M = m.max(axis=-1, keepdims=True)
    a = np.where(np.isneginf(m), 0.0, np.exp2(m - np.where(np.isneginf(M), 0.0, M)))
    num = np.zeros(O.shape[:-2] + O.shape[-1:])
    den = np.zeros(m.shape[:-1])
    for s in range(m.shape[-1]):
        num = num + a[..., s, None] * O[..., s, :]
        den = den + a[..., s] * l[..., s]
    return num / den[..., None]


def attend(pool: dict, block_table, row_seq, row_pos, q_bits, sel, softmax_scale: float) -> np.ndarray:
    """Attention of each query row over the visible tokens of its selected
    blocks, one softmax per query head, float64 [rows][Hq][D].

    Query head h reads KV head h // 16 ([Rubin] Description: 16 query heads per
    KV head; reading: contiguous grouping). logit = softmax_scale * q . K_p.
    sel is [rows][k] (one table per row) or [rows][Hkv][k] (KV head g attends
    the blocks of table g).
    """
    rows = sel.shape[0]
    Hq = q_bits.shape[1]
    out = np.zeros((rows, Hq, pool["D"]))
    for r in range(rows):
        seq, pos = int(row_seq[r]), int(row_pos[r])
        q = bf16_bits_to_f64(q_bits[r])
        for g in range(pool["Hkv"]):
            toks = _row_tokens(sel[r] if sel.ndim == 2 else sel[r, g], pos)
            K, V = _gather_kv(pool, block_table, seq, toks, g)
            for h in range(g * HEADS_PER_KV, (g + 1) * HEADS_PER_KV):
                x = softmax_scale * (K @ q[h])
                p = np.exp(x - x.max())
                out[r, h] = (p @ V) / p.sum()
    return out


def decode_step(pool: dict, block_table, row_seq, row_pos, slot, k_new, v_new, idx_new,
                q_idx_bits, w, q_bits, k: int, softmax_scale: float, max_blocks: int,
                n_init: int = 0, n_local: int = 1, tables: int = 1):
    """One decode step in the method's order: append, score, select, attend.
    Mutates `pool` (the append). Returns (S, sel, out); tables = Hkv selects per
    KV head."""
    kv_append(pool, slot, k_new, v_new, idx_new)
    S = index_score(pool, block_table, row_seq, row_pos, q_idx_bits, w, max_blocks, tables)
    sel = select_topk(S, row_pos, k, n_init, n_local)
    out = attend(pool, block_table, row_seq, row_pos, q_bits, sel, softmax_scale)
    return S, sel, out
