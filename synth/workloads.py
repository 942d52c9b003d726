"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic).

Both the HIP path and the CPU oracle consume these arrays; neither side's
computation lives here. Everything is drawn from numpy's PCG64 generator
(`numpy.random.default_rng`) with a fixed seed and a fixed draw order, so a
workload is reproducible bit for bit on any host.

Values are stored the way the library's boundary takes them: bf16 tensors as
uint16 bit patterns, fp32 as float32, metadata as int32/int64.

Input recipe (per workload):
  * cached context lengths L_s, rows per request R, appended tokens per request A
    (appended token j of request s sits at position L_s + j; query row j of the
    request is at the same position and attends positions [0, L_s + j]; a request
    without appended tokens has one row at L_s - 1);
  * a global random permutation of physical page ids, carved into per-request
    page lists in request order (pages of different requests interleave in the
    pool);
  * K/V source values ~ N(0, 1) per (token, KV head, dim), rounded to bf16;
  * Q ~ N(0, 1) bf16 [rows][Hq][128]; index queries ~ N(0, 1) bf16
    [rows][Hi][64]; index head weights ~ U(0, 1) fp32 [rows][Hi];
  * index-K source ~ N(0, 1) bf16 per token (or the tie construction below);
  * FP8 pools: one fp32 scale per (page, K) and per (page, V), set to
    amax(|source values the page will hold|) / 448;
  * NVFP4 pools: one fp32 tensor scale for K and one for V, set to
    amax(|all source values|) / (6 * 448).
The scales are the caller's calibration inputs to the append; the library only
reads them.

Tie construction (long-context tie workload): a seeded set of blocks (never the
last) each holds one token whose index key is 2 * sign(sum_h w_h q_h) of that
request's only row (an exactly representable E4M3 vector, so every such block
scores the same and above all others); every other index key is 0.05 * N(0, 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

PAGE = 128
FMT_FP8 = 1
FMT_NVFP4 = 2
IDX_E4M3 = 1
IDX_NVFP4 = 2


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest even) and return the bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = u >> np.uint32(16)
    lsb &= np.uint32(1)
    lsb += np.uint32(0x7FFF)
    lsb += u
    lsb >>= np.uint32(16)
    return lsb.astype(np.uint16)


def bf16_absmax(bits: np.ndarray) -> float:
    """Largest magnitude among bf16 bit patterns (finite values)."""
    m = np.uint16(np.max(np.asarray(bits, dtype=np.uint16) & np.uint16(0x7FFF)))
    return float(bf16_bits_to_f32(np.array([m], np.uint16))[0])


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    name: str
    seed: int
    fmt: int
    num_kv_heads: int
    k: int
    ctx_lens: np.ndarray          # int64 [B] cached tokens before the step
    n_append: int                 # appended tokens per request this step
    rows_per_req: int
    head_dim: int = 128
    index_heads: int = 4
    index_dim: int = 64
    n_init: int = 0
    n_local: int = 1
    spare_pages: int = 3
    index_fmt: int = IDX_E4M3
    # filled by build()
    num_pages: int = 0
    max_blocks: int = 0
    block_table: np.ndarray = field(default=None, repr=False)   # int32 [B][max_blocks]
    row_seq: np.ndarray = field(default=None, repr=False)       # int32 [rows]
    row_pos: np.ndarray = field(default=None, repr=False)       # int32 [rows]
    k_src: list = field(default=None, repr=False)               # per request bf16 bits [T_s][Hkv][D]
    v_src: list = field(default=None, repr=False)
    idx_src: list = field(default=None, repr=False)             # per request bf16 bits [T_s][di]
    q: np.ndarray = field(default=None, repr=False)             # bf16 bits [rows][Hq][D]
    q_idx: np.ndarray = field(default=None, repr=False)         # bf16 bits [rows][Hi][di]
    w: np.ndarray = field(default=None, repr=False)             # f32 [rows][Hi]
    k_tensor_scale: float = 1.0
    v_tensor_scale: float = 1.0
    index_tensor_scale: float = 1.0   # NVFP4 index keys
    k_page_scale: np.ndarray = field(default=None, repr=False)  # f32 [pages] (FP8)
    v_page_scale: np.ndarray = field(default=None, repr=False)
    tie_blocks: list = field(default=None, repr=False)

    @property
    def num_heads(self) -> int:
        return 16 * self.num_kv_heads

    @property
    def num_rows(self) -> int:
        return len(self.row_pos)

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.head_dim)))

    def total_len(self, s: int) -> int:
        return int(self.ctx_lens[s]) + self.n_append

    # ---- slots -------------------------------------------------------------
    def slots(self, s: int, positions: np.ndarray) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        pages = self.block_table[s][positions // PAGE].astype(np.int64)
        return pages * PAGE + positions % PAGE

    def prefill_tokens(self):
        """(slot int64 [n], k bits [n][Hkv][D], v bits, idx bits [n][di]) for all
        cached tokens of every request, in request order."""
        sl, ks, vs, ids = [], [], [], []
        for s in range(len(self.ctx_lens)):
            L = int(self.ctx_lens[s])
            sl.append(self.slots(s, np.arange(L)))
            ks.append(self.k_src[s][:L]); vs.append(self.v_src[s][:L]); ids.append(self.idx_src[s][:L])
        return (np.concatenate(sl), np.concatenate(ks), np.concatenate(vs), np.concatenate(ids))

    def step_tokens(self):
        """The tokens appended by the step: (slot, k, v, idx) in request order."""
        if self.n_append == 0:
            e = np.zeros(0, np.int64)
            return (e, np.zeros((0, self.num_kv_heads, self.head_dim), np.uint16),
                    np.zeros((0, self.num_kv_heads, self.head_dim), np.uint16),
                    np.zeros((0, self.index_dim), np.uint16))
        sl, ks, vs, ids = [], [], [], []
        for s in range(len(self.ctx_lens)):
            L = int(self.ctx_lens[s])
            pos = np.arange(L, L + self.n_append)
            sl.append(self.slots(s, pos))
            ks.append(self.k_src[s][L:]); vs.append(self.v_src[s][L:]); ids.append(self.idx_src[s][L:])
        return (np.concatenate(sl), np.concatenate(ks), np.concatenate(vs), np.concatenate(ids))

    def prefill_slices(self, s: int, positions: np.ndarray):
        """Source data of request s at the given positions (for sampled checks)."""
        positions = np.asarray(positions, dtype=np.int64)
        return (self.slots(s, positions), self.k_src[s][positions], self.v_src[s][positions],
                self.idx_src[s][positions])


def build(wl: Workload) -> Workload:
    """Draw every array of the workload (fixed order: page permutation, K/V
    source, queries, index keys)."""
    rng = np.random.default_rng(wl.seed)
    B = len(wl.ctx_lens)
    Hkv, D, Hi, di = wl.num_kv_heads, wl.head_dim, wl.index_heads, wl.index_dim
    totals = [wl.total_len(s) for s in range(B)]
    pages_per = [(t + PAGE - 1) // PAGE for t in totals]
    wl.num_pages = int(sum(pages_per)) + wl.spare_pages
    wl.max_blocks = int(max(pages_per))
    perm = rng.permutation(wl.num_pages).astype(np.int32)
    wl.block_table = np.full((B, wl.max_blocks), -1, dtype=np.int32)
    at = 0
    for s in range(B):
        wl.block_table[s, : pages_per[s]] = perm[at: at + pages_per[s]]
        at += pages_per[s]
    # rows
    rs, rp = [], []
    for s in range(B):
        L = int(wl.ctx_lens[s])
        if wl.n_append == 0:
            assert wl.rows_per_req == 1
            rs.append(s); rp.append(L - 1)
        else:
            assert wl.rows_per_req == wl.n_append
            for j in range(wl.n_append):
                rs.append(s); rp.append(L + j)
    wl.row_seq = np.asarray(rs, dtype=np.int32)
    wl.row_pos = np.asarray(rp, dtype=np.int32)
    # K / V source, one generator stream per request so a request can be rebuilt alone
    wl.k_src, wl.v_src = [], []
    for s in range(B):
        r2 = np.random.default_rng([wl.seed, 1, s])
        wl.k_src.append(to_bf16_bits(r2.standard_normal((totals[s], Hkv, D), dtype=np.float32)))
        wl.v_src.append(to_bf16_bits(r2.standard_normal((totals[s], Hkv, D), dtype=np.float32)))
    rows = len(rp)
    wl.q = to_bf16_bits(rng.standard_normal((rows, wl.num_heads, D), dtype=np.float32))
    wl.q_idx = to_bf16_bits(rng.standard_normal((rows, Hi, di), dtype=np.float32))
    wl.w = rng.random((rows, Hi), dtype=np.float32)
    wl.idx_src = []
    for s in range(B):
        r3 = np.random.default_rng([wl.seed, 2, s])
        wl.idx_src.append(to_bf16_bits(r3.standard_normal((totals[s], di), dtype=np.float32)))
    # scales (calibration inputs)
    if wl.index_fmt == IDX_NVFP4:
        ia = max(bf16_absmax(x) for x in wl.idx_src)
        wl.index_tensor_scale = float(np.float32(ia / (6.0 * 448.0)))
    if wl.fmt == FMT_NVFP4:
        ka = max(bf16_absmax(x) for x in wl.k_src)
        va = max(bf16_absmax(x) for x in wl.v_src)
        wl.k_tensor_scale = float(np.float32(ka / (6.0 * 448.0)))
        wl.v_tensor_scale = float(np.float32(va / (6.0 * 448.0)))
    else:
        kps = np.ones(wl.num_pages, np.float32)
        vps = np.ones(wl.num_pages, np.float32)
        for s in range(B):
            for b in range(pages_per[s]):
                lo, hi = b * PAGE, min((b + 1) * PAGE, totals[s])
                page = wl.block_table[s, b]
                kps[page] = np.float32(bf16_absmax(wl.k_src[s][lo:hi]) / 448.0)
                vps[page] = np.float32(bf16_absmax(wl.v_src[s][lo:hi]) / 448.0)
        wl.k_page_scale, wl.v_page_scale = kps, vps
    return wl


def inject_ties(wl: Workload, n_tied: int, seed_tag: int = 3) -> Workload:
    """Rewrite the index keys so that n_tied blocks (never a request's last block)
    share exactly the same block score, above every other block's."""
    assert wl.n_append == 0 and wl.rows_per_req == 1
    wl.tie_blocks = []
    for s in range(len(wl.ctx_lens)):
        r4 = np.random.default_rng([wl.seed, seed_tag, s])
        L = wl.total_len(s)
        nb = (L + PAGE - 1) // PAGE
        qsum = (wl.w[s][:, None].astype(np.float64) *
                bf16_bits_to_f32(wl.q_idx[s]).astype(np.float64)).sum(axis=0)
        kstar = np.where(qsum >= 0, 2.0, -2.0).astype(np.float32)
        small = 0.05 * r4.standard_normal((L, wl.index_dim), dtype=np.float32)
        idx = small.astype(np.float32)
        blocks = np.sort(r4.choice(nb - 1, size=n_tied, replace=False))
        offs = r4.integers(0, PAGE, size=n_tied)
        idx[blocks * PAGE + offs] = kstar
        wl.idx_src[s] = to_bf16_bits(idx)
        wl.tie_blocks.append(blocks)
    return wl


def verify_tables(wl: Workload, overlap: float, seed_tag: int = 5) -> np.ndarray:
    """Seeded selection tables with the structure of a top-k selection ([rows][k], each
    row's visible blocks in strictly ascending order, its last visible block always
    present, -1 padding only when the row sees fewer than k blocks), where the rows of
    one request share a fraction `overlap` of their picks: every request draws k - 1
    blocks that all its rows see, and each row keeps each of them with probability
    `overlap` (else it draws another block it sees). overlap = 1 gives every row of a
    request the same earlier blocks; 0 gives independent draws."""
    rng = np.random.default_rng([wl.seed, seed_tag])
    k = wl.k
    sel = np.full((wl.num_rows, k), -1, dtype=np.int32)
    for s in range(len(wl.ctx_lens)):
        rows = np.nonzero(wl.row_seq == s)[0]
        if len(rows) == 0:
            continue
        nb_min = int(wl.row_pos[rows].min()) // PAGE + 1
        shared = rng.choice(max(nb_min - 1, 1), size=min(k - 1, max(nb_min - 1, 0)), replace=False) \
            if nb_min > 1 else np.zeros(0, np.int64)
        for r in rows:
            nb = int(wl.row_pos[r]) // PAGE + 1
            if nb <= k:
                sel[r, :nb] = np.arange(nb)
                continue
            picks = {nb - 1}
            for b in shared:
                if len(picks) < k and rng.random() < overlap:
                    picks.add(int(b))
            while len(picks) < k:
                picks.add(int(rng.integers(0, nb - 1)))
            sel[r] = np.sort(np.fromiter(picks, dtype=np.int64))
    return sel


def keep_rows(wl: Workload, rows) -> Workload:
    """The same workload with only the given query rows (request-major order kept):
    requests then have different numbers of rows, or none."""
    import dataclasses
    rows = np.asarray(sorted(rows), dtype=np.int64)
    return dataclasses.replace(wl, row_seq=wl.row_seq[rows], row_pos=wl.row_pos[rows], q=wl.q[rows],
                               q_idx=wl.q_idx[rows], w=wl.w[rows])


# --------------------------------------------------------------------------------
# The five benchmark workloads and small parity workloads
# --------------------------------------------------------------------------------
def config(cfg: int, index_fmt: int = IDX_E4M3) -> Workload:
    """The five workloads (index keys E4M3 as specified; index_fmt=IDX_NVFP4 gives
    the same workload with NVFP4 index keys, which draws the same random numbers)."""
    seed = 1000 + cfg
    if cfg == 0:   # tiny FP8 case
        wl = Workload("tiny_fp8_b1_ctx4096", seed, FMT_FP8, 1, 8, np.array([4096]), 0, 1)
    elif cfg == 1:  # the measured workload
        wl = Workload("b8_ctx32k_nvfp4_top16", seed, FMT_NVFP4, 4, 16, np.full(8, 32768), 1, 1)
    elif cfg == 2:  # speculative verify
        r = np.random.default_rng([seed, 0])
        lens = r.integers(8192, 65536, size=40, endpoint=True)
        wl = Workload("verify_40x4_ctx8k-64k_nvfp4_top16", seed, FMT_NVFP4, 4, 16, lens, 4, 4)
    elif cfg == 3:  # long context with ties
        wl = Workload("b2_ctx256k_fp8_top32_ties", seed, FMT_FP8, 4, 32, np.full(2, 262144), 0, 1)
    elif cfg == 4:  # mixed lengths, shared interleaved pool
        r = np.random.default_rng([seed, 0])
        lens = np.clip(np.rint(r.lognormal(np.log(8192.0), 1.0, size=48)), 512, 131072).astype(np.int64)
        wl = Workload("mixed48_lognormal8k_nvfp4_top16", seed, FMT_NVFP4, 4, 16, lens, 1, 1)
    else:
        raise ValueError(cfg)
    wl.index_fmt = index_fmt
    if index_fmt == IDX_NVFP4:
        wl.name += "_idxnvfp4"
    build(wl)
    if cfg == 3:
        inject_ties(wl, 1100)
    if cfg == 4:
        dense = int(((wl.row_pos // PAGE + 1) <= wl.k).sum())
        assert dense >= 1, "mixed workload must contain at least one dense row"
    return wl


def small(fmt: int, ctx_lens, n_append: int, num_kv_heads: int = 2, k: int = 4,
          seed: int = 7, rows_per_req: int | None = None, index_fmt: int = IDX_E4M3) -> Workload:
    """A small workload for parity tests (several tiles and ragged tails)."""
    rows_per_req = rows_per_req or max(1, n_append)
    wl = Workload(f"small_{'fp8' if fmt == FMT_FP8 else 'nvfp4'}", seed, fmt, num_kv_heads, k,
                  np.asarray(ctx_lens, dtype=np.int64), n_append, rows_per_req, index_fmt=index_fmt)
    if index_fmt == IDX_NVFP4:
        wl.name += "_idxnvfp4"
    return build(wl)
