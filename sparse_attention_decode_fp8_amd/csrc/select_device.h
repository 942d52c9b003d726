// Deterministic top-k block selection for one query row, shared by msa_select_topk,
// the fused score-and-select kernel and the selecting decode:
//   block_select_row     256+ threads, radix select over LDS histograms (any length)
//   wave_select_table    one wave, threshold search over the keys it holds (<= 2048)
//   multiwave_select_*   several waves of a workgroup, two levels (the selecting decode)
//
// Contract ([Rubin] commit messages: ascending, -1-padded table with init / local
// forcing; [GB300] "The TP4 decode target", numerics: ties to the smaller block):
// rows with nb <= k select 0..nb-1; otherwise the n_init first and n_local last blocks
// are forced and the other k - n_init - n_local slots go to the best remaining blocks by
// (score desc, index asc). Every variant finds the exact want-th largest order-
// preserving key and ranks the blocks tied at it in block order, so none depends on the
// order in which atomics land.
#pragma once

#include "msa_device.h"

namespace msa {

constexpr int kSelectThreads = 256;

struct SelectSmem {
  int hist[256];
  int tmp[16];
  int digit, above;
};

// Exclusive prefix sum over a block of kThreads threads, in thread order.
template <int kThreads>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_tmp) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_tmp[wave] = x;
  __syncthreads();
  int base = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i)
    if (i < wave) base += lds_tmp[i];
  __syncthreads();
  return base + x - v;
}

// Radix select for one row: the want-th largest key by an MSB-first radix select over
// LDS histograms, then the blocks tied at it ranked by a scan in block order.
// All kThreads (>= 256, a multiple of 64) threads must call it. `srow` is the row's score array
// (index = block), `bt` the request's block-table row, `out`/`outp` the row's k-entry
// outputs (outp may be null), `keys` LDS scratch of at least nb - n_init - n_local
// entries. kCoherent: read the scores with agent-coherent loads (they were written by
// other workgroups of the same launch).
template <bool kCoherent, int kThreads = kSelectThreads>
__device__ void block_select_row(const float* srow, int nb, int k, int n_init, int n_local,
                                 const int32_t* bt, int32_t* out, int32_t* outp, uint32_t* keys,
                                 SelectSmem& sm) {
  const int tid = threadIdx.x;
  __syncthreads();                               // LDS may still be in use by a previous row
  if (nb <= k) {                                 // identity table
    for (int i = tid; i < k; i += kThreads) {
      out[i] = i < nb ? i : -1;
      if (outp) outp[i] = i < nb ? bt[i] : -1;
    }
    return;
  }
  const int lo = n_init, C = nb - n_init - n_local;   // candidates: blocks lo .. lo + C - 1
  const int want = k - n_init - n_local;
  for (int i = tid; i < n_init; i += kThreads) {
    out[i] = i;
    if (outp) outp[i] = bt[i];
  }
  for (int i = tid; i < n_local; i += kThreads) {
    out[k - n_local + i] = nb - n_local + i;
    if (outp) outp[k - n_local + i] = bt[nb - n_local + i];
  }
  if (want == 0) return;
  for (int c = tid; c < C; c += kThreads) {
    float v;
    if constexpr (kCoherent)
      v = __hip_atomic_load(srow + lo + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      v = srow[lo + c];
    keys[c] = float_key(v);
  }

  uint32_t prefix = 0, pmask = 0;
  int remaining = want;                          // rank still to find among matching keys
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sm.hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < C; c += kThreads) {
      const uint32_t kk = keys[c];
      const bool match = (kk & pmask) == prefix;
      const uint32_t dg = (kk >> shift) & 255u;
      // Lanes that all add to the same bin (ties, or a shared digit) add once, by
      // their first lane: equal keys would otherwise serialise on one LDS address.
      const uint64_t mm = __ballot(match);
      if (mm == 0) continue;
      const int first = __ffsll(static_cast<unsigned long long>(mm)) - 1;
      const uint32_t d0 = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(dg), first));
      const uint64_t same = __ballot(match && dg == d0);
      if (same == mm) {
        if ((tid & 63) == first) atomicAdd(&sm.hist[d0], __popcll(mm));
      } else if (match) {
        atomicAdd(&sm.hist[dg], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {                              // wave 0 finds the digit holding the rank
      // lane L owns digits 255-4L .. 252-4L (descending); suffix sums from the top
      int c4[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c4[i] = sm.hist[255 - 4 * tid - i]; s += c4[i]; }
      int incl = s;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (tid >= d) incl += y;
      }
      int above = incl - s;                      // keys with a larger digit than my first
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (above < remaining && remaining <= above + c4[i]) {
          sm.digit = 255 - 4 * tid - i;
          sm.above = above;
        }
        above += c4[i];
      }
    }
    __syncthreads();
    remaining -= sm.above;
    prefix |= static_cast<uint32_t>(sm.digit) << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix is the exact key of the want-th largest candidate; `remaining` of the keys
  // equal to it are taken, those with the smallest block index.
  const uint32_t T = prefix;
  const int chunk = (C + kThreads - 1) / kThreads;
  const int c0 = min(tid * chunk, C), c1 = min(c0 + chunk, C);
  int nties = 0;
  for (int c = c0; c < c1; ++c) nties += keys[c] == T;
  const int tie_before = block_exclusive_scan<kThreads>(nties, sm.tmp);
  int nsel = 0;
  {
    int tb = tie_before;
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = keys[c];
      nsel += kk > T || (kk == T && tb < remaining);
      tb += kk == T;
    }
  }
  const int sel_before = block_exclusive_scan<kThreads>(nsel, sm.tmp);
  int tb = tie_before, at = n_init + sel_before;
  for (int c = c0; c < c1; ++c) {
    const uint32_t kk = keys[c];
    const bool take = kk > T || (kk == T && tb < remaining);
    tb += kk == T;
    if (take && at < k - n_local) {
      if (outp) outp[at] = bt[lo + c];
      out[at++] = lo + c;
    }
  }
}

}  // namespace msa

namespace msa {

// Candidate order of the keys a wave holds, kR per lane: lane-major (lane L holds
// candidates L kR .. L kR + kR - 1) or register-major (register i of lane L holds
// candidate 64 i + L, so that a load of one register is 64 consecutive words).
//
// Ranks in candidate order of the keys where p holds: r[i] counts the such keys before
// key i; returns their number. With 32 keys per lane (lane-major only) each lane counts
// its own and one DPP prefix sum adds the lanes; otherwise one ballot per register.
template <int kR, bool kLaneMajor>
__device__ __forceinline__ int wave_ranks(const bool (&p)[kR], int (&r)[kR]) {
  if constexpr (kLaneMajor && kR >= 32) {
    uint32_t c = 0u;
#pragma unroll
    for (int i = 0; i < kR; ++i) c += p[i];
    const uint32_t incl = wave_scan_add_u32(c);
    int b = static_cast<int>(incl - c);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      r[i] = b;
      b += p[i];
    }
    return __builtin_amdgcn_readlane(static_cast<int>(incl), 63);
  } else if constexpr (kLaneMajor) {
    int b = 0, total = 0;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const uint64_t m = __ballot(p[i]);
      b += __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u));
      total += __popcll(m);
    }
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      r[i] = b;
      b += p[i];
    }
    return total;
  } else {
    int base = 0;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const uint64_t m = __ballot(p[i]);
      r[i] = base + static_cast<int>(__builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(m >> 32),
                                                               __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(m), 0u)));
      base += __popcll(m);
    }
    return base;
  }
}

// Exact top `want` of the keys a wave holds (kR per lane, in the candidate order above):
// take[i] marks the chosen keys, those above the want-th largest key T and, of the keys
// equal to T, the first ones in candidate order; pos[i] is a chosen key's rank among the
// chosen ones in candidate order. Returns how many are chosen. Key 0 marks an empty slot
// (below every real key); if there are no more than `want` real keys, all are taken.
//
// T is built two bits at a time from the highest bit in which the candidates differ
// (three independent counts per step); ties at T are ranked in candidate order.
// No barriers, no LDS.
template <int kR, bool kLaneMajor = true>
__device__ __forceinline__ int wave_topk(const uint32_t (&key)[kR], int want, bool (&take)[kR], int (&pos)[kR]) {
  // Counting: up to 16 keys per lane one ballot and popcount per register; with 32 each
  // lane counts its own keys and one DPP sum (or prefix sum) adds the lanes (measured:
  // faster with 32 keys per lane, slightly slower with 16, the same with 8).
  constexpr bool kLaneCount = kR >= 32;
  static_assert(kLaneMajor || !kLaneCount, "32 keys per lane are held lane-major");
  // Ties at the largest real key (want or more candidates share it): that key is the
  // threshold, nothing lies above it, and the first `want` keys equal to it in candidate
  // order are the selection, found without the bit-by-bit search (which could never
  // stop early) and without the counts below.
  uint32_t k_max = 0u;
#pragma unroll
  for (int i = 0; i < kR; ++i) k_max = max(k_max, key[i]);
  k_max = wave_max_u32(k_max);
  bool p[kR];
  int r[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) p[i] = key[i] == k_max;
  const int n_max = wave_ranks<kR, kLaneMajor>(p, r);
  if (k_max != 0u && n_max >= want) {
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      take[i] = p[i] && r[i] < want;
      pos[i] = r[i];
    }
    return want;
  }
  int n_real = 0;
#pragma unroll
  for (int i = 0; i < kR; ++i) n_real += __popcll(__ballot(key[i] != 0u));
  if (n_real <= want) {                                   // every real key
#pragma unroll
    for (int i = 0; i < kR; ++i) take[i] = key[i] != 0u;
    wave_ranks<kR, kLaneMajor>(take, pos);
    return n_real;
  }
  // The bits every candidate shares are the threshold's too: start below them.
  uint32_t k_or = 0u, k_and = ~0u;
#pragma unroll
  for (int i = 0; i < kR; ++i)
    if (key[i] != 0u) { k_or |= key[i]; k_and &= key[i]; }
  k_or = wave_or(k_or);                          // wave-uniform (scalar) from here
  k_and = wave_and(k_and);
  const uint32_t diff = k_or ^ k_and;
  const int top = diff != 0u ? 31 - __builtin_clz(diff) : -1;   // highest differing bit
  // T keeps count(key >= T) >= want. It starts as the shared prefix (<= every key) and
  // ends as the exact want-th largest key or, if some count hit want exactly (then the
  // keys >= T are the selection and the search stops), as that candidate.
  uint32_t T = top < 0 ? k_and : top >= 31 ? 0u : (k_and & ~((2u << top) - 1u));
  auto count_ge = [&](uint32_t c) {
    int n = 0;
    if constexpr (kLaneCount) {
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < kR; ++i) m += key[i] >= c;
      n = static_cast<int>(wave_sum_u32(m));
    } else {
#pragma unroll
      for (int i = 0; i < kR; ++i) n += __popcll(__ballot(key[i] >= c));
    }
    return n;
  };
  // Two thresholds in one sum: per-lane counts (at most 32) in the two 16-bit halves.
  auto count_ge2 = [&](uint32_t c_lo, uint32_t c_hi, int& n_lo, int& n_hi) {
    if constexpr (kLaneCount) {
      uint32_t m = 0u;
#pragma unroll
      for (int i = 0; i < kR; ++i) m += (key[i] >= c_lo ? 1u : 0u) + (key[i] >= c_hi ? 0x10000u : 0u);
      const uint32_t t = wave_sum_u32(m);
      n_lo = static_cast<int>(t & 0xffffu);
      n_hi = static_cast<int>(t >> 16);
    } else {
      n_lo = count_ge(c_lo);
      n_hi = count_ge(c_hi);
    }
  };
  int bit = top;
  bool done = false;
  for (; bit >= 1; bit -= 2) {                   // bits bit, bit-1
    const uint32_t c1 = T | (1u << (bit - 1)), c2 = T | (2u << (bit - 1)), c3 = T | (3u << (bit - 1));
    int n1, n2;
    count_ge2(c1, c2, n1, n2);
    const int n3 = count_ge(c3);   // n1 >= n2 >= n3
    if (n3 >= want) {
      T = c3;
      done = n3 == want;
    } else if (n2 >= want) {
      T = c2;
      done = n2 == want;
    } else if (n1 >= want) {
      T = c1;
      done = n1 == want;
    }
    if (done) break;
  }
  if (!done && bit == 0 && count_ge(T | 1u) >= want) T |= 1u;

  // keys above T (their number) and the ranks of the keys equal to T
  int gt = 0;
  if constexpr (kLaneCount) {
    uint32_t m = 0u;   // this lane's keys above T (low half) and equal to T (high half)
#pragma unroll
    for (int i = 0; i < kR; ++i) m += (key[i] > T ? 1u : 0u) + (key[i] == T ? 0x10000u : 0u);
    const uint32_t incl = wave_scan_add_u32(m);
    gt = static_cast<int>(static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(incl), 63)) & 0xffffu);
    int tb = static_cast<int>((incl - m) >> 16);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      r[i] = tb;
      tb += key[i] == T;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kR; ++i) gt += __popcll(__ballot(key[i] > T));
#pragma unroll
    for (int i = 0; i < kR; ++i) p[i] = key[i] == T;
    wave_ranks<kR, kLaneMajor>(p, r);
  }
  const int need = want - gt;                            // keys equal to T to take
#pragma unroll
  for (int i = 0; i < kR; ++i) take[i] = key[i] > T || (key[i] == T && r[i] < need);
  wave_ranks<kR, kLaneMajor>(take, pos);
  return want;
}

// Wave-level (64-lane) selection for one row, without barriers or LDS atomics. Lane L
// holds candidates L*kR .. L*kR+kR-1 (block lo + c), so block order is lane-major.
//
// The want-th largest key T is built two bits at a time from the highest bit in which
// the candidates differ (three independent ballot + popcount counts per step). Keys
// above T are taken, and of the keys equal to T the ones with the smallest block
// index (rank by mbcnt prefix counts).
//
// The scores and the block-table row are read for every candidate slot inside the
// row's max_blocks before the row's position (and so its length) is read, so all three
// loads overlap. The table is written to LDS: entry e (block, and its page from `bt`)
// at sel[e], pages[e] for e < 64, -1 past the k entries; the caller synchronises the
// workgroup before reading it.
template <int kR>
__device__ __forceinline__ void wave_select_table(const float* srow, const int32_t* bt, int max_blocks,
                                                  const int32_t* row_pos, int k, int n_init, int n_local,
                                                  int* sel, int* pages) {
  const int lane = threadIdx.x & 63;
  const int lo = n_init, want = k - n_init - n_local;
  float sv[kR];
  int32_t pg[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int c = lane * kR + i;
    const bool in_row = lo + c < max_blocks;
    sv[i] = in_row ? srow[lo + c] : 0.0f;
    pg[i] = in_row ? bt[lo + c] : -1;
  }
  const int32_t pg_init = lane < n_init && lane < max_blocks ? bt[lane] : -1;   // blocks below lo
  // Slots 64 kR .. 64 kR + 63 past the keys hold only forced last blocks (n_local <= 64):
  // their pages are read now too, so no block-table read waits for the row's length.
  const int32_t pg_tail = lo + 64 * kR + lane < max_blocks ? bt[lo + 64 * kR + lane] : -1;
  // The row's position is read only now, so its load queues behind the score loads
  // instead of holding them back.
  asm volatile("" ::: "memory");
  const int nb = min(*row_pos / MSA_PAGE_SIZE + 1, max_blocks);
  const int C = nb - n_init - n_local;
  uint32_t key[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) key[i] = lane * kR + i < C ? float_key(sv[i]) : 0u;   // 0: below every real key
  // Pages come from the registers loaded above (block lo + c is in slot c), so writing
  // the table never waits for another block-table read.
  if (nb <= k) {                                           // identity table
    if (lane < lo && lane < nb) { sel[lane] = lane; pages[lane] = pg_init; }
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int b = lo + lane * kR + i;
      if (b < nb) { sel[b] = b; pages[b] = pg[i]; }
    }
    if (lane >= nb) { sel[lane] = -1; pages[lane] = -1; }
    return;
  }
  // Forced entries and padding; the `want` entries in between come from the search.
  // Lane j < n_local takes the page of block nb - n_local + j from the lane holding its
  // slot c (lane c / kR, register c % kR, or the tail registers past 64 kR).
  int32_t pg_local = -1;
  {
    const int c = nb - n_local + min(lane, n_local - 1) - lo;   // 0 <= c < 64 kR + 64
    const bool tail = c >= 64 * kR;
    const int src = tail ? c - 64 * kR : c / kR;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int32_t v = __shfl(pg[i], src, 64);
      if (!tail && c % kR == i) pg_local = v;
    }
    const int32_t v = __shfl(pg_tail, src, 64);
    if (tail) pg_local = v;
  }
  if (lane < n_init) { sel[lane] = lane; pages[lane] = pg_init; }
  if (lane >= k) { sel[lane] = -1; pages[lane] = -1; }
  auto write_local = [&]() {
    if (lane < n_local) { sel[k - n_local + lane] = nb - n_local + lane; pages[k - n_local + lane] = pg_local; }
  };
  if (want == 0) {
    write_local();
    return;
  }

  bool take[kR];
  int pos[kR];
  wave_topk<kR>(key, want, take, pos);
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (take[i]) {
      sel[n_init + pos[i]] = lo + lane * kR + i;
      pages[n_init + pos[i]] = pg[i];
    }
  }
  write_local();
}

// LDS of the two-level selection: each first-level wave's picks (key, block, page),
// want slots per wave (at most 8 waves x 63).
struct MultiSelectSmem {
  uint32_t key[8 * MSA_MAX_TOPK];
  int32_t blk[8 * MSA_MAX_TOPK];
  int32_t pg[8 * MSA_MAX_TOPK];
};

// Two-level selection for one row by `nw` waves of a workgroup (1 <= nw <= 8; nw * 64 kR
// slots cover every candidate, and nw * want <= 64 kR): multiwave_select_level1 in every
// wave, a workgroup barrier, and, with nw > 1, multiwave_select_level2 in wave 0 and
// another barrier; the table is then in sel / pages as wave_select_table writes it.
// kOneWave (the caller's nw is 1): the single first-level wave writes the whole table
// itself, and the caller runs no second level.
//
// Level 1: wave w (< nw) takes candidate slots [64 kR w, 64 kR (w + 1)) (block lo + c,
// register-major inside the wave: one load per register reads 64 consecutive words, where
// lane-major loads would touch kR times as many cache lines each, and the compute unit
// looks them up one by one), reads their scores and pages, and picks its own top
// `want` by the selection order (higher score, then smaller block); it writes them in
// block order to slots [w want, (w + 1) want) of the LDS list (key 0 in unused slots).
// The block-order list then holds every block of the row's top `want`: such a block is
// also among the top `want` of its own wave's candidates. Level 1 also writes what
// needs no search: the identity table of a short row (wave 0), the forced first blocks
// (wave 0), the forced last blocks (the wave holding their slots, or the last wave for
// slots past every wave's), and the padding.
// Level 2: wave 0 picks the top `want` of the list (kR per lane, block order kept) and
// writes them, ascending, between the forced entries.
// Each level-1 wave searches 64 kR keys instead of one wave searching all of them.
// Level 1 returns the row's visible block count in the waves below nw (0 in the others).
//
// kPoll: the scores are still being written, by other workgroups of the same launch,
// into an exchange row whose words hold MSA_MERGE_IDLE_BITS until written (the
// single-launch step). The row's length is then read first, and the words of its
// visible blocks are read agent-coherently, again until none is idle, for at most
// poll->limit rounds (poll->timed_out reports the bound reached; the picks are then
// meaningless). A row with nb <= k needs no score and reads none.
struct ScorePoll {
  const float* row;   // the row's exchange words, [0, nb) written in this launch
  int limit;
  bool timed_out;
};
template <int kR, bool kPoll = false, bool kOneWave = false>
__device__ __forceinline__ int multiwave_select_level1(const float* srow, const int32_t* bt, int max_blocks,
                                                       const int32_t* row_pos, int k, int n_init, int n_local,
                                                       int nw, int* sel, int* pages, MultiSelectSmem& ms,
                                                       ScorePoll* poll = nullptr) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lo = n_init, want = k - n_init - n_local;
  int nb = 0;
  if (wave < nw) {
    const int c0 = 64 * kR * wave;
    float sv[kR];
    int32_t pg[kR];
    if constexpr (kPoll) nb = min(*row_pos / MSA_PAGE_SIZE + 1, max_blocks);
    // Candidate slots past the row's table read as 0 through buffer resources of the
    // table's extent (no branch around a load); nothing uses their values.
    const uint32_t row_bytes = static_cast<uint32_t>(max(max_blocks - lo, 0)) * 4u;
    const __amdgpu_buffer_rsrc_t br = make_rsrc(uniform_ptr(bt + lo), row_bytes);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(uniform_ptr(srow + lo), kPoll ? 0u : row_bytes);
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int off = (c0 + 64 * i + lane) * 4;
      if constexpr (!kPoll) sv[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, off, 0, 0));
      pg[i] = static_cast<int32_t>(__builtin_amdgcn_raw_buffer_load_b32(br, off, 0, 0));
    }
    const int32_t pg_init = wave == 0 && lane < n_init && lane < max_blocks ? bt[lane] : -1;   // blocks below lo
    // slots past every wave's hold only forced last blocks (n_local <= 64): the last
    // wave reads their pages too, so no block-table read waits for the row's length
    const int ct = 64 * kR * nw + lane;
    const int32_t pg_tail = wave == nw - 1 && lo + ct < max_blocks ? bt[lo + ct] : -1;
    if constexpr (kPoll) {
#pragma unroll
      for (int i = 0; i < kR; ++i) sv[i] = 0.0f;
      if (nb > k) {
        // (words past nb lie outside the resource: they read as 0, which is not idle)
        const __amdgpu_buffer_rsrc_t xr = make_rsrc(uniform_ptr(poll->row), static_cast<uint32_t>(nb) * 4u);
        bool ready = false;
        for (int spin = 0; !ready && spin < poll->limit; ++spin) {
          if (spin > 0) __builtin_amdgcn_s_sleep(2);
          uint32_t key = ~0u;
#pragma unroll
          for (int i = 0; i < kR; ++i) {
            sv[i] = load_coherent1(xr, static_cast<uint32_t>(lo + c0 + 64 * i + lane) * 4u);
            key = idle_key(key, sv[i]);
          }
          ready = __ballot(key == 0u) == 0;
        }
        if (!ready) poll->timed_out = true;
      }
    } else {
      asm volatile("" ::: "memory");   // the position's load queues behind the others
      nb = min(*row_pos / MSA_PAGE_SIZE + 1, max_blocks);
    }
    const int C = nb - n_init - n_local;
    if (nb <= k) {                                           // identity table (wave 0 holds it all)
      if (wave == 0) {
        if (lane < lo && lane < nb) { sel[lane] = lane; pages[lane] = pg_init; }
#pragma unroll
        for (int i = 0; i < kR; ++i) {
          const int b = lo + 64 * i + lane;
          if (b < nb) { sel[b] = b; pages[b] = pg[i]; }
        }
        if (lane >= nb) { sel[lane] = -1; pages[lane] = -1; }
      }
    } else {
      if (wave == 0) {
        if (lane < n_init) { sel[lane] = lane; pages[lane] = pg_init; }
        if (lane >= k) { sel[lane] = -1; pages[lane] = -1; }
      }
      // forced last blocks: slots C .. C + n_local - 1
#pragma unroll
      for (int i = 0; i < kR; ++i) {
        const int c = c0 + 64 * i + lane;
        if (c >= C && c < C + n_local) { sel[k - n_local + c - C] = lo + c; pages[k - n_local + c - C] = pg[i]; }
      }
      if (wave == nw - 1 && ct >= C && ct < C + n_local) {
        sel[k - n_local + ct - C] = lo + ct;
        pages[k - n_local + ct - C] = pg_tail;
      }
      uint32_t key[kR];
#pragma unroll
      for (int i = 0; i < kR; ++i) key[i] = c0 + 64 * i + lane < C ? float_key(sv[i]) : 0u;   // 0: below every real key
      if (want > 0) {
        bool take[kR];
        int pos[kR];
        const int n_taken = wave_topk<kR, false>(key, want, take, pos);
        if constexpr (kOneWave) {
          // one first-level wave: its picks are the selection (no second level)
#pragma unroll
          for (int i = 0; i < kR; ++i) {
            if (take[i]) {
              sel[n_init + pos[i]] = lo + c0 + 64 * i + lane;
              pages[n_init + pos[i]] = pg[i];
            }
          }
        } else {
          // this wave's picks, in block order, then key-0 slots up to `want`
#pragma unroll
          for (int i = 0; i < kR; ++i) {
            if (take[i]) {
              const int at = wave * want + pos[i];
              ms.key[at] = key[i];
              ms.blk[at] = lo + c0 + 64 * i + lane;
              ms.pg[at] = pg[i];
            }
          }
          for (int j = n_taken + lane; j < want; j += 64) ms.key[wave * want + j] = 0u;
        }
      }
    }
  }
  return nb;
}

// Level 2, wave 0 (nb from its level 1): the top `want` of the nw * want picks (block
// order: wave-major, ascending inside each wave), written between the forced entries.
template <int kR>
__device__ __forceinline__ void multiwave_select_level2(int nb, int k, int n_init, int n_local, int nw, int* sel,
                                                        int* pages, const MultiSelectSmem& ms) {
  static_assert(64 * kR <= 8 * MSA_MAX_TOPK, "the level-2 reads stay inside the lists");
  const int lane = threadIdx.x & 63;
  const int want = k - n_init - n_local;
  if (nb <= k || want <= 0) return;
  const int n = nw * want;
  uint32_t key[kR];
  int32_t blk[kR], pg[kR];
  // (every read stays inside the lists, 64 kR <= 8 * MSA_MAX_TOPK entries; blk and pg
  // of a slot past n are never used, since its key is 0 and it is not taken)
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    const int j = lane * kR + i;
    key[i] = ms.key[j];
    blk[i] = ms.blk[j];
    pg[i] = ms.pg[j];
    if (j >= n) key[i] = 0u;
  }
  bool take[kR];
  int pos[kR];
  wave_topk<kR>(key, want, take, pos);
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (take[i]) {
      sel[n_init + pos[i]] = blk[i];
      pages[n_init + pos[i]] = pg[i];
    }
  }
}

// Largest number of candidate blocks the wave-level selection handles (64 lanes x 32).
constexpr int kWaveSelectMax = 64 * 32;

// Dispatch on the largest candidate count the row table allows (known before the row's
// length is): kR = 4, 8, 16 or 32 keys per lane, up to kMaxR (a caller that never has
// more than 64 kMaxR candidates leaves the wider searches, and their registers, out).
template <int kMaxR = 32>
__device__ __forceinline__ void wave_select(const float* srow, const int32_t* bt, int max_blocks,
                                            const int32_t* row_pos, int k, int n_init, int n_local,
                                            int* sel, int* pages) {
  static_assert(kMaxR == 16 || kMaxR == 32, "16 or 32 keys per lane at most");
  const int C = max_blocks - n_init - n_local;
  if (C <= 256) wave_select_table<4>(srow, bt, max_blocks, row_pos, k, n_init, n_local, sel, pages);
  else if (C <= 512) wave_select_table<8>(srow, bt, max_blocks, row_pos, k, n_init, n_local, sel, pages);
  else if (kMaxR == 16 || C <= 1024)
    wave_select_table<16>(srow, bt, max_blocks, row_pos, k, n_init, n_local, sel, pages);
  else wave_select_table<kMaxR>(srow, bt, max_blocks, row_pos, k, n_init, n_local, sel, pages);
}

}  // namespace msa
