// Sparse GQA flash-decode over the selected P128 pages with split-KV partials:
//   msa_sparse_decode          selection table in, partials out
//   msa_sparse_decode_combine  selection table in, partials + merged bf16 output out
//   msa_select_decode_combine  block scores in: each workgroup selects its row's blocks
//                              itself, then decodes and merges
//
// Prior art on the pages: [Rubin] commit messages describe a block-sparse verify
// decode with one unit of work per (top-k split, KV head, query row) and NVFP4
// dequantised in registers, merging splits across CTAs; [Rubin] "Items and numerics"
// (LC_ONEDIV) fixes the merge to a single divide per output in a fixed order.
//
// MI355X design. One workgroup per (split, KV head, query row). The split's pages are
// cut into 32-token chunks and each wave takes its chunks (one chunk per wave at the
// default launch), so a page is consumed by several SIMDs at once; the waves merge
// their softmax states in LDS. All 16 query heads of the KV head ride in the MFMA N
// dimension, so both contractions keep "head" on lane % 16:
//   S^T[token][head] = K[token][d] . Q^T[d][head]      A = K  (dequantised in registers)
//   O^T[d][head]    += V^T[d][token] . P^T[token][head] A = V^T (LDS, transposing read)
// and the softmax state (max, sum, rescale) is per lane, with no cross-lane transpose.
// K and V are dequantised exactly to fp16 (E2M1 x E4M3 has at most 6 significant bits;
// E4M3 fits fp16), Q is pre-scaled by a power of two per head so its fp16 conversion
// is exact, accumulation is fp32. The NVFP4 tensor scales and FP8 page scales are
// applied outside the MFMAs (folded into the logit scale and the output rescale).
// Every load a wave needs (selection entry, page id, K/V codes and scales, Q) is
// issued before the first MFMA, so the kernel pays the memory latency once.
//
// The combining variants have the last workgroups of each (row, KV head) to count
// themselves in merge all splits, each a slice of the 16 heads, so the step needs no
// separate combine launch and no one compute unit pulls every partial; with a single
// split that workgroup writes the output directly and the merge workspace is not
// touched. The partials cross workgroups (and XCDs, whose L2s are not coherent
// with each other) through agent-coherent stores that the merger polls against an idle
// pattern: no cache-flushing fence (on this part such fences cost more than the whole
// merge) and no wait for store acknowledgements. Two exchange buffers alternate
// between calls, and each split returns its slot of the idle one to the idle pattern
// early in the call. The selecting variant runs the top-k selection of its row in
// every workgroup (the scores are 4 bytes per block), which costs less than a launch
// plus a cross-workgroup handoff.
//
// Page data is read through buffer resources based at each selected (page, KV head):
// every chunk issues the same loads (an empty one from a zero-byte resource, which
// returns zeros without a memory access), so the query's conversion and everything
// else that waits on earlier loads does not wait for the page data.
#include <algorithm>
#include <type_traits>

#include "msa_device.h"
#include "msa_host.h"
#include "decode_device.h"
#include "score_device.h"
#include "select_device.h"

namespace msa {
namespace {

struct DecodeArgs {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_scales;
  const uint8_t* v_scales;
  float k_t, v_t;
  int hkv;
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int max_blocks;
  int num_rows;
  uint64_t seq_mul;           // seq_guess multiplier
  const uint16_t* q;
  int sel_tables;             // 1: one table per row; hkv: one per (row, KV head)
  const int32_t* sel;         // selection table (table variants)
  const int32_t* sel_pages;   // may be null: translate through the block table
  int32_t* sel_out;           // selecting variant: optional copy of the selection
  int32_t* sel_pages_out;
  const float* scores;        // selecting variant
  int n_init, n_local;
  int sel_waves;              // selecting variant: first-level waves of the two-level selection
                              // (0: the row is too long for it; the block radix select runs)
  int k;
  float softmax_scale;
  int num_splits;
  float* part_o;
  float* part_ml;
  int32_t* counters;          // combining variants: merge state words [rows][hkv]
  int num_seqs, num_pages;
  int32_t* err;               // debug library: the error word of failed metadata checks
  uint16_t* out;              // combining variants: bf16 [rows][hq][128]
  // Bound on the last split's poll rounds (kMergePollLimit; the debug library can lower
  // it). Every slot it polls has been stored by a split that is already past its
  // compute, so a few rounds suffice; the bound only keeps the loop finite.
  int poll_limit;
  // Bound on the poll rounds of a merging split that is not the last to arrive, before
  // it hands its slice to the last one (kMergeHelperPolls; the debug library can set it).
  int helper_poll_limit;
};

// The single-launch step (msa_decode_step): scoring, append and the row's score
// exchange, on top of the selecting decode's arguments.
struct StepArgs {
  StepScoreArgs sc;
  int32_t* words;      // [rows]: workgroups that have read the row's scores (0 between launches)
  int rows_per_seq;    // every request's row count (stated by the caller)
  int readers;         // workgroups that read one row's scores: hkv * num_splits
  AppendArgs app;      // at most 64 new tokens
};
// Index heads of the single-launch step.
constexpr int kStepHi = 4;

template <int kFmt, int kItems>
struct Round {
  ChunkRegs<kFmt> R[kItems];
  int nvis[kItems];                // visible tokens of each chunk (0: no chunk)
  uint64_t hits[kItems];           // single-launch step: new tokens in each chunk
  float kps[kItems], vps[kItems];  // FP8 page scales (1 for NVFP4)
};

// Issue every load of one round: chunk `it = round + wave + j * kW` of this split is
// entry lo + it / 4, 32-token chunk it % 4. `lookup(e, b, page)` gives the logical
// block and physical page of selection entry e (b < 0: empty entry). Chunks past the
// split, of empty entries or with no visible token issue the same loads from
// zero-byte resources (see load_chunk).
// kStep: tokens appended in the same launch are patched into the loaded chunk from
// their encoding in LDS (patch_new_tokens; slot0 as there).
template <int kFmt, int kW, int kItems, bool kStep, class Lookup>
__device__ __forceinline__ void load_round(Round<kFmt, kItems>& rd, const DecodeArgs& a, const KvArrays& kv,
                                           const StepArgs& st, const NewKv<kFmt>* nk, int64_t slot0,
                                           const Lookup& lookup, int round, int wave, int g, int pos, int lo,
                                           int n_items, int n, int q) {
  // The row position, block and page are the same in every lane; reading them through
  // readfirstlane tells the compiler so, and the buffer resources below stay in scalar
  // registers (a resource it cannot prove uniform costs a loop over lanes per load).
  const int upos = __builtin_amdgcn_readfirstlane(pos);
#pragma unroll
  for (int j = 0; j < kItems; ++j) {
    const int it = round + wave + j * kW;
    const int e = lo + min(it, n_items - 1) / 4, c = it & 3;
    int b;
    int64_t page;
    lookup(e, b, page);
    b = __builtin_amdgcn_readfirstlane(b);
    const int nv = min(upos - b * kPage + 1, kPage) - 32 * c;   // visible tokens in the chunk
    const bool valid = it < n_items && b >= 0 && nv > 0;
    rd.nvis[j] = valid ? min(nv, 32) : 0;
    page = valid ? checked_page(page, a.num_pages, a.err) : 0;
    page = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(page))));
    load_chunk<kFmt>(rd.R[j], kv, page * a.hkv + g, valid, c, n, q);
    rd.kps[j] = rd.vps[j] = 1.0f;
    if constexpr (kFmt == MSA_KV_FP8_E4M3) {   // the page's scales (page 0 for an empty chunk)
      // (vector loads through resources: a plain load from the register-pinned pointer
      // would be a flat access, which every later wait on the LDS counter also waits for)
      rd.kps[j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(kv.k_scales + page * 4, 4u), 0, 0, 0));
      rd.vps[j] = __builtin_bit_cast(
          float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(kv.v_scales + page * 4, 4u), 0, 0, 0));
    }
    rd.hits[j] = 0u;
    if constexpr (kStep)
      if (valid) rd.hits[j] = new_tokens_in_chunk(slot0, page, c);
  }
}

// kV consecutive floats of one split's partial, read agent-coherently.
template <int kV>
__device__ __forceinline__ void load_slot(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[kV]) {
  if constexpr (kV == 4) {
    const float4_t x = load_coherent4(r, off);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  } else if constexpr (kV == 2) {
    const float2_t x = load_coherent2(r, off);
    v[0] = x[0]; v[1] = x[1];
  } else {
    v[0] = load_coherent1(r, off);
  }
}

// A merging split's read of kV consecutive output dims d.. of head h: all S <= kS
// slots (its own included: it stored them and reads them back), then the fixed-order
// log-sum-exp sums of msa_combine. Slots whose words have not all landed are read
// again. Entries S..kS-1 repeat the last slot and are not used, so every entry is
// redefined on each read and none is carried from one poll to the next. Returns false
// if some word was still idle after `limit` rounds (num and den are then meaningless).
template <int kS, int kV>
__device__ __forceinline__ bool merge_slots(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rm, int S,
                                            int h, int d, int limit, float (&num)[kV], float& den) {
  float2_t mls[kS];
  float ot[kS][kV];
  bool ready = false;
  for (int spin = 0; !ready && spin < limit; ++spin) {
    if (spin > 0) {
      __builtin_amdgcn_s_sleep(2);
      asm volatile("" ::: "memory");   // load again
    }
#pragma unroll
    for (int t = 0; t < kS; ++t) {   // every load first, one wait
      const int tt = min(t, S - 1);
      mls[t] = load_coherent2(rm, (h * S + tt) * 8u);
      load_slot<kV>(ro, ((h * S + tt) * kHeadDim + d) * 4u, ot[t]);
    }
    asm volatile("" ::: "memory");   // the loads stay together, ahead of their tests
    uint32_t key = ~0u;
#pragma unroll
    for (int t = 0; t < kS; ++t) {
      key = idle_key(key, mls[t]);
#pragma unroll
      for (int i = 0; i < kV; ++i) key = idle_key(key, ot[t][i]);
    }
    ready = key != 0u;
  }
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < kS; ++t)
    if (t < S) M = fmaxf(M, mls[t][0]);
#pragma unroll
  for (int i = 0; i < kV; ++i) num[i] = 0.0f;
  den = 0.0f;
#pragma unroll
  for (int t = 0; t < kS; ++t) {
    if (t < S) {
      const float m = mls[t][0];
      const float wgt = m == -INFINITY ? 0.0f : exp2_raw(m - M);   // M > -inf whenever m is
      den += wgt * mls[t][1];
#pragma unroll
      for (int i = 0; i < kV; ++i) num[i] += wgt * ot[t][i];
    }
  }
  return ready;
}

template <int kV>
__device__ __forceinline__ bool merge_slots_any(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rm, int S, int h,
                                                int d, int limit, float (&num)[kV], float& den) {
  if (S <= 2) return merge_slots<2, kV>(ro, rm, S, h, d, limit, num, den);
  if (S <= 4) return merge_slots<4, kV>(ro, rm, S, h, d, limit, num, den);
  if (S <= 8) return merge_slots<8, kV>(ro, rm, S, h, d, limit, num, den);
  return merge_slots<16, kV>(ro, rm, S, h, d, limit, num, den);
}

// A merging split that is not the last to arrive hands its slice to the last one: it
// sets the slice's bit in the state word, which succeeds only while the last split has
// not yet counted itself in (the bit is then in the old word that split's count
// returns). Returns false once the last split has arrived (or the word is invalid):
// every split has then counted itself in. Each failed exchange means the word changed
// (an arrival or another slice's handoff, a bounded number per launch).
__device__ __forceinline__ bool merge_handoff(int32_t* word, uint32_t buffer, int S, int slice) {
  uint32_t w = static_cast<uint32_t>(__hip_atomic_load(word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  for (int tries = 0; tries < 64; ++tries) {
    if ((w >> 31) != buffer || (w & kMergeTimeoutBit) != 0u || (w & kMergeArrivalMask) >= static_cast<uint32_t>(S))
      return false;
    int32_t expected = static_cast<int32_t>(w);
    if (__hip_atomic_compare_exchange_strong(word, &expected,
                                             static_cast<int32_t>(w | (1u << (kMergeHandoffShift + slice))),
                                             __ATOMIC_RELAXED, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
      return true;
    w = static_cast<uint32_t>(expected);
  }
  return false;
}

// What a workgroup writes: its split's partial (kOutPartials), the bf16 output of the
// only split (kOutDirect), or its partial through the merge workspace, the last splits
// of the (row, KV head) merging them all into the bf16 output (kOutMerged). The direct
// variant holds none of the merge code, and so fewer registers. kSelect: 0 = the
// caller's table; 1, 2, 4 or 8 = the workgroup selects, with the two-level selection at
// kSelect keys per lane (or the block radix select for rows too long for it);
// kSelectOneWave = at most 64 candidates, one first-level wave and no second level.
constexpr int kOutPartials = 0, kOutDirect = 1, kOutMerged = 2;
constexpr int kSelectOneWave = 16;

// The single-launch step's scoring share of one workgroup. The decode workgroups of a
// group of rows (up to 16 / kStepHi rows of one request, cut in request order, as the
// scorer groups them) score that group's blocks: block b by the group's wave
// b mod (its waves), so with max_blocks at most twice the smallest group's waves (a
// host check) a wave scores at most two blocks, whose loads go out together.
// Returns the page of row r's last visible block.
template <int kW>
__device__ __forceinline__ int32_t step_score_share(const DecodeArgs& a, const StepArgs& st, int r, int g, int s,
                                                    int wave, int64_t slot0) {
  constexpr int kRpg = 16 / kStepHi;
  const int R = st.rows_per_seq;
  const int seq = r / R, i = r - seq * R;
  const int r0 = seq * R + (i / kRpg) * kRpg, nr = min(kRpg, R - (i / kRpg) * kRpg);
  const int nwv = nr * a.hkv * a.num_splits * kW;
  const int gw = (((r - r0) * a.hkv + g) * a.num_splits + s) * kW + wave;
  const int b[2] = {gw, gw + nwv};
  return score_blocks<kStepHi, 2>(st.sc, a.block_table, a.row_pos, a.max_blocks, a.num_pages, a.err, r0, nr, seq,
                                  b, slot0, r - r0);
}

// 8-wave workgroups that do not merge run two per compute unit when the launch is large
// (one split per (row, KV head) pair): four waves per SIMD, so at most 128 registers.
// (Not the single-launch step, whose scoring phase holds two blocks of keys at once.)
template <int kW, int kOut, bool kStep>
constexpr int decode_min_waves_per_simd() { return kW == 8 && kOut != 2 && !kStep ? 4 : 1; }

// kStep (the single-launch step, selecting variants only): the workgroup first scores
// its share of its row group's blocks into the score exchange and encodes its share of
// the new tokens into the pool, then selects from the exchange as the scores land
// (multiwave_select_level1 in its polling form), decodes with the new tokens patched
// into its registers, and merges. The workgroups of a row group are consecutive in the
// grid (split fastest, then KV head, then row), so those it waits for are dispatched
// before it or with it.
template <int kFmt, int kW, int kItems, int kOut, int kSelect, bool kStep = false>
__global__ void __launch_bounds__(64 * kW)
__attribute__((amdgpu_waves_per_eu(decode_min_waves_per_simd<kW, kOut, kStep>())))
sparse_decode_kernel(DecodeArgs a, StepArgs st) {
  static_assert(!kStep || kSelect, "the single-launch step selects");
  constexpr int kSelR = kSelect == kSelectOneWave ? 1 : kSelect;   // keys per lane of the selection
  // Dynamic LDS: the row's selection keys (selecting variant, before any V is staged),
  // then the per-wave V staging buffers and, at the end, the per-wave O tiles.
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  __shared__ float mbuf[kW][16], lbuf[kW][16];
  __shared__ int s_word;
  __shared__ int s_rlast;   // kStep: this workgroup was the row's last reader
  // kStep: the new tokens' K and V of this KV head, encoded
  __shared__ typename std::conditional<kStep, NewKv<kFmt>, char>::type newkv;
  __shared__ int32_t lsel[kSelect ? MSA_MAX_TOPK : 1], lpage[kSelect ? MSA_MAX_TOPK : 1];
  __shared__ half8_t qlds[kSelect ? 4 : 1][64];   // selecting variant: the converted Q operand
  __shared__ float qcs[kSelect ? 64 : 1];
  __shared__ SelectSmem sm;
  const int pair = blockIdx.y, s = blockIdx.x;   // (row, KV head) pair, split
  if (pair >= a.num_rows * a.hkv) return;
  const int r = pair / a.hkv, g = pair % a.hkv;
  // (the wave index through readfirstlane: the compiler then knows it is the same in
  // every lane, and so is everything derived from it, such as a chunk's page)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int hq = a.hkv * kHeadsPerKv;
  int lo = (s * a.k) / a.num_splits, hi = ((s + 1) * a.k) / a.num_splits;
  // (computed here, in scalar registers: the compiler would otherwise sink the two
  // divisions to their first use, after the selection)
  asm volatile("" : "+s"(lo), "+s"(hi));
  const int n_items = (hi - lo) * 4;   // (entry, 32-token chunk) pairs of this split
  const int64_t head0 = static_cast<int64_t>(r) * hq + kHeadsPerKv * g;
  // The pool's arrays and the partials, held in scalar registers from here (the compiler
  // would otherwise reload them from the kernel arguments between the selection and the
  // page loads, behind a wait that also covers the selection's LDS reads).
  KvArrays kv{uniform_ptr(a.k_codes), uniform_ptr(a.v_codes), uniform_ptr(a.k_scales), uniform_ptr(a.v_scales)};
  float* const part_o = uniform_ptr(a.part_o);
  float* const part_ml = uniform_ptr(a.part_ml);
  asm volatile("" : "+s"(kv.k_codes), "+s"(kv.v_codes), "+s"(kv.k_scales), "+s"(kv.v_scales));

  int64_t slot0 = -1;     // kStep: lane i < n_new holds new token i's slot
  uint64_t in_lds = 0u;   // kStep: new tokens whose K and V of this KV head are encoded in LDS
  if constexpr (kStep) {
    if (lane < st.app.n_new) slot0 = st.app.slot[lane];
    // (the scorer also reads the page of this row's last visible block)
    const int32_t last_page = step_score_share<kW>(a, st, r, g, s, wave, slot0);
    // The append (which nothing in this launch reads: the scorer and the decode encode
    // the new tokens themselves) is written by split 0 of row i % num_rows for new token
    // i: its K and V of each KV head, and its index key from the workgroup of KV head 0.
    // The split that holds the row's last block (split S - 1: the forced local blocks
    // are the table's last entries) is the one that meets tokens appended to the row's
    // last page; it encodes those for its KV head. Both kinds are encoded into LDS (the
    // decode patches them in from there; any other new token it meets is encoded where
    // it is met) by the waves that take no part in the first selection level (all of
    // them if every wave does), during that level's wait for the scores: one group of
    // 16 elements per row of 16 lanes.
    in_lds = __ballot(slot0 >= 0 && ((s == 0 && lane % a.num_rows == r) ||
                                     (s == a.num_splits - 1 && (slot0 >> 7) == last_page)));
    const uint64_t own_idx = s == 0 && g == 0 && st.app.idx_new != nullptr
                                 ? __ballot(lane < st.app.n_new && lane % a.num_rows == r)
                                 : 0u;
    const int enc0 = a.sel_waves < kW ? 64 * a.sel_waves : 0;   // (whole waves)
    const int e = static_cast<int>(threadIdx.x) - enc0;
    if (e >= 0) {
      const int rows = (64 * kW - enc0) >> 4, row = e >> 4, l = e & 15;
      // items: 16 K/V groups of each token in in_lds, then 4 index-key groups of each
      // token in own_idx
      const int n_kv = 16 * __popcll(in_lds), n_items = n_kv + 4 * __popcll(own_idx);
      // up to four items per row at a time: every element load of the four goes out
      // before the first encoding
      for (int base = 0; base < n_items; base += 4 * rows) {   // (the same trip count in every lane)
        int it_[4], tok_[4];
        int64_t sl_[4];
        float x_[4], ps_[4];   // (ps_: FP8 K/V items, the page's scale)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int it = base + u * rows + row;
          it_[u] = it;
          tok_[u] = it >= n_items ? 0 : it < n_kv ? nth_set_bit(in_lds, it >> 4) : nth_set_bit(own_idx, (it - n_kv) >> 2);
          sl_[u] = __shfl(slot0, tok_[u], 64);
          x_[u] = 0.0f;
          ps_[u] = 1.0f;
          if (it < n_items && sl_[u] >= 0) {
            const uint16_t* src;
            int64_t at;
            if (it < n_kv) {
              src = ((it >> 3) & 1) == 0 ? st.app.k_new : st.app.v_new;
              at = (static_cast<int64_t>(tok_[u]) * a.hkv + g) * kHeadDim + 16 * (it & 7) + l;
              if constexpr (kFmt == MSA_KV_FP8_E4M3)
                if (sl_[u] / kPage < a.num_pages)
                  ps_[u] = reinterpret_cast<const float*>(((it >> 3) & 1) == 0 ? a.k_scales : a.v_scales)[sl_[u] / kPage];
            } else {
              src = st.app.idx_new;
              at = static_cast<int64_t>(tok_[u]) * kIndexDim + 16 * ((it - n_kv) & 3) + l;
            }
            if (src != nullptr) x_[u] = bf16_to_f32(src[at]);
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int it = it_[u], tok = tok_[u];
          const int64_t sl = sl_[u];
          // (everything below is the same in the 16 lanes of a row)
          if (it >= n_items || sl < 0 || !dcheck(sl / kPage < a.num_pages, MSA_DEBUG_BAD_SLOT, a.err)) continue;
          if (it < n_kv) {
            const int kv = (it >> 3) & 1, gg = it & 7;
            if ((kv == 0 ? st.app.k_new : st.app.v_new) == nullptr) continue;
            const int64_t prow = (sl / kPage * a.hkv + g) * kPage + sl % kPage;   // the token's row in the pool
            const bool owner = s == 0 && tok % a.num_rows == r;
            if constexpr (kFmt == MSA_KV_NVFP4) {
              uint2 c;
              const uint32_t sc = nvfp4_encode_row(x_[u], kv == 0 ? a.k_t : a.v_t, c);
              if (l == 0) {
                newkv.codes[tok][kv][gg] = c;
                newkv.scales[tok][kv][gg] = static_cast<uint8_t>(sc);
                if (owner) {
                  *reinterpret_cast<uint2*>((kv == 0 ? st.app.k_codes : st.app.v_codes) + prow * (kHeadDim / 2) +
                                            8 * gg) = c;
                  (kv == 0 ? st.app.k_scales : st.app.v_scales)[prow * (kHeadDim / 16) + gg] = static_cast<uint8_t>(sc);
                }
              }
            } else {
              const uint4 c = e4m3_encode_row(x_[u], ps_[u]);
              if (l == 0) {
                newkv.codes[tok][kv][gg] = c;
                if (owner)
                  *reinterpret_cast<uint4*>((kv == 0 ? st.app.k_codes : st.app.v_codes) + prow * kHeadDim + 16 * gg) = c;
              }
            }
          } else if (st.app.idx_new != nullptr) {
            const int j = (it - n_kv) & 3;
            const uint4 c = e4m3_encode_row(x_[u], 1.0f);
            if (l == 0) *reinterpret_cast<uint4*>(st.app.index_k + sl * kIndexDim + 16 * j) = c;
          }
        }
      }
    }
  }

  // Combining variants with several splits: the pair's merge state word (which of the
  // two exchange buffers this launch uses, the split count the workspace was set up
  // for, arrivals so far), read once at the start. Its buffer and split-count fields
  // change only when this launch's merger finishes, after every split has arrived.
  const bool merging = kOut == kOutMerged && a.num_splits > 1;
  uint32_t mstate = 0u;
  if (merging)   // (a per-lane address, so the word stays in a vector register and is
                 // not moved to a scalar one, which would wait for the load right here)
    mstate = static_cast<uint32_t>(__hip_atomic_load(
        a.counters + static_cast<int64_t>(r) * a.hkv + g + lane_varying_zero(), __ATOMIC_RELAXED,
        __HIP_MEMORY_SCOPE_AGENT));
  // The merge workspace is pair-major, [rows][KV heads][2 buffers][16 heads][S][...], so
  // its layout does not depend on how many rows a call has: this pair's slots of
  // buffer b start at row (2 * head0 + 16 * b) * S of 128 (or 2) words.

  // Q^T operand: lane (n, q) holds head 16g + n, dims 32q + 8j .. +7 for k-step j.
  const uint16_t* qh = a.q + (static_cast<int64_t>(r) * hq + kHeadsPerKv * g + n) * kHeadDim + 32 * q;
  uint4 qraw[4];
  auto load_q = [&]() { load_q_raw(qraw, qh); };
  half8_t Qop[4];
  float cscale;
  auto convert_q = [&]() {
    convert_q_op(qraw, Qop, cscale, a.softmax_scale * kLog2e, kFmt == MSA_KV_NVFP4 ? a.k_t : 1.0f);
  };
  // Selecting variant: Q is the same for every wave of the workgroup, so wave 1 loads
  // and converts it while wave 0 selects, and hands it over through LDS.
  auto q_to_lds = [&]() {
    load_q();
    convert_q();
#pragma unroll
    for (int j = 0; j < 4; ++j) qlds[j][lane] = Qop[j];
    qcs[lane] = cscale;
  };
  auto q_from_lds = [&]() {
#pragma unroll
    for (int j = 0; j < 4; ++j) Qop[j] = qlds[j][lane];
    cscale = qcs[lane];
  };
  // Selection table in a register: lane e < k holds entry e (block) and its page.
  // With per-KV-head tables, KV head g reads table g of the row.
  const int64_t trow = static_cast<int64_t>(r) * a.sel_tables + (a.sel_tables > 1 ? g : 0);
  int selv = -1, pagev = -1;
  int pos;
  bool score_timeout = false;   // kStep: some score was still idle after the poll bound
  int32_t reader_old = 0;       // kStep, thread 0: readers of the row before this one
  if constexpr (!kSelect) {
    // the caller's table: one load per lane, issued before the query loads so that
    // the page addresses wait for these alone (the counter retires in order)
    if (lane < a.k) {
      selv = a.sel[trow * a.k + lane];
      if (a.sel_pages) pagev = a.sel_pages[trow * a.k + lane];
    }
    pos = a.row_pos[r];
    load_q();
    // (debug library: an entry that is neither -1 nor a visible block is dropped)
    if (lane < a.k && !dcheck(selv >= -1 && selv < min(pos / kPage + 1, a.max_blocks), MSA_DEBUG_BAD_SEL, a.err))
      selv = -1;
    if (a.sel_pages == nullptr && selv >= 0)
      pagev = a.block_table[static_cast<int64_t>(checked_seq(a.row_seq[r], a.num_seqs, a.err)) * a.max_blocks + selv];
  }
  if constexpr (kSelect) {
    const float* srow = a.scores + trow * a.max_blocks;
    if (a.sel_waves > 0) {
      // The first-level waves read their share of the scores and the block-table row
      // of the request r belongs to when every request has the same number of rows;
      // the pages are read again if row_seq says otherwise. The last wave converts Q
      // (its load goes out first) and hands it over through LDS with the table.
      const int guess = seq_guess(r, a.seq_mul);
      if (wave == kW - 1) load_q();
      // every wave's own copy of the row's position and request, read before the
      // selection so that no wave waits for them after it
      pos = a.row_pos[r];
      const int seq = checked_seq(a.row_seq[r], a.num_seqs, a.err);
      const int32_t* btg = a.block_table + static_cast<int64_t>(guess) * a.max_blocks;
      MultiSelectSmem& ms = *reinterpret_cast<MultiSelectSmem*>(dyn_lds);
      ScorePoll sp{kStep ? st.sc.xscores + trow * a.max_blocks : nullptr, a.poll_limit, false};
      const int nb = multiwave_select_level1<kSelR, kStep, kSelect == kSelectOneWave>(
          srow, btg, a.max_blocks, a.row_pos + r, a.k, a.n_init, a.n_local, a.sel_waves, lsel, lpage, ms, &sp);
      if (wave == kW - 1) {   // (while the first level runs, unless this wave is part of it)
        convert_q();
#pragma unroll
        for (int j = 0; j < 4; ++j) qlds[j][lane] = Qop[j];
        qcs[lane] = cscale;
      }
      if constexpr (kStep) {
        // every score read of the workgroup is done: count it in as a reader of the row
        score_timeout = __syncthreads_or(sp.timed_out);
        if (threadIdx.x == 0) reader_old = atomicAdd(st.words + r, 1);
      } else {
        __syncthreads();
      }
      if constexpr (kSelect != kSelectOneWave) {   // (one first-level wave wrote the table itself)
        if (wave == 0) multiwave_select_level2<kSelR>(nb, a.k, a.n_init, a.n_local, a.sel_waves, lsel, lpage, ms);
        __syncthreads();
      }
      selv = lsel[lane];
      pagev = lpage[lane];
      if (seq != guess) {
        const int32_t* bt = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
        pagev = selv >= 0 ? bt[selv] : -1;
      }
    } else {
      if (wave == 1) q_to_lds();
      pos = a.row_pos[r];
      const int nb = min(pos / kPage + 1, a.max_blocks);
      const int32_t* bt =
          a.block_table + static_cast<int64_t>(checked_seq(a.row_seq[r], a.num_seqs, a.err)) * a.max_blocks;
      block_select_row<false, 64 * kW>(srow, nb, a.k, a.n_init, a.n_local, bt, lsel, nullptr,
                                       reinterpret_cast<uint32_t*>(dyn_lds), sm);
      __syncthreads();
      selv = lane < a.k ? lsel[lane] : -1;
      pagev = selv >= 0 ? bt[selv] : -1;
    }
    if (lane >= a.k) selv = pagev = -1;
  }
  if (wave == 0 && lane == 0 && s == 0) check_pos(pos, a.max_blocks, a.err);
  auto lookup = [&](int e, int& b, int64_t& page) {
    b = __builtin_amdgcn_readlane(selv, e);   // e is the same in every lane
    page = __builtin_amdgcn_readlane(pagev, e);
  };

  Round<kFmt, kItems> rd;
  const NewKv<kFmt>* nk = nullptr;
  if constexpr (kStep) nk = &newkv;
  load_round<kFmt, kW, kItems, kStep>(rd, a, kv, st, nk, slot0, lookup, 0, wave, g, pos, lo, n_items, n, q);
  if constexpr (kSelect) {
    // with the page loads out: the query operand from LDS, and the optional outputs
    q_from_lds();
    if constexpr (kStep) {
      // the selection came from scores that never landed: make every output NaN
      if (score_timeout) {
        dcheck(false, MSA_DEBUG_SCORE_TIMEOUT, a.err);
        cscale = __builtin_nanf("");
      }
    }
    if (s == 0 && (g == 0 || a.sel_tables > 1) && wave == 0 && a.sel_out != nullptr && lane < a.k) {
      a.sel_out[trow * a.k + lane] = selv;
      if (a.sel_pages_out) a.sel_pages_out[trow * a.k + lane] = pagev;
    }
  }

  // This split's slot in the other exchange buffer was read by the previous launch's
  // merger; the last wave puts it back to idle now, off the critical path (its page
  // loads are already out, and they retire before these stores in the counter order).
  if (merging && wave == kW - 1 && merge_state_ok(mstate, a.num_splits)) {
    const int other = static_cast<int>(mstate >> 31) ^ 1;
    const float iv = __uint_as_float(MSA_MERGE_IDLE_BITS);
    const __amdgpu_buffer_rsrc_t xo = make_rsrc(
        uniform_ptr(part_o + (2 * head0 + 16 * other) * a.num_splits * kHeadDim), 16u * a.num_splits * kHeadDim * 4);
    const __amdgpu_buffer_rsrc_t xm =
        make_rsrc(uniform_ptr(part_ml + (2 * head0 + 16 * other) * a.num_splits * 2), 16u * a.num_splits * 8);
#pragma unroll
    for (int j = 0; j < 8; ++j) {   // 16 heads x 32 four-float groups
      const int idx = lane + 64 * j, h = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      store_coherent(xo, ((h * a.num_splits + s) * kHeadDim + 4 * d4) * 4u, float4_t{iv, iv, iv, iv});
    }
    if (lane < 16) store_coherent(xm, (lane * a.num_splits + s) * 8u, float2_t{iv, iv});
  }

  if constexpr (!kSelect) convert_q();

  float m_run = -INFINITY, l_run = 0.0f, v_cur = 0.0f;   // v_cur: FP8 page scale O is kept in
  float4_t O[8];
#pragma unroll
  for (int d = 0; d < 8; ++d) O[d] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  half_t* vb = reinterpret_cast<half_t*>(dyn_lds + wave * kVBufBytes);
  typedef __attribute__((address_space(3))) short4_t lds_s4;

  for (int round = 0; round < n_items; round += kW * kItems) {
    if (round > 0)
      load_round<kFmt, kW, kItems, kStep>(rd, a, kv, st, nk, slot0, lookup, round, wave, g, pos, lo, n_items, n, q);
#pragma unroll
    for (int j = 0; j < kItems; ++j) {
      if (rd.nvis[j] <= 0) continue;
      if constexpr (kStep)
        if (rd.hits[j] != 0u)
          patch_new_tokens<kFmt>(rd.R[j], *nk, st.app, slot0, rd.hits[j], in_lds, g, n, q, rd.kps[j], rd.vps[j]);
      const uint32_t* ksc = nullptr;
      const uint32_t* vsc = nullptr;
      if constexpr (kFmt == MSA_KV_NVFP4) { ksc = rd.R[j].ks; vsc = rd.R[j].vs; }
      const float cs = cscale * rd.kps[j];
      float ratio = 1.0f;
      if constexpr (kFmt == MSA_KV_FP8_E4M3) {
        ratio = v_cur > 0.0f ? v_cur / rd.vps[j] : 1.0f;   // keep O in units of this page's scale
        v_cur = rd.vps[j];
      }
      // ---- scores of 32 tokens for 16 heads
      float4_t acc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        acc[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          acc[u] = mfma16x16x32(dequant8<kFmt>(rd.R[j].k, ksc, u, kk), Qop[kk], acc[u]);
      }
      // ---- V chunk to LDS (natural [token][d] layout, fp16). It does not depend on the
      // scores, so its dequantisation runs while the matrix core computes them. (A wave's
      // LDS accesses execute in order, so the transposing reads below see these writes
      // without a wait; the empty asm only keeps the compiler from reordering them.)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          *reinterpret_cast<half8_t*>(vb + (16 * u + n) * kVRowHalves + 32 * q + 8 * kk) =
              dequant8<kFmt>(rd.R[j].v, vsc, u, kk);
      asm volatile("" ::: "memory");
      float x[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[u][i] = (16 * u + 4 * q + i) < rd.nvis[j] ? acc[u][i] * cs : -INFINITY;
      // ---- online softmax (per lane: one head)
      float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_raw(m_run - m_new);
      float psum = 0.0f;
      half8_t Pt;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2_raw(x[u][i] - m_new);
          psum += p;
          Pt[4 * u + i] = static_cast<half_t>(p);
        }
      if (m_run != -INFINITY) {                         // O is still zero on a wave's first chunk
        const float ao = alpha * ratio;
#pragma unroll
        for (int d = 0; d < 8; ++d) O[d] *= ao;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      // ---- O^T += V^T . P^T
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const half_t* p0 = vb + (4 * q + (n >> 2)) * kVRowHalves + 16 * d + 4 * (n & 3);
        const half_t* p1 = p0 + 16 * kVRowHalves;
        const half4_t h0 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0)));
        const half4_t h1 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1)));
        const half8_t Vt = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        O[d] = mfma16x16x32(Vt, Pt, O[d]);
      }
      asm volatile("" ::: "memory");   // (the next chunk's V writes stay behind these reads)
    }
  }

  // ---- merge the waves of the workgroup, write this split's partial
  const float l_tot = rows_sum(l_run);
  float oscale;
  if constexpr (kFmt == MSA_KV_NVFP4) oscale = a.v_t; else oscale = v_cur;
  {
    // (the lane's head and dim quarter again, from the hardware lane count: otherwise
    // the compiler keeps the lane index live across the loop, and in the 16-wave
    // variants, at 128 registers, spills it to scratch and reloads it here)
    const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int ne = lane_e & 15, qe = lane_e >> 4;
    // each wave's O tile goes to its own V buffer, which only it used: no barrier first
    float* ob = reinterpret_cast<float*>(dyn_lds + wave * kVBufBytes);   // [16 heads][kORowFloats]
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4_t*>(ob + ne * kORowFloats + 16 * d + 4 * qe) = O[d] * oscale;
    if (qe == 0) { mbuf[wave][ne] = m_run; lbuf[wave][ne] = l_tot; }
  }
  if constexpr (kStep)
    if (threadIdx.x == 0) s_rlast = reader_old == st.readers - 1;
  __syncthreads();
  if constexpr (kStep) {
    // The row's last reader: every reader of the row is past its score reads, so its
    // exchange words go back to idle (and its reader count to zero) for the next launch.
    if (s_rlast) {
      const int nbr = min(pos / kPage + 1, a.max_blocks);
      float* xr = st.sc.xscores + trow * a.max_blocks;
      for (int b = threadIdx.x; b < nbr; b += 64 * kW)
        __hip_atomic_store(xr + b, __uint_as_float(MSA_MERGE_IDLE_BITS), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      if (threadIdx.x == 0) __hip_atomic_store(st.words + r, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  // this (row, KV head)'s partials: O [16 heads][S][128], (m, l) [16 heads][S][2]
  const uint32_t o_bytes = 16u * a.num_splits * kHeadDim * 4, ml_bytes = 16u * a.num_splits * 8;
  const int cur = merging ? static_cast<int>(mstate >> 31) : 0;   // this launch's exchange buffer
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(uniform_ptr(part_o + (2 * head0 + 16 * cur) * a.num_splits * kHeadDim), o_bytes);
  const __amdgpu_buffer_rsrc_t rm =
      make_rsrc(uniform_ptr(part_ml + (2 * head0 + 16 * cur) * a.num_splits * 2), ml_bytes);
  constexpr int kTasks = 16 * (kHeadDim / 4);                     // (head, 4 dims) items
  // (a merger's slice, at most 8 heads, is at most 4 floats per thread)
  static_assert(kOut != kOutMerged || kW >= 4, "merging needs 256 threads");
  constexpr int kPer = (kTasks + 64 * kW - 1) / (64 * kW);        // items per thread
  // In-workgroup merge of one item over the waves' O tiles. Every LDS read is issued
  // before the first use, so their latencies overlap.
  auto wg_merge = [&](int h, int d4, float4_t& acc, float& M, float& l) {
    float mw[kW], lw[kW];
    float4_t tw[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      mw[w] = mbuf[w][h];
      lw[w] = lbuf[w][h];
      tw[w] = *reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(dyn_lds + w * kVBufBytes) +
                                                 h * kORowFloats + 4 * d4);
    }
    M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, mw[w]);
    acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float wt = exp2_raw(mw[w] - M);
        acc += wt * tw[w];
        l += wt * lw[w];
      }
    }
  };
  if constexpr (kOut == kOutPartials) {
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int idx = threadIdx.x + it * 64 * kW;
      if (idx >= kTasks) break;
      const int h = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      float4_t acc;
      float M, l;
      wg_merge(h, d4, acc, M, l);
      // (through the argument pointers, which the compiler knows to be global memory)
      float* po = a.part_o + ((head0 + h) * a.num_splits + s) * kHeadDim + 4 * d4;
      float* pm = a.part_ml + ((head0 + h) * a.num_splits + s) * 2;
      *reinterpret_cast<float4_t*>(po) = acc;
      if (d4 == 0) {
        pm[0] = M;
        pm[1] = l;
      }
    }
  } else if constexpr (kOut == kOutDirect) {
    // the only split: its merge is the output (merge weight exp2(0) = 1)
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      const int idx = threadIdx.x + it * 64 * kW;
      if (idx >= kTasks) break;
      const int h = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      float4_t acc;
      float M, l;
      wg_merge(h, d4, acc, M, l);
      uint16_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = l > 0.0f ? f32_to_bf16_rne(acc[i] / l) : 0;
      *reinterpret_cast<uint2*>(a.out + (head0 + h) * kHeadDim + 4 * d4) =
          make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
    }
  } else {
    // ---- several splits: the last K = merge_slices(S) splits of this (row, KV head) to
    // count themselves in merge them, each a slice of 16 / K heads. Each split counts
    // itself in as soon as its compute is done, then stores its partial (agent-coherent)
    // into this launch's exchange buffer and only then reads the old count, so nothing
    // waits for the stores to land; a merger polls each slot of its slice until none of
    // its words holds the idle pattern. The last split waits only for splits that have
    // counted themselves in, which are resident with only in-workgroup work left before
    // their stores: its polls end. The other mergers may wait for splits that have not
    // counted themselves in yet, so their polls are bounded by helper_poll_limit, after
    // which they hand their slice to the last split (merge_handoff) or, if it has arrived
    // meanwhile, poll on under the last split's bound. Every slice is merged by exactly
    // one workgroup with msa_combine's arithmetic. The mergers leave the slots as they
    // are (each split returns its own slot to idle early in the next launch that uses
    // the other buffer), and the last split flips the state word to the other buffer
    // with no arrivals and no handoffs.
    if (!merge_state_ok(mstate, a.num_splits)) {
      // The workspace was not set up for this split count (or not set up): touch
      // nothing and make the failure visible in the output (bf16 NaN).
      if (s == 0)
        for (int idx = threadIdx.x; idx < kTasks; idx += 64 * kW)
          *reinterpret_cast<uint2*>(a.out + (head0 + idx / (kHeadDim / 4)) * kHeadDim + 4 * (idx % (kHeadDim / 4))) =
              make_uint2(0x7fc07fc0u, 0x7fc07fc0u);
      return;
    }
    int32_t* const word = a.counters + static_cast<int64_t>(r) * a.hkv + g;
    int32_t arrival = 0;   // the old state word; its low byte counts the earlier splits
    if (threadIdx.x == 0) arrival = atomicAdd(word, 1);
#pragma unroll
    for (int it = 0; it < kPer; ++it) {
      // threads past the last item repeat an item (same values, same addresses), so no
      // thread skips the stores
      const int idx = (threadIdx.x + it * 64 * kW) % kTasks;
      const int h = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      float4_t acc;
      float M, l;
      wg_merge(h, d4, acc, M, l);
      store_coherent(ro, ((h * a.num_splits + s) * kHeadDim + 4 * d4) * 4u,
                     float4_t{not_idle(acc[0]), not_idle(acc[1]), not_idle(acc[2]), not_idle(acc[3])});
      // (m, l) from all 32 threads of the head (same value): with no branch anywhere
      // here, the number of stores issued after the count is fixed and reading the count
      // does not wait for them
      store_coherent(rm, (h * a.num_splits + s) * 8u, float2_t{not_idle(M), not_idle(l)});
    }
    // (the empty asm keeps the compiler from folding the use into the atomic's block,
    // where it would wait for the count before the stores above are issued)
    asm volatile("" : "+v"(arrival));
    if (threadIdx.x == 0) s_word = arrival;
    lds_barrier();
    const uint32_t w0 = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(s_word));
    const int S = a.num_splits, K = merge_slices(S);
    const int slice0 = static_cast<int>(w0 & kMergeArrivalMask) - (S - K);
    if (slice0 < 0) return;
    const bool last = slice0 == K - 1;
    // slices this workgroup merges: its own, and (the last split) every handed-over one
    uint32_t todo = 1u << slice0;
    if (last) todo |= (w0 >> kMergeHandoffShift) & ((1u << (K - 1)) - 1u);
    const int slice_floats = (16 / K) * kHeadDim;
    // floats per thread: 1, 2 or 4, whichever lets every thread's loads go out at once
    const int per = min(4, max(1, slice_floats / (64 * kW)));
    const bool active = static_cast<int>(threadIdx.x) * per < slice_floats;
    auto merge_into = [&](auto kv, int slice, int limit, bool helper) -> bool {
      constexpr int kV = decltype(kv)::value;
      const int e = slice * slice_floats + min(static_cast<int>(threadIdx.x) * kV, slice_floats - kV);
      const int h = e / kHeadDim, d = e % kHeadDim;
      float num[kV], den;
      bool ok = active ? merge_slots_any<kV>(ro, rm, S, h, d, limit, num, den) : true;
      if (helper && !__syncthreads_and(ok)) {
        // some word of the slice is still idle: hand the slice over, or, if the last
        // split has arrived in the meantime, wait for it under that split's bound
        if (threadIdx.x == 0) s_word = merge_handoff(word, mstate >> 31, S, slice);
        __syncthreads();
        if (s_word) return true;
        if (!ok) ok = merge_slots_any<kV>(ro, rm, S, h, d, a.poll_limit, num, den);
      }
      if (!active) return true;
      uint16_t o[kV];
#pragma unroll
      for (int i = 0; i < kV; ++i) o[i] = ok ? (den > 0.0f ? f32_to_bf16_rne(num[i] / den) : 0) : 0x7fc0;
      uint16_t* dst = a.out + (head0 + h) * kHeadDim + d;
      if constexpr (kV == 4)
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
      else if constexpr (kV == 2)
        *reinterpret_cast<uint32_t*>(dst) = o[0] | (static_cast<uint32_t>(o[1]) << 16);
      else
        *dst = o[0];
      return ok;
    };
    bool all_ok = true;
    while (todo != 0u) {
      const int slice = __builtin_ctz(todo);
      todo &= todo - 1u;
      const int limit = last ? a.poll_limit : min(a.poll_limit, a.helper_poll_limit);
      if (per == 4) all_ok &= merge_into(std::integral_constant<int, 4>{}, slice, limit, !last);
      else if (per == 2) all_ok &= merge_into(std::integral_constant<int, 2>{}, slice, limit, !last);
      else all_ok &= merge_into(std::integral_constant<int, 1>{}, slice, limit, !last);
    }
    if (!all_ok) {
      // gave up waiting: NaN outputs (written above), and the pair's state word stays
      // invalid until the workspace is set up again (an OR that commutes with the flip)
      dcheck(false, MSA_DEBUG_MERGE_TIMEOUT, a.err);
      __hip_atomic_fetch_or(word, static_cast<int32_t>(kMergeTimeoutBit), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // The last split: the other buffer, no arrivals, no handoffs: ready for the next
    // launch. All S arrivals have been counted and no handoff can follow the last one,
    // so one XOR flips the buffer bit, clears the arrivals and the handoff bits it saw,
    // and leaves any timeout bit in place.
    if (last && threadIdx.x == 0)
      __hip_atomic_fetch_xor(word,
                             static_cast<int32_t>((1u << 31) | static_cast<uint32_t>(S) |
                                                  (w0 & kMergeHandoffMask)),
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <int kFmt, int kW, int kItems, int kOut, int kSelect, bool kStep = false>
void launch(const DecodeArgs& a, dim3 grid, hipStream_t s, const StepArgs& st = StepArgs{}) {
  size_t lds = static_cast<size_t>(kW) * kVBufBytes;
  if (kSelect) lds = std::max({lds, static_cast<size_t>(a.max_blocks) * sizeof(uint32_t), sizeof(MultiSelectSmem)});
  sparse_decode_kernel<kFmt, kW, kItems, kOut, kSelect, kStep><<<grid, dim3(64 * kW), lds, s>>>(a, st);
}

// Waves per workgroup for a split of `per_split` pages, one chunk per wave and round:
// 4 waves for one page, 8 for two. Longer splits take rounds of 8 chunks, which keeps
// the registers low enough for two workgroups per compute unit where the variant
// allows, or, with one split, of 16 chunks (one round for up to four pages, or more
// waves per compute unit when the launch has fewer workgroups than the 256 compute
// units); with several splits 16 waves would leave the merging variant 128 registers
// and make it spill. Several chunks per wave and round measured slower: fewer waves
// hide less of each chunk's latency. The choice depends only on k, the split count and
// the launch size, so every output variant of a call shape computes its partials in
// the same order (the merged and direct outputs equal the partials + msa_combine bit
// for bit). The selecting variant needs at least 4 waves (its selection uses 256
// threads or more).
int decode_waves(const DecodeArgs& a, dim3 grid) {
  const int per_split = (a.k + a.num_splits - 1) / a.num_splits;
  const int chunks = 4 * per_split;
  const bool rounds16 = a.num_splits == 1 && (chunks <= 16 || static_cast<int64_t>(grid.x) * grid.y < 256);
  return chunks <= 4 ? 4 : chunks <= 8 ? 8 : rounds16 ? 16 : 8;
}

template <int kFmt, int kOut, int kSelect>
msa_status_t dispatch(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  switch (decode_waves(a, grid)) {
    case 4: launch<kFmt, 4, 1, kOut, kSelect>(a, grid, s); break;
    case 8: launch<kFmt, 8, 1, kOut, kSelect>(a, grid, s); break;   // (rounds of 8 chunks past 8)
    default:
      if constexpr (kOut != kOutMerged) launch<kFmt, 16, 1, kOut, kSelect>(a, grid, s);
      else return MSA_ERR_UNSUPPORTED;   // (never: one split writes its output directly)
  }
  return launch_status();
}

// Shape of the two-level selection for a launch of `waves` waves: the fewest keys per
// lane (1, 2, 4 or 8) for which ceil(C / 64 kR) first-level waves fit in the workgroup
// (and in 8) and their picks (nw * want) fit one wave at kR keys per lane. kR = 0: the
// row is too long for it (the block radix select runs).
void select_shape(int c_max, int want, int waves, int& kR, int& nw) {
  for (kR = 1; kR <= 8; kR *= 2) {
    nw = std::max(1, (c_max + 64 * kR - 1) / (64 * kR));
    if (nw <= std::min(waves, 8) && nw * std::max(want, 0) <= 64 * kR) return;
  }
  kR = 0;
  nw = 0;
}

// Host checks and arguments common to every decode entry; `grid` receives the launch
// grid. Returns MSA_OK with a.num_rows == 0 for an empty step (nothing to launch).
msa_status_t prepare_decode(const msa_kv_pool_t* pool, const msa_step_t* step, int32_t num_q_heads,
                            const void* q, DecodeArgs& a, bool combine, bool select, dim3& grid) {
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (num_q_heads != MSA_HEADS_PER_KV * pool->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  if (a.k < 1 || a.k > MSA_MAX_TOPK || a.num_splits < 1 || a.num_splits > a.k) return MSA_ERR_UNSUPPORTED;
  if (combine && a.num_splits > kMaxMergeSplits) return MSA_ERR_UNSUPPORTED;
  if (select && (a.n_init < 0 || a.n_local < 0 || a.n_init + a.n_local > a.k)) return MSA_ERR_UNSUPPORTED;
  if (!(a.softmax_scale > 0.0f)) return MSA_ERR_INVALID_ARG;
  a.sel_tables = sel_tables(step);
  if (a.sel_tables != 1 && a.sel_tables != pool->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  a.num_rows = step->num_rows;
  if (step->num_rows == 0) return MSA_OK;
  if (q == nullptr || a.part_o == nullptr || a.part_ml == nullptr) return MSA_ERR_INVALID_ARG;
  if (select ? a.scores == nullptr : a.sel == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(a.part_o) || (reinterpret_cast<uintptr_t>(a.part_ml) & 7u))
    return MSA_ERR_INVALID_ARG;
  if (combine && (a.counters == nullptr || a.out == nullptr || (reinterpret_cast<uintptr_t>(a.out) & 7u)))
    return MSA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(step->num_rows) * pool->num_kv_heads > 65535) return MSA_ERR_UNSUPPORTED;
  a.k_codes = static_cast<const uint8_t*>(pool->k_codes);
  a.v_codes = static_cast<const uint8_t*>(pool->v_codes);
  a.k_scales = static_cast<const uint8_t*>(pool->k_scales);
  a.v_scales = static_cast<const uint8_t*>(pool->v_scales);
  a.k_t = pool->k_tensor_scale;
  a.v_t = pool->v_tensor_scale;
  a.hkv = pool->num_kv_heads;
  a.block_table = step->block_table;
  a.row_seq = step->row_seq;
  a.num_seqs = step->num_seqs;
  a.num_pages = pool->num_pages;
  a.err = debug_error_word();
  a.poll_limit = merge_poll_limit();
  a.helper_poll_limit = merge_helper_poll_limit();
  a.row_pos = step->row_pos;
  a.max_blocks = step->max_blocks_per_seq;
  a.q = static_cast<const uint16_t*>(q);
  a.seq_mul = seq_guess_mul(step->num_seqs, step->num_rows);
  grid = dim3(a.num_splits, step->num_rows * pool->num_kv_heads);
  return MSA_OK;
}

msa_status_t decode_entry(const msa_kv_pool_t* pool, const msa_step_t* step, int32_t num_q_heads,
                          const void* q, DecodeArgs a, hipStream_t s, bool combine, bool select) {
  dim3 grid;
  const msa_status_t st = prepare_decode(pool, step, num_q_heads, q, a, combine, select, grid);
  if (st != MSA_OK || a.num_rows == 0) return st;
  const bool direct = a.num_splits == 1;
  int kr = 0;
  if (select) select_shape(a.max_blocks - a.n_init - a.n_local, a.k - a.n_init - a.n_local, decode_waves(a, grid),
                           kr, a.sel_waves);
  // (rows too long for the two-level selection take the block radix select, in the
  // 8-keys-per-lane instance of the kernel)
#define MSA_DECODE_SELECT(FMT, OUT)                                                                    \
  (kr == 1 ? (a.sel_waves == 1 ? dispatch<FMT, OUT, kSelectOneWave>(a, grid, s) : dispatch<FMT, OUT, 1>(a, grid, s)) \
   : kr == 2 ? dispatch<FMT, OUT, 2>(a, grid, s)                                                       \
   : kr == 4 ? dispatch<FMT, OUT, 4>(a, grid, s) : dispatch<FMT, OUT, 8>(a, grid, s))
#define MSA_DECODE_DISPATCH(FMT)                                                                       \
  (select ? (direct ? MSA_DECODE_SELECT(FMT, kOutDirect) : MSA_DECODE_SELECT(FMT, kOutMerged))        \
   : combine ? (direct ? dispatch<FMT, kOutDirect, 0>(a, grid, s) : dispatch<FMT, kOutMerged, 0>(a, grid, s)) \
             : dispatch<FMT, kOutPartials, 0>(a, grid, s))
  if (pool->fmt == MSA_KV_NVFP4) return MSA_DECODE_DISPATCH(MSA_KV_NVFP4);
  return MSA_DECODE_DISPATCH(MSA_KV_FP8_E4M3);
#undef MSA_DECODE_DISPATCH
#undef MSA_DECODE_SELECT
}

template <int kFmt, int kOut, int kSelect>
msa_status_t dispatch_step(const DecodeArgs& a, const StepArgs& st, dim3 grid, int waves, hipStream_t s) {
  if (waves == 4) launch<kFmt, 4, 1, kOut, kSelect, true>(a, grid, s, st);
  else launch<kFmt, 8, 1, kOut, kSelect, true>(a, grid, s, st);
  return launch_status();
}

DecodeArgs base_args(const int32_t* sel, const int32_t* sel_pages, int32_t k, float softmax_scale,
                     int32_t num_splits, float* part_o, float* part_ml) {
  DecodeArgs a{};
  a.sel = sel;
  a.sel_pages = sel_pages;
  a.k = k;
  a.softmax_scale = softmax_scale;
  a.num_splits = num_splits;
  a.part_o = part_o;
  a.part_ml = part_ml;
  return a;
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_sparse_decode(const msa_kv_pool_t* pool, const msa_step_t* step,
                                          int32_t num_q_heads, const void* q, const int32_t* sel,
                                          const int32_t* sel_pages, int32_t k, float softmax_scale,
                                          int32_t num_splits, float* part_o, float* part_ml,
                                          void* stream) {
  using namespace msa;
  DecodeArgs a = base_args(sel, sel_pages, k, softmax_scale, num_splits, part_o, part_ml);
  return decode_entry(pool, step, num_q_heads, q, a, static_cast<hipStream_t>(stream), false, false);
}

extern "C" msa_status_t msa_sparse_decode_combine(const msa_kv_pool_t* pool, const msa_step_t* step,
                                                  int32_t num_q_heads, const void* q,
                                                  const int32_t* sel, const int32_t* sel_pages,
                                                  int32_t k, float softmax_scale, int32_t num_splits,
                                                  float* part_o, float* part_ml, int32_t* counters,
                                                  void* out, void* stream) {
  using namespace msa;
  if (counters == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  DecodeArgs a = base_args(sel, sel_pages, k, softmax_scale, num_splits, part_o, part_ml);
  a.counters = counters;
  a.out = static_cast<uint16_t*>(out);
  return decode_entry(pool, step, num_q_heads, q, a, static_cast<hipStream_t>(stream), true, false);
}

extern "C" msa_status_t msa_select_decode_combine(
    const msa_kv_pool_t* pool, const msa_step_t* step, int32_t num_q_heads, const void* q,
    const float* block_scores, int32_t k, int32_t n_init, int32_t n_local, float softmax_scale,
    int32_t num_splits, float* part_o, float* part_ml, int32_t* counters, void* out, int32_t* sel,
    int32_t* sel_pages, void* stream) {
  using namespace msa;
  if (counters == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  DecodeArgs a = base_args(nullptr, nullptr, k, softmax_scale, num_splits, part_o, part_ml);
  a.scores = block_scores;
  a.n_init = n_init;
  a.n_local = n_local;
  a.sel_out = sel;
  a.sel_pages_out = sel_pages;
  a.counters = counters;
  a.out = static_cast<uint16_t*>(out);
  return decode_entry(pool, step, num_q_heads, q, a, static_cast<hipStream_t>(stream), true, true);
}

extern "C" msa_status_t msa_decode_step(
    const msa_kv_pool_t* pool, const msa_step_t* step, int32_t n_new, const int64_t* slot, const void* k_new,
    const void* v_new, const void* idx_k_new, int32_t n_idx_heads, const void* q_idx, const float* w,
    int32_t num_q_heads, const void* q, int32_t k, int32_t n_init, int32_t n_local, float softmax_scale,
    int32_t num_splits, float* score_x, int32_t* score_words, float* part_o, float* part_ml, int32_t* counters,
    void* out, float* block_scores, int32_t* sel, int32_t* sel_pages, void* stream) {
  using namespace msa;
  if (counters == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (n_new < 0) return MSA_ERR_INVALID_ARG;
  DecodeArgs a = base_args(nullptr, nullptr, k, softmax_scale, num_splits, part_o, part_ml);
  a.scores = score_x;   // (checked as the selection's input)
  a.n_init = n_init;
  a.n_local = n_local;
  a.sel_out = sel;
  a.sel_pages_out = sel_pages;
  a.counters = counters;
  a.out = static_cast<uint16_t*>(out);
  dim3 grid;
  msa_status_t st = prepare_decode(pool, step, num_q_heads, q, a, true, true, grid);
  if (st != MSA_OK) return st;
  if (n_new > 0 && slot == nullptr) return MSA_ERR_INVALID_ARG;
  for (const void* p : {k_new, v_new, idx_k_new})
    if (p != nullptr && !aligned16(p)) return MSA_ERR_INVALID_ARG;
  if (step->num_rows == 0) {
    return n_new > 0 ? msa_kv_append(pool, n_new, slot, k_new, v_new, idx_k_new, stream) : MSA_OK;
  }
  // the single-launch contract: 4 index heads, E4M3 keys, one table per row, a stated
  // row count per request, at most 64 new tokens
  if (n_idx_heads != kStepHi || index_nvfp4(pool) || a.sel_tables != 1 || step->rows_per_seq <= 0 || n_new > 64)
    return MSA_ERR_UNSUPPORTED;
  if (q_idx == nullptr || w == nullptr || score_words == nullptr || !aligned16(q_idx)) return MSA_ERR_INVALID_ARG;
  const int waves = decode_waves(a, grid);
  int kr = 0;
  select_shape(a.max_blocks - a.n_init - a.n_local, a.k - a.n_init - a.n_local, waves, kr, a.sel_waves);
  // Workgroup and selection shapes of the single launch, and at most two scoring blocks
  // per wave: a group of rows (16 / 4 index heads = 4 rows of one request) has
  // rows * hkv * num_splits workgroups; the smallest group has R % 4 rows (4 if R is a
  // multiple of 4), and max_blocks must be at most twice its waves. A group waits only
  // on its own workgroups, which must fit on the GPU at once (at most 256 workgroups,
  // one per compute unit).
  constexpr int kRpg = 16 / kStepHi;
  const int R = step->rows_per_seq;
  const int64_t per_row = static_cast<int64_t>(a.hkv) * a.num_splits;
  const int64_t small_waves = (R % kRpg == 0 ? kRpg : R % kRpg) * per_row * waves;
  if ((waves != 4 && waves != 8) || (kr != 1 && kr != 2) || a.max_blocks > 2 * small_waves ||
      std::min(R, kRpg) * per_row > 256)
    return MSA_ERR_UNSUPPORTED;
  StepArgs sa{};
  sa.sc.index_k = static_cast<const uint8_t*>(pool->index_k);
  sa.sc.q_idx = static_cast<const uint16_t*>(q_idx);
  sa.sc.w = w;
  sa.sc.idx_new = static_cast<const uint16_t*>(idx_k_new);
  sa.sc.xscores = score_x;
  sa.sc.scores_out = block_scores;
  sa.words = score_words;
  sa.rows_per_seq = R;
  sa.readers = static_cast<int>(per_row);
  sa.app = make_append_args(pool, n_new, slot, k_new, v_new, idx_k_new);
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const bool direct = a.num_splits == 1;
#define MSA_STEP_DISPATCH(FMT)                                                                              \
  (direct ? (kr == 1 ? dispatch_step<FMT, kOutDirect, 1>(a, sa, grid, waves, hs)                           \
                     : dispatch_step<FMT, kOutDirect, 2>(a, sa, grid, waves, hs))                          \
          : (kr == 1 ? dispatch_step<FMT, kOutMerged, 1>(a, sa, grid, waves, hs)                           \
                     : dispatch_step<FMT, kOutMerged, 2>(a, sa, grid, waves, hs)))
  if (pool->fmt == MSA_KV_NVFP4) return MSA_STEP_DISPATCH(MSA_KV_NVFP4);
  return MSA_STEP_DISPATCH(MSA_KV_FP8_E4M3);
#undef MSA_STEP_DISPATCH
}
