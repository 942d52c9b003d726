// Index-scoring building blocks shared by the scoring kernels (index_score.hip) and
// the single-launch step (sparse_decode.hip): the MFMA operands of index keys, the
// encoding of a new token's key, and the step's per-wave block scorer.
//
// The score of token p for a query row ([GB300] "The TP4 decode target": an index
// scorer over index-K pages; [Rubin] commit messages: a proxy max-score pass with one
// score per block) is s_p = sum_h w_h * relu(q_h . key_p), and a block's score is the
// maximum over its visible tokens. The contraction [128 tokens x 64] . [64 x (rows *
// heads)] runs on the matrix cores with fp16 operands (E4M3 keys convert exactly; bf16
// queries are pre-scaled by a power of two per (row, head)) and fp32 accumulation;
// lane (n, q) of the result holds every head of row-slot q for token n, so the head sum
// is in-lane, in a fixed order that does not depend on the token's position.
#pragma once

#include "append_device.h"
#include "msa_device.h"

namespace msa {

// A lane's share of one 16-token row of keys (token 16t + n, dims 16q .. 16q+15):
// E4M3 keys: 16 codes. NVFP4 keys: .x, .y = 16 E2M1 codes (element 2j in the low
// nibble of byte j), .z = the group's E4M3 scale code.
template <bool kIdxNv>
__device__ __forceinline__ void key_operands(uint4 kt, half8_t& B0, half8_t& B1) {
  if constexpr (kIdxNv) {
    const half2_t s2 = e4m3x2_to_f16(kt.z);
    const half2_t sc2 = {s2[0], s2[0]};
    B0 = e2m1x8_to_f16(kt.x, sc2);
    B1 = e2m1x8_to_f16(kt.y, sc2);
  } else {
    B0 = e4m3x8_to_f16(kt.x, kt.y);
    B1 = e4m3x8_to_f16(kt.z, kt.w);
  }
}

// The same share of a new token's key, encoded from its 16 bf16 values.
template <bool kIdxNv>
__device__ __forceinline__ uint4 encode_key16(uint4 lo, uint4 hi, float idx_t) {
  if constexpr (kIdxNv) {
    uint32_t w0, w1;
    const uint32_t sc = nvfp4_encode16_bits(lo, hi, idx_t, w0, w1);
    return make_uint4(w0, w1, sc, 0u);
  } else {
    return encode_index16_bits(lo, hi);
  }
}

// Inputs of the single-launch step's scorer (E4M3 index keys).
struct StepScoreArgs {
  const uint8_t* index_k;    // E4M3 [pages][128][64]
  const uint16_t* q_idx;     // bf16 [rows][heads][64]
  const float* w;            // [rows][heads]
  const uint16_t* idx_new;   // bf16 [n_new][64], or null: no new key
  float* xscores;            // exchange [rows][max_blocks]: idle (MSA_MERGE_IDLE_BITS) until written
  float* scores_out;         // optional [rows][max_blocks], as msa_index_score writes them
};

// One wave of the single-launch step scores up to kNB blocks b[j] (b[j] >= max_blocks:
// none) of one group of rows: rows r0 .. r0 + nr - 1 (nr <= 16 / kHi) of request seq.
// Every key load of the wave's blocks is issued before the first MFMA. A new token
// landing in a scored page (slot0: lane i < 64 holds new token i's slot, else -1) has
// its key encoded here from the bf16 source instead of read from the pool, whose
// append runs in the same launch. The score of a visible block of a row (b <= row_pos /
// 128) goes to the exchange agent-coherently (its readers are other workgroups of the
// launch) and, like every other block's, to scores_out if given: a block past a row's
// last visible token scores -inf for that row, as msa_index_score defines it. Returns
// the page of the last visible block of row r0 + self (read once the key loads are out).
template <int kHi, int kNB>
__device__ __forceinline__ int32_t score_blocks(const StepScoreArgs& sa, const int32_t* block_table,
                                                const int32_t* row_pos, int max_blocks, int num_pages, int32_t* err,
                                                int r0, int nr, int seq, const int (&b)[kNB], int64_t slot0, int self) {
  constexpr int kRowsPerLane = 4 / kHi;
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  // the blocks' pages (entries past the table read its last entry, unused), then the
  // rows' positions and the query side, all in one round of loads
  const int32_t* btr = block_table + static_cast<int64_t>(seq) * max_blocks;
  int32_t page32[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) page32[j] = btr[min(b[j], max_blocks - 1)];
  const int pl = row_pos[r0 + min(lane, nr - 1)];
  // A operand: lane (m, q) holds row-slot m / kHi, head m % kHi, dims 16q + 8ks .. +7
  const int rs = n / kHi, hd = n % kHi;
  uint4 qa0 = make_uint4(0u, 0u, 0u, 0u), qa1 = qa0;
  if (rs < nr) {
    const uint16_t* qp = sa.q_idx + (static_cast<int64_t>(r0 + rs) * kHi + hd) * kIndexDim + 16 * q;
    qa0 = reinterpret_cast<const uint4*>(qp)[0];
    qa1 = reinterpret_cast<const uint4*>(qp)[1];
  }
  // after the MFMA, lane (n, q) holds M = 4q + jj: the matching (row, head) weight
  float wj[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int mm = 4 * q + jj;
    const int rr = mm / kHi, hh = mm % kHi;
    wj[jj] = rr < nr ? sa.w[static_cast<int64_t>(r0 + rr) * kHi + hh] : 0.0f;
  }
  int64_t page[kNB];
#pragma unroll
  for (int j = 0; j < kNB; ++j) page[j] = b[j] < max_blocks ? page32[j] : -1;
  int max_pos = pl;
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) max_pos = max(max_pos, __shfl_xor(max_pos, m, 64));
  const int last_block = max_pos / kPage;
  int rowslot[kRowsPerLane], pos[kRowsPerLane];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) {
    rowslot[i] = q * kRowsPerLane + i;
    pos[i] = rowslot[i] < nr ? __shfl(pl, rowslot[i], 64) : -1;
  }

  // Key loads through a buffer resource per block, of zero bytes for a block that is
  // not scored (its loads then return zeros without a memory access): no branch around
  // any load, so all of them go out back to back.
  bool act[kNB];
  uint4 key[kNB][8];
#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    act[j] = b[j] < max_blocks && b[j] <= last_block;
    int64_t pg = act[j] ? checked_page(page[j], num_pages, err) : 0;
    if (pg < 0) pg = 0;   // (an entry of -1 here is invalid input: read page 0, not before the pool)
    pg = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(pg))));
    const __amdgpu_buffer_rsrc_t kr =
        make_rsrc(uniform_ptr(sa.index_k + pg * kPage * kIndexDim), act[j] ? kPage * kIndexDim : 0u);
#pragma unroll
    for (int t = 0; t < 8; ++t)
      key[j][t] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(kr, static_cast<int>((16 * t + n) * kIndexDim + 16 * q), 0,
                                                       kStreamPolicy));
  }
  // the page of row r0 + self's last visible block (its load queues behind the keys')
  const int32_t self_last_page = btr[min(__shfl(pl, self, 64) / kPage, max_blocks - 1)];
  // new tokens landing in a scored page: their keys from the bf16 source
  if (sa.idx_new != nullptr) {
#pragma unroll
    for (int j = 0; j < kNB; ++j) {
      if (!act[j]) continue;
      uint64_t hits = __ballot(slot0 >= 0 && slot0 / kPage == page[j]);
      while (hits != 0u) {
        const int i = __ffsll(static_cast<unsigned long long>(hits)) - 1;
        hits &= hits - 1;
        const int off = __builtin_amdgcn_readlane(static_cast<int>(slot0 % kPage), i);
        if ((off & 15) == n) {
          const uint4* src = reinterpret_cast<const uint4*>(sa.idx_new + static_cast<int64_t>(i) * kIndexDim + 16 * q);
          const uint4 v = encode_key16<false>(src[0], src[1], 1.0f);
#pragma unroll
          for (int t = 0; t < 8; ++t)
            if (t == (off >> 4)) key[j][t] = v;
        }
      }
    }
  }

  // the query operand, exact in fp16 after a power-of-two scale per (row, head)
  float qa[16];
  bf16x16_to_f32(qa0, qa1, qa);
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(qa[i]));
  amax = rows_max(amax);
  const int e = f16_prescale_exp(amax);
  half8_t A0, A1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A0[i] = static_cast<half_t>(ldexpf(qa[i], e));
    A1[i] = static_cast<half_t>(ldexpf(qa[8 + i], e));
  }
  // head weight times the inverse pre-scale of the (row, head) of result M = 4q + jj:
  // the scale is a positive power of two, so w * relu(x * inv) = (w * inv) * relu(x)
  float wi[4];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) wi[jj] = wj[jj] * ldexpf(1.0f, -__shfl(e, 4 * q + jj, 64));

#pragma unroll
  for (int j = 0; j < kNB; ++j) {
    if (b[j] >= max_blocks) continue;
    if (!act[j]) {   // past every row of the group
      if (sa.scores_out != nullptr && lane < nr)
        sa.scores_out[static_cast<int64_t>(r0 + lane) * max_blocks + b[j]] = -INFINITY;
      continue;
    }
    float best[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) best[i] = -INFINITY;
    // tokens past a row's position are masked only in a block that holds one
    bool ends_here = false;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) ends_here |= rowslot[i] < nr && b[j] * kPage + kPage - 1 > pos[i];
    auto score_tokens = [&](auto masked) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        half8_t B0, B1;
        key_operands<false>(key[j][t], B0, B1);
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = mfma16x16x32(A0, B0, acc);
        acc = mfma16x16x32(A1, B1, acc);
        const int p = b[j] * kPage + 16 * t + n;   // absolute position of this lane's token
#pragma unroll
        for (int i = 0; i < kRowsPerLane; ++i) {
          float s = 0.0f;
#pragma unroll
          for (int hh = 0; hh < kHi; ++hh) s = fmaf(wi[i * kHi + hh], relu_raw(acc[i * kHi + hh]), s);
          if constexpr (decltype(masked)::value) {
            if (p <= pos[i]) best[i] = max_raw(best[i], s);
          } else {
            best[i] = max_raw(best[i], s);
          }
        }
      }
    };
    if (__ballot(ends_here) != 0) score_tokens(std::true_type{});
    else score_tokens(std::false_type{});
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      const float v = row_max_to_first(best[i]);   // the block maximum, in lane n == 0
      if (n == 0 && rowslot[i] < nr) {
        const int64_t at = static_cast<int64_t>(r0 + rowslot[i]) * max_blocks + b[j];
        if (b[j] <= pos[i] / kPage)
          __hip_atomic_store(sa.xscores + at, not_idle(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (sa.scores_out != nullptr) sa.scores_out[at] = v;
      }
    }
  }
  return self_last_page;
}

}  // namespace msa
