// msa_index_score: per-token index score, max-pooled over 128-token blocks.
//
// The scorer streams every visible token's 64-byte E4M3 index key once per request
// ([GB300] "The TP4 decode target": an index scorer reading index-K pages; [Rubin]
// commit messages: a proxy max-score pass producing one score per block). The
// per-block contraction is [128 tokens x 64] . [64 x (rows * heads)], done on the
// matrix cores with fp16 operands (E4M3 keys convert exactly; bf16 queries are
// pre-scaled by a power of two per (row, head) so the conversion is exact) and fp32
// accumulation.
//
// Work split: one wave per (group of rows of one request, block). A group holds up
// to 16 / Hi consecutive rows of the same request, so a request's index keys are read
// once for all of its query rows. MFMA A = queries (M = row * Hi + head), B = keys
// (N = 16 tokens), so lane (n, q) ends up with all heads of row-slot q for token n:
// the head sum is in-lane and its order never depends on the token's position.
#include "msa_device.h"
#include "msa_host.h"

namespace msa {
namespace {

constexpr int kWaves = 4;

template <int kHi>
__global__ void __launch_bounds__(64 * kWaves)
index_score_kernel(const uint8_t* __restrict__ index_k, const int32_t* __restrict__ block_table,
                   const int32_t* __restrict__ row_seq, const int32_t* __restrict__ row_pos,
                   const uint16_t* __restrict__ q_idx, const float* __restrict__ w,
                   float* __restrict__ scores, int num_rows, int max_blocks) {
  constexpr int kRowsPerGroup = 16 / kHi;
  constexpr int kRowsPerLane = 4 / kHi;
  const int r0 = blockIdx.y;
  const int seq = row_seq[r0];
  // Is r0 the first row of a group? Count earlier rows of the same request.
  int j = 0;
  while (r0 - j - 1 >= 0 && row_seq[r0 - j - 1] == seq) ++j;
  if (j % kRowsPerGroup != 0) return;
  int nr = 1;
  while (nr < kRowsPerGroup && r0 + nr < num_rows && row_seq[r0 + nr] == seq) ++nr;

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int b = blockIdx.x * kWaves + wave;
  if (b >= max_blocks) return;
  const int n = lane & 15, q = lane >> 4;

  int max_pos = -1;
  for (int i = 0; i < nr; ++i) max_pos = max(max_pos, row_pos[r0 + i]);
  if (b > max_pos / kPage) {           // past every row's last visible block
    if (lane < nr) scores[static_cast<int64_t>(r0 + lane) * max_blocks + b] = -INFINITY;
    return;
  }
  const int64_t page = block_table[static_cast<int64_t>(seq) * max_blocks + b];

  // Issue all 8 key loads of the block: lane (n, q) reads 16 bytes of token 16t + n,
  // dims 16q .. 16q+15 (k-step 0 uses the first 8, k-step 1 the last 8).
  const uint8_t* kp = index_k + (page * kPage + n) * kIndexDim + 16 * q;
  uint4 key[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) key[t] = *reinterpret_cast<const uint4*>(kp + t * 16 * kIndexDim);

  // A operand: lane (m, q) holds query row-slot m / Hi, head m % Hi, dims
  // 16q + 8ks .. +7, times 2^e (e per (row, head), from the amax over 64 dims).
  const int m = n;
  const int rs = m / kHi, hd = m % kHi;
  float qa[16];
  bool has_row = rs < nr;
  if (has_row) {
    const uint16_t* qp = q_idx + (static_cast<int64_t>(r0 + rs) * kHi + hd) * kIndexDim + 16 * q;
    const uint4 a0 = reinterpret_cast<const uint4*>(qp)[0], a1 = reinterpret_cast<const uint4*>(qp)[1];
    const uint32_t wv[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      qa[2 * i] = __uint_as_float(wv[i] << 16);
      qa[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) qa[i] = 0.0f;
  }
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(qa[i]));
  amax = xor_max(xor_max(amax, 16), 32);
  const int e = f16_prescale_exp(amax);
  half8_t A0, A1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    A0[i] = static_cast<half_t>(ldexpf(qa[i], e));
    A1[i] = static_cast<half_t>(ldexpf(qa[8 + i], e));
  }
  // After the MFMA, lane (n, q) holds M = 4q + jj; fetch the matching (row, head)
  // weight and inverse pre-scale from the lane that owns that M.
  float wj[4], inv[4];
  int rowslot[kRowsPerLane];
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const int mm = 4 * q + jj;
    const int ej = __shfl(e, mm, 64);
    inv[jj] = ldexpf(1.0f, -ej);
    const int rr = mm / kHi, hh = mm % kHi;
    wj[jj] = rr < nr ? w[static_cast<int64_t>(r0 + rr) * kHi + hh] : 0.0f;
  }
  int pos[kRowsPerLane];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) {
    rowslot[i] = q * kRowsPerLane + i;
    pos[i] = rowslot[i] < nr ? row_pos[r0 + rowslot[i]] : -1;
  }

  float best[kRowsPerLane];
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) best[i] = -INFINITY;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const half8_t B0 = e4m3x8_to_f16(key[t].x, key[t].y);
    const half8_t B1 = e4m3x8_to_f16(key[t].z, key[t].w);
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mfma16x16x32(A0, B0, acc);
    acc = mfma16x16x32(A1, B1, acc);
    const int p = b * kPage + 16 * t + n;      // absolute position of this lane's token
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      float s = 0.0f;
#pragma unroll
      for (int hh = 0; hh < kHi; ++hh) {
        const int jj = i * kHi + hh;
        s = fmaf(wj[jj], fmaxf(acc[jj] * inv[jj], 0.0f), s);
      }
      if (p <= pos[i]) best[i] = fmaxf(best[i], s);
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerLane; ++i) {
    float v = best[i];
    v = xor_max(v, 1);
    v = xor_max(v, 2);
    v = xor_max(v, 4);
    v = xor_max(v, 8);
    if (n == 0 && rowslot[i] < nr)
      scores[static_cast<int64_t>(r0 + rowslot[i]) * max_blocks + b] = v;
  }
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_index_score(const msa_kv_pool_t* pool, const msa_step_t* step,
                                        int32_t n_idx_heads, const void* q_idx, const float* w,
                                        float* block_scores, void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (n_idx_heads != 1 && n_idx_heads != 2 && n_idx_heads != 4) return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0) return MSA_OK;
  if (q_idx == nullptr || w == nullptr || block_scores == nullptr || !aligned16(q_idx))
    return MSA_ERR_INVALID_ARG;
  if (step->num_rows > 65535) return MSA_ERR_UNSUPPORTED;
  dim3 grid((step->max_blocks_per_seq + kWaves - 1) / kWaves, step->num_rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto ik = static_cast<const uint8_t*>(pool->index_k);
  auto qi = static_cast<const uint16_t*>(q_idx);
  switch (n_idx_heads) {
    case 1:
      index_score_kernel<1><<<grid, 64 * kWaves, 0, s>>>(ik, step->block_table, step->row_seq,
          step->row_pos, qi, w, block_scores, step->num_rows, step->max_blocks_per_seq);
      break;
    case 2:
      index_score_kernel<2><<<grid, 64 * kWaves, 0, s>>>(ik, step->block_table, step->row_seq,
          step->row_pos, qi, w, block_scores, step->num_rows, step->max_blocks_per_seq);
      break;
    default:
      index_score_kernel<4><<<grid, 64 * kWaves, 0, s>>>(ik, step->block_table, step->row_seq,
          step->row_pos, qi, w, block_scores, step->num_rows, step->max_blocks_per_seq);
  }
  return launch_status();
}
