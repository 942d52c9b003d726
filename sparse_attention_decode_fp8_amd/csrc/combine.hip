// msa_combine: fixed-order log-sum-exp merge of split-KV partials into bf16 outputs.
//
// [Rubin] "Items and numerics", LC_ONEDIV: the long-context sparse-decode split-K merge
// divides once per output, in a fixed order, with no atomics. Each thread owns four
// consecutive output dims of one (row, head); the splits are summed in ascending
// order and each output is one division, rounded once to bf16 (nearest even).
#include <algorithm>

#include "msa_device.h"
#include "msa_host.h"

namespace msa {
namespace {

template <int kS>
__device__ __forceinline__ void combine_item(const float* ml, const float* po, int num_splits, float4_t& num,
                                             float& den) {
  // every split's (m, l) and O first (entries past the last split repeat it, unused),
  // then the sums in ascending split order
  float2_t mls[kS];
  float4_t ot[kS];
#pragma unroll
  for (int t = 0; t < kS; ++t) {
    const int tt = min(t, num_splits - 1);
    mls[t] = *reinterpret_cast<const float2_t*>(ml + 2 * tt);
    ot[t] = *reinterpret_cast<const float4_t*>(po + static_cast<int64_t>(tt) * kHeadDim);
  }
  float M = -INFINITY;
#pragma unroll
  for (int t = 0; t < kS; ++t)
    if (t < num_splits) M = fmaxf(M, mls[t][0]);
  num = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  den = 0.0f;
#pragma unroll
  for (int t = 0; t < kS; ++t) {
    if (t < num_splits) {
      const float m = mls[t][0];
      const float wgt = m == -INFINITY ? 0.0f : exp2_raw(m - M);   // M > -inf whenever m is
      den += wgt * mls[t][1];
      num += wgt * ot[t];
    }
  }
}

__global__ void __launch_bounds__(256)
combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml,
               uint16_t* __restrict__ out, int64_t row_heads, int num_splits) {
  constexpr int kQuads = kHeadDim / 4;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= row_heads * kQuads) return;
  const int64_t rh = idx / kQuads;
  const int d4 = static_cast<int>(idx % kQuads);
  const float* ml = part_ml + rh * num_splits * 2;
  const float* po = part_o + rh * num_splits * kHeadDim + 4 * d4;
  float4_t num;
  float den;
  if (num_splits <= 4) combine_item<4>(ml, po, num_splits, num, den);
  else if (num_splits <= 16) combine_item<16>(ml, po, num_splits, num, den);
  else {   // up to 64 splits: the same sums, loads in a loop
    float M = -INFINITY;
    for (int s = 0; s < num_splits; ++s) M = fmaxf(M, ml[2 * s]);
    num = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    den = 0.0f;
    for (int s = 0; s < num_splits; ++s) {
      const float m = ml[2 * s];
      const float wgt = m == -INFINITY ? 0.0f : exp2_raw(m - M);
      den += wgt * ml[2 * s + 1];
      num += wgt * *reinterpret_cast<const float4_t*>(po + static_cast<int64_t>(s) * kHeadDim);
    }
  }
  uint16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = den > 0.0f ? f32_to_bf16_rne(num[i] / den) : 0;
  *reinterpret_cast<uint2*>(out + rh * kHeadDim + 4 * d4) =
      make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_combine(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                                    int32_t num_splits, const float* part_o, const float* part_ml,
                                    void* out, void* stream) {
  using namespace msa;
  if (rows < 0 || num_q_heads <= 0 || num_splits <= 0) return MSA_ERR_INVALID_ARG;
  if (head_dim != MSA_HEAD_DIM || num_splits > MSA_MAX_TOPK) return MSA_ERR_UNSUPPORTED;
  if (rows == 0) return MSA_OK;
  if (part_o == nullptr || part_ml == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned16(part_o) || (reinterpret_cast<uintptr_t>(out) & 7u) ||
      (reinterpret_cast<uintptr_t>(part_ml) & 7u))
    return MSA_ERR_INVALID_ARG;
  const int64_t rh = static_cast<int64_t>(rows) * num_q_heads;
  const int64_t threads = rh * (MSA_HEAD_DIM / 4);
  combine_kernel<<<dim3(static_cast<unsigned>((threads + 255) / 256)), dim3(256), 0,
                   static_cast<hipStream_t>(stream)>>>(part_o, part_ml, static_cast<uint16_t*>(out),
                                                        rh, num_splits);
  return launch_status();
}

namespace msa {
namespace {

// Initial state of a split-merge workspace: every word of both exchange buffers holds
// the idle pattern, and every pair's state word selects buffer 0 for the given split
// count with no arrivals.
__global__ void __launch_bounds__(256)
merge_idle_kernel(uint32_t* __restrict__ part_o, int64_t n_o, uint32_t* __restrict__ part_ml,
                  int64_t n_ml, int32_t* __restrict__ counters, int64_t n_c, uint32_t state0) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n_o + n_ml + n_c;
       i += stride) {
    if (i < n_o) part_o[i] = MSA_MERGE_IDLE_BITS;
    else if (i < n_o + n_ml) part_ml[i - n_o] = MSA_MERGE_IDLE_BITS;
    else counters[i - n_o - n_ml] = static_cast<int32_t>(state0);
  }
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_merge_workspace_init(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                                                 int32_t num_splits, float* part_o, float* part_ml,
                                                 int32_t* counters, void* stream) {
  using namespace msa;
  if (rows < 0 || num_q_heads <= 0 || num_splits <= 0) return MSA_ERR_INVALID_ARG;
  if (head_dim != MSA_HEAD_DIM || num_q_heads % MSA_HEADS_PER_KV != 0) return MSA_ERR_UNSUPPORTED;
  if (rows == 0) return MSA_OK;
  if (part_o == nullptr || part_ml == nullptr || counters == nullptr) return MSA_ERR_INVALID_ARG;
  if (num_splits > kMaxMergeSplits) return MSA_ERR_UNSUPPORTED;
  const int64_t rh = static_cast<int64_t>(rows) * num_q_heads;
  const int64_t n_o = 2 * rh * num_splits * MSA_HEAD_DIM, n_ml = 2 * rh * num_splits * 2;   // two buffers
  const int64_t n_c = rh / MSA_HEADS_PER_KV;
  const int64_t blocks = std::min<int64_t>((n_o + n_ml + n_c + 255) / 256, 4096);
  merge_idle_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<uint32_t*>(part_o), n_o, reinterpret_cast<uint32_t*>(part_ml), n_ml, counters, n_c,
      merge_state(0, num_splits));
  return launch_status();
}

extern "C" msa_status_t msa_step_workspace_init(int32_t rows, int32_t max_blocks, float* score_x,
                                                int32_t* score_words, void* stream) {
  using namespace msa;
  if (rows < 0 || max_blocks <= 0) return MSA_ERR_INVALID_ARG;
  if (max_blocks > MSA_MAX_BLOCKS) return MSA_ERR_UNSUPPORTED;
  if (rows == 0) return MSA_OK;
  if (score_x == nullptr || score_words == nullptr) return MSA_ERR_INVALID_ARG;
  const int64_t n_x = static_cast<int64_t>(rows) * max_blocks;
  const int64_t blocks = std::min<int64_t>((n_x + rows + 255) / 256, 4096);
  // (the merge workspace's fill kernel: idle words, then zero state words)
  merge_idle_kernel<<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream)>>>(
      reinterpret_cast<uint32_t*>(score_x), n_x, nullptr, 0, score_words, rows, 0u);
  return launch_status();
}
