// msa_kv_append: quantise new tokens' K, V and index-K into their page slots.
//
// [GB300] "Step-loop runtime hooks" names the KV update as its own step; [Rubin]
// Description requires saturating FP8 casts. One thread encodes one group of 16
// contiguous elements of one token (the encoder is in append_device.h).
#include "append_device.h"
#include "msa_host.h"

namespace msa {
namespace {

template <int kFmt>
__global__ void __launch_bounds__(256) kv_append_kernel(AppendArgs a) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= static_cast<int64_t>(a.n_new) * a.groups_per_tok) return;
  append_group<kFmt>(a, gid);
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_kv_append(const msa_kv_pool_t* pool, int32_t n_new, const int64_t* slot,
                                      const void* k_new, const void* v_new, const void* idx_k_new,
                                      void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if (n_new < 0) return MSA_ERR_INVALID_ARG;
  if (n_new == 0) return MSA_OK;
  if (slot == nullptr) return MSA_ERR_INVALID_ARG;
  for (const void* p : {k_new, v_new, idx_k_new})
    if (p != nullptr && !aligned16(p)) return MSA_ERR_INVALID_ARG;
  const AppendArgs a = make_append_args(pool, n_new, slot, k_new, v_new, idx_k_new);
  const int64_t total = static_cast<int64_t>(n_new) * a.groups_per_tok;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return MSA_ERR_UNSUPPORTED;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pool->fmt == MSA_KV_NVFP4)
    kv_append_kernel<MSA_KV_NVFP4><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(a);
  else
    kv_append_kernel<MSA_KV_FP8_E4M3><<<dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s>>>(a);
  return launch_status();
}
