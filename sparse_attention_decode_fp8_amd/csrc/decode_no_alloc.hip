// msa_sparse_decode_combine_noalloc: msa_sparse_decode_combine for callers that cannot
// allocate device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc). Its split partials live in a fixed array of this library,
// one per GPU, instead of a caller-provided merge workspace.
//
// One split: the one-split decode writes the output itself and needs no scratch.
// Several: the decode writes its partials into the array and msa_combine merges them
// (the fused entry's merge is msa_combine's arithmetic in the same order, so the two
// give the same output bit for bit). Every call overwrites the partials it reads, so
// nothing in the array has to start at a known value.
#include <atomic>
#include <mutex>

#include "msa_decode.h"
#include "msa_device.h"
#include "msa_host.h"

namespace msa {
namespace {

constexpr size_t kScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;

// The partials of the allocation-free entry, one copy per GPU for the life of the
// process. In host code this name is a host-side stand-in, not a device address:
// kernels get the address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The array's address on the current device, looked up once per device.
msa_status_t scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MSA_ERR_LAUNCH;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return MSA_ERR_LAUNCH;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return MSA_OK;
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_sparse_decode_combine_noalloc(const msa_kv_pool_t* pool, const msa_step_t* step,
                                                          int32_t num_q_heads, const void* q, const int32_t* sel,
                                                          const int32_t* sel_pages, int32_t k, float softmax_scale,
                                                          int32_t num_splits, void* out, void* stream) {
  using namespace msa;
  if (pool == nullptr || step == nullptr || out == nullptr) return MSA_ERR_INVALID_ARG;
  if (num_splits < 1 || step->num_rows < 0 || num_q_heads <= 0) return MSA_ERR_INVALID_ARG;
  if (num_splits > kMaxMergeSplits) return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0)   // validation only (msa_sparse_decode launches nothing for no rows)
    return msa_sparse_decode(pool, step, num_q_heads, q, sel, sel_pages, k, softmax_scale, num_splits, nullptr,
                             nullptr, stream);
  // the partials, part_o then part_ml at a 256-byte boundary, must fit the array
  const size_t n = static_cast<size_t>(step->num_rows) * num_q_heads * num_splits;
  const size_t o_bytes = (n * MSA_HEAD_DIM * sizeof(float) + 255) / 256 * 256;
  if (o_bytes + n * 2 * sizeof(float) > kScratchBytes) return MSA_ERR_TOO_LARGE;
  void* base = nullptr;
  msa_status_t st = scratch_address(&base);
  if (st != MSA_OK) return st;
  float* part_o = static_cast<float*>(base);
  float* part_ml = reinterpret_cast<float*>(static_cast<uint8_t*>(base) + o_bytes);
  if (num_splits == 1)   // the one-split decode writes `out` and leaves the workspace untouched
    return msa_sparse_decode_combine(pool, step, num_q_heads, q, sel, sel_pages, k, softmax_scale, 1, part_o, part_ml,
                                     static_cast<int32_t*>(base), out, stream);
  st = msa_sparse_decode(pool, step, num_q_heads, q, sel, sel_pages, k, softmax_scale, num_splits, part_o, part_ml,
                         stream);
  if (st != MSA_OK) return st;
  return msa_combine(step->num_rows, num_q_heads, MSA_HEAD_DIM, num_splits, part_o, part_ml, out, stream);
}
