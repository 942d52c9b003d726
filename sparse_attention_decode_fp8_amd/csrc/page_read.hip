// A plain read of the K/V bytes that one decode step selects, page by page through
// the selection's page list: the read floor the decode kernel is measured against.
// Built into libmsaprobe.so with the streaming-read reference; no entry point of the
// decode path uses it.
//
// Each work unit is one (physical page, KV head, visible tokens) triple, i.e. one
// selected block of one KV head (blocks a request's rows share count once). One
// workgroup of 256 threads reads the unit's visible tokens of all four arrays of the
// pool layout (K codes, V codes, K scales, V scales) with 16-byte loads, every load
// issued before any use, and folds them into one word that is stored only if it hits
// a constant, so the loads cannot be dropped and almost nothing is written. It does
// no dequantisation and no arithmetic: only the address computation through the page
// id that the decode also does.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;
constexpr int kPage = 128;
constexpr int kHeadDim = 128;

__device__ __forceinline__ uint32_t fold(uint4 a) { return a.x ^ a.y ^ a.z ^ a.w; }

// NVFP4: 64 code bytes + 8 scale bytes per token and array. The unit's codes of one
// array are ntok * 4 sixteen-byte words (at most 512: two per thread), its scales
// ceil(ntok / 2) words (at most 64).
__global__ void __launch_bounds__(kThreads)
page_read_nvfp4(const int32_t* __restrict__ units, const uint4* __restrict__ kc, const uint4* __restrict__ vc,
                const uint4* __restrict__ ks, const uint4* __restrict__ vs, int hkv, uint32_t* __restrict__ sink) {
  const int32_t* u = units + 3 * static_cast<int64_t>(blockIdx.x);
  const int64_t ph = static_cast<int64_t>(u[0]) * hkv + u[1];   // (page, head)
  const int ntok = u[2];
  const int t = threadIdx.x;
  const int code_words = ntok * 4, scale_words = (ntok + 1) / 2;
  const uint4* kcp = kc + ph * (kPage * 4);
  const uint4* vcp = vc + ph * (kPage * 4);
  const uint4* ksp = ks + ph * (kPage / 2);
  const uint4* vsp = vs + ph * (kPage / 2);
  const uint4 z = make_uint4(0, 0, 0, 0);
  const uint4 a0 = t < code_words ? kcp[t] : z;
  const uint4 a1 = t + kThreads < code_words ? kcp[t + kThreads] : z;
  const uint4 b0 = t < code_words ? vcp[t] : z;
  const uint4 b1 = t + kThreads < code_words ? vcp[t + kThreads] : z;
  const uint4 c0 = t < scale_words ? ksp[t] : z;
  const uint4 d0 = t < scale_words ? vsp[t] : z;
  const uint32_t acc = fold(a0) + fold(a1) + fold(b0) + fold(b1) + fold(c0) + fold(d0);
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

// FP8: 128 code bytes per token and array (ntok * 8 words, at most 1024: four per
// thread), plus the page's two fp32 scales.
__global__ void __launch_bounds__(kThreads)
page_read_fp8(const int32_t* __restrict__ units, const uint4* __restrict__ kc, const uint4* __restrict__ vc,
              const float* __restrict__ ks, const float* __restrict__ vs, int hkv, uint32_t* __restrict__ sink) {
  const int32_t* u = units + 3 * static_cast<int64_t>(blockIdx.x);
  const int64_t page = u[0];
  const int64_t ph = page * hkv + u[1];
  const int ntok = u[2];
  const int t = threadIdx.x;
  const int code_words = ntok * (kHeadDim / 16);
  const uint4* kcp = kc + ph * (kPage * kHeadDim / 16);
  const uint4* vcp = vc + ph * (kPage * kHeadDim / 16);
  const uint4 z = make_uint4(0, 0, 0, 0);
  uint4 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = t + i * kThreads < code_words ? kcp[t + i * kThreads] : z;
    b[i] = t + i * kThreads < code_words ? vcp[t + i * kThreads] : z;
  }
  const float s = t == 0 ? ks[page] + vs[page] : 0.0f;
  uint32_t acc = __float_as_uint(s);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc += fold(a[i]) + fold(b[i]);
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

// Reads the K/V bytes of `n_units` work units, units = int32 [n_units][3] device array
// of (physical page, KV head, visible tokens 1..128), from a pool of format `fmt`
// (1 = FP8 E4M3 with fp32 page scales, 2 = NVFP4) laid out as msa_kv_pool_t describes
// (k_codes, v_codes, k_scales, v_scales; num_kv_heads heads), on `stream` (a
// hipStream_t). One workgroup per unit. The caller guarantees that every page and
// head is inside the pool and every token count is in [1, 128]. `sink` is one device
// word written only when a fold hits its constant. Returns 0, -1 for bad arguments,
// -3 if the launch fails.
extern "C" int msa_probe_page_read(const int32_t* units, int32_t n_units, int32_t fmt, const void* k_codes,
                                   const void* v_codes, const void* k_scales, const void* v_scales,
                                   int32_t num_kv_heads, uint32_t* sink, void* stream) {
  if (n_units < 0 || num_kv_heads < 1 || sink == nullptr || (fmt != 1 && fmt != 2)) return -1;
  if (n_units == 0) return 0;
  if (units == nullptr || k_codes == nullptr || v_codes == nullptr || k_scales == nullptr || v_scales == nullptr)
    return -1;
  const auto s = static_cast<hipStream_t>(stream);
  if (fmt == 2)
    page_read_nvfp4<<<dim3(static_cast<unsigned>(n_units)), dim3(kThreads), 0, s>>>(
        units, static_cast<const uint4*>(k_codes), static_cast<const uint4*>(v_codes),
        static_cast<const uint4*>(k_scales), static_cast<const uint4*>(v_scales), num_kv_heads, sink);
  else
    page_read_fp8<<<dim3(static_cast<unsigned>(n_units)), dim3(kThreads), 0, s>>>(
        units, static_cast<const uint4*>(k_codes), static_cast<const uint4*>(v_codes),
        static_cast<const float*>(k_scales), static_cast<const float*>(v_scales), num_kv_heads, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
