// A plain streaming read of one device buffer: the reference for the read bandwidth
// the part sustains, against which the decode kernel's achieved rate is also stated.
// Built into its own library (libmsaprobe.so); no entry point of the decode path uses it.
//
// Every lane reads 16-byte words in a grid-stride loop, four loads in flight per
// iteration, and folds them into one word; the fold is stored only if it equals a
// constant, so the loads cannot be dropped and almost nothing is written.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

__global__ void __launch_bounds__(kThreads)
stream_read_kernel(const uint4* __restrict__ p, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
  int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = p[i], b = p[i + stride], c = p[i + 2 * stride], d = p[i + 3 * stride];
    acc ^= (a.x ^ a.y ^ a.z ^ a.w) + (b.x ^ b.y ^ b.z ^ b.w) + (c.x ^ c.y ^ c.z ^ c.w) +
           (d.x ^ d.y ^ d.z ^ d.w);
  }
  for (; i < n16; i += stride) {
    const uint4 a = p[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9e3779b9u) sink[0] = acc;
}

}  // namespace

// Reads `bytes` (a multiple of 16, 16-byte aligned) of device memory at `buf` once, on
// `stream` (a hipStream_t), with `workgroups` workgroups of 256 threads. `sink` is one
// device word that is written only when the fold hits its constant. Returns 0, -1 for
// bad arguments, -3 if the launch fails.
extern "C" int msa_probe_stream_read(const void* buf, int64_t bytes, uint32_t* sink, int32_t workgroups,
                                     void* stream) {
  if (buf == nullptr || sink == nullptr || bytes < 0 || bytes % 16 != 0 || workgroups < 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return -1;
  if (bytes == 0) return 0;
  stream_read_kernel<<<dim3(static_cast<unsigned>(workgroups)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream)>>>(static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
