// msa_select_topk: deterministic top-k block selection per query row.
//
// Contract ([Rubin] commit messages; [GB300] "The TP4 decode target", numerics):
// forced init/local blocks, the best other blocks by (score desc, index asc), output
// ascending and -1 padded. Ties are resolved by block index at any tie width, never
// by arrival order: the k'-th largest score is found with an MSB-first radix select
// (LDS histograms, whose counts do not depend on atomic order), then blocks tied at
// that score are ranked by an exclusive scan in block order.
#include "msa_device.h"
#include "msa_host.h"

namespace msa {
namespace {

constexpr int kThreads = 256;

// Exclusive prefix sum over the block in thread order; also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds_tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds_tmp[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    const int t = lds_tmp[i];
    if (i < wave) base += t;
    tot += t;
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__global__ void __launch_bounds__(kThreads)
select_topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ row_pos,
                   int32_t* __restrict__ sel, int max_blocks, int k, int n_init, int n_local) {
  extern __shared__ uint32_t keys[];            // [candidates]
  __shared__ int hist[256];
  __shared__ int tmp[kThreads / 64];
  __shared__ int s_digit, s_above;
  const int r = blockIdx.x, tid = threadIdx.x;
  const int nb = min(row_pos[r] / kPage + 1, max_blocks);   // the table covers nb blocks
  int32_t* out = sel + static_cast<int64_t>(r) * k;
  if (nb <= k) {                                 // identity table
    for (int i = tid; i < k; i += kThreads) out[i] = i < nb ? i : -1;
    return;
  }
  const int lo = n_init, C = nb - n_init - n_local;   // candidates are blocks lo .. lo + C - 1
  const int want = k - n_init - n_local;
  for (int i = tid; i < n_init; i += kThreads) out[i] = i;
  for (int i = tid; i < n_local; i += kThreads) out[k - n_local + i] = nb - n_local + i;
  if (want == 0) return;
  const float* srow = scores + static_cast<int64_t>(r) * max_blocks + lo;
  for (int c = tid; c < C; c += kThreads) keys[c] = float_key(srow[c]);

  uint32_t prefix = 0, pmask = 0;
  int remaining = want;                          // rank still to find among matching keys
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int c = tid; c < C; c += kThreads) {
      const uint32_t kk = keys[c];
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid < 64) {                              // wave 0 finds the digit holding the rank
      // lane L owns digits 255-4L .. 252-4L (descending); suffix sums from the top
      int c4[4], s = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c4[i] = hist[255 - 4 * tid - i]; s += c4[i]; }
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
          s_digit = 255 - 4 * tid - i;
          s_above = above;
        }
        above += c4[i];
      }
    }
    __syncthreads();
    const uint32_t dg = static_cast<uint32_t>(s_digit);
    remaining -= s_above;
    prefix |= dg << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  // prefix is now the exact key of the want-th largest candidate; `remaining` of the
  // keys equal to it are taken, the ones with the smallest block index.
  const uint32_t T = prefix;
  const int chunk = (C + kThreads - 1) / kThreads;
  const int c0 = min(tid * chunk, C), c1 = min(c0 + chunk, C);
  int nties = 0;
  for (int c = c0; c < c1; ++c) nties += keys[c] == T;
  int tot;
  int tie_before = block_exclusive_scan(nties, tmp, &tot);
  int nsel = 0;
  {
    int tb = tie_before;
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = keys[c];
      const bool take = kk > T || (kk == T && tb < remaining);
      tb += kk == T;
      nsel += take;
    }
  }
  int sel_before = block_exclusive_scan(nsel, tmp, &tot);
  {
    int tb = tie_before, at = n_init + sel_before;
    for (int c = c0; c < c1; ++c) {
      const uint32_t kk = keys[c];
      const bool take = kk > T || (kk == T && tb < remaining);
      tb += kk == T;
      if (take && at < k - n_local) out[at++] = lo + c;
    }
  }
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_select_topk(const msa_step_t* step, const float* block_scores,
                                        int32_t k, int32_t n_init, int32_t n_local, int32_t* sel,
                                        void* stream) {
  using namespace msa;
  msa_status_t st = check_step(step);
  if (st != MSA_OK) return st;
  if (k < 1 || k > MSA_MAX_TOPK || n_init < 0 || n_local < 0 || n_init + n_local > k)
    return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0) return MSA_OK;
  if (block_scores == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  const size_t lds = static_cast<size_t>(step->max_blocks_per_seq) * sizeof(uint32_t);
  select_topk_kernel<<<dim3(step->num_rows), dim3(kThreads), lds, static_cast<hipStream_t>(stream)>>>(
      block_scores, step->row_pos, sel, step->max_blocks_per_seq, k, n_init, n_local);
  return launch_status();
}
