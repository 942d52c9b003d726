// msa_sparse_decode: GQA flash-decode over the selected P128 pages, split-KV partials.
//
// Prior art on the pages: [Rubin] commit messages describe a block-sparse verify
// decode with one unit of work per (top-k split, KV head, query row) and NVFP4
// dequantised in registers, merging splits across CTAs; [Rubin] "Items and numerics"
// (LC_ONEDIV) fixes the merge to a single divide per output in a fixed order.
//
// MI355X design. One workgroup of W waves per (split, KV head, query row); each wave
// takes one selected page at a time (128 tokens, 4 chunks of 32) and keeps its own
// online softmax, and the W waves merge in LDS at the end. All 16 query heads of the
// KV head ride in the MFMA N dimension, so both contractions keep "head" on lane % 16:
//   S^T[token][head] = K[token][d] . Q^T[d][head]      A = K  (dequantised in registers)
//   O^T[d][head]    += V^T[d][token] . P^T[token][head] A = V^T (LDS, transposing read)
// and the softmax state (max, sum, rescale) is per lane, with no cross-lane transpose.
// K and V are dequantised exactly to fp16 (E2M1 x E4M3 has at most 6 significant bits;
// E4M3 fits fp16), Q is pre-scaled by a power of two per head so its fp16 conversion
// is exact, accumulation is fp32. The NVFP4 tensor scales and FP8 page scales are
// applied outside the MFMAs (folded into the logit scale and the output rescale).
#include "msa_device.h"
#include "msa_host.h"

namespace msa {
namespace {

constexpr int kVRowHalves = 144;   // 128 fp16 + 16 pad: 288-byte rows keep 4 rows on disjoint banks

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
  const uint16_t* q;
  const int32_t* sel;
  int k;
  float softmax_scale;
  int num_splits;
  float* part_o;
  float* part_ml;
};

__device__ __forceinline__ half2_t bcast_lo(half2_t v) { return half2_t{v[0], v[0]}; }
__device__ __forceinline__ half2_t bcast_hi(half2_t v) { return half2_t{v[1], v[1]}; }

template <int kFmt>
struct PageRegs;

template <>
struct PageRegs<MSA_KV_NVFP4> {
  uint4 k[8], v[8];          // [chunk * 2 + tile]: 32 E2M1 codes of one token (dims 32q..32q+31)
  uint32_t ks[8], vs[8];     // the two E4M3 scales of those dims
};
template <>
struct PageRegs<MSA_KV_FP8_E4M3> {
  uint4 k[16], v[16];        // [(chunk * 2 + tile) * 2 + half]: 32 E4M3 codes
};

template <int kFmt>
__device__ __forceinline__ void load_page(PageRegs<kFmt>& R, const DecodeArgs& a, int64_t page, int g,
                                          int n, int q, int nchunks) {
  const int64_t tok0 = (page * a.hkv + g) * kPage + n;      // token row of (page, head, n)
  if constexpr (kFmt == MSA_KV_NVFP4) {
    const uint8_t* kc = a.k_codes + tok0 * (kHeadDim / 2) + 16 * q;
    const uint8_t* vc = a.v_codes + tok0 * (kHeadDim / 2) + 16 * q;
    const uint8_t* kss = a.k_scales + tok0 * (kHeadDim / 16) + 2 * q;
    const uint8_t* vss = a.v_scales + tok0 * (kHeadDim / 16) + 2 * q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i / 2 < nchunks) {
        R.k[i] = *reinterpret_cast<const uint4*>(kc + i * 16 * (kHeadDim / 2));
        R.v[i] = *reinterpret_cast<const uint4*>(vc + i * 16 * (kHeadDim / 2));
        R.ks[i] = *reinterpret_cast<const uint16_t*>(kss + i * 16 * (kHeadDim / 16));
        R.vs[i] = *reinterpret_cast<const uint16_t*>(vss + i * 16 * (kHeadDim / 16));
      }
    }
  } else {
    const uint8_t* kc = a.k_codes + tok0 * kHeadDim + 32 * q;
    const uint8_t* vc = a.v_codes + tok0 * kHeadDim + 32 * q;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i / 2 < nchunks) {
        R.k[2 * i] = *reinterpret_cast<const uint4*>(kc + i * 16 * kHeadDim);
        R.k[2 * i + 1] = *reinterpret_cast<const uint4*>(kc + i * 16 * kHeadDim + 16);
        R.v[2 * i] = *reinterpret_cast<const uint4*>(vc + i * 16 * kHeadDim);
        R.v[2 * i + 1] = *reinterpret_cast<const uint4*>(vc + i * 16 * kHeadDim + 16);
      }
    }
  }
}

// Dims 32q + 8j .. +7 of tile `ti` (= chunk * 2 + tile) as an fp16 MFMA operand.
template <int kFmt>
__device__ __forceinline__ half8_t dequant8(const uint4* codes, const uint32_t* scales, int ti, int j) {
  if constexpr (kFmt == MSA_KV_NVFP4) {
    const uint4 c = codes[ti];
    const uint32_t w = j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
    const half2_t sc = e4m3x2_to_f16(scales[ti]);
    return e2m1x8_to_f16(w, j < 2 ? bcast_lo(sc) : bcast_hi(sc));
  } else {
    const uint4 c = codes[2 * ti + (j >> 1)];
    return (j & 1) ? e4m3x8_to_f16(c.z, c.w) : e4m3x8_to_f16(c.x, c.y);
  }
}

template <int kFmt, int kW>
__global__ void __launch_bounds__(64 * kW) sparse_decode_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) half_t vbuf[kW][32 * kVRowHalves];
  __shared__ float mbuf[kW][16], lbuf[kW][16];
  const int s = blockIdx.x, g = blockIdx.y, r = blockIdx.z;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int hq = a.hkv * kHeadsPerKv;
  const int seq = a.row_seq[r], pos = a.row_pos[r];
  const int lo = (s * a.k) / a.num_splits, hi = ((s + 1) * a.k) / a.num_splits;

  // Q^T operand: lane (n, q) holds head 16g + n, dims 32q + 8j .. +7 for k-step j.
  half8_t Qop[4];
  float cscale;
  {
    const uint4* qp = reinterpret_cast<const uint4*>(
        a.q + (static_cast<int64_t>(r) * hq + kHeadsPerKv * g + n) * kHeadDim + 32 * q);
    float qf[32];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = qp[i];
      const uint32_t wv[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        qf[8 * i + 2 * t] = __uint_as_float(wv[t] << 16);
        qf[8 * i + 2 * t + 1] = __uint_as_float(wv[t] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qf[i]));
    amax = xor_max(xor_max(amax, 16), 32);
    const int e = f16_prescale_exp(amax);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) Qop[j][i] = static_cast<half_t>(ldexpf(qf[8 * j + i], e));
    cscale = ldexpf(a.softmax_scale * kLog2e, -e);
    if constexpr (kFmt == MSA_KV_NVFP4) cscale *= a.k_t;
  }

  float m_run = -INFINITY, l_run = 0.0f, v_cur = 0.0f;   // v_cur: FP8 page scale O is kept in
  float4_t O[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) O[c] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  half_t* vb = vbuf[wave];

  for (int e = lo + wave; e < hi; e += kW) {
    const int b = a.sel[static_cast<int64_t>(r) * a.k + e];
    if (b < 0) continue;
    int n_vis = pos - b * kPage + 1;
    if (n_vis <= 0) continue;
    n_vis = min(n_vis, kPage);
    const int nchunks = (n_vis + 31) >> 5;
    const int64_t page = a.block_table[static_cast<int64_t>(seq) * a.max_blocks + b];
    PageRegs<kFmt> R;
    load_page<kFmt>(R, a, page, g, n, q, nchunks);
    float cs = cscale, ratio = 1.0f;
    if constexpr (kFmt == MSA_KV_FP8_E4M3) {
      cs *= reinterpret_cast<const float*>(a.k_scales)[page];
      const float vp = reinterpret_cast<const float*>(a.v_scales)[page];
      ratio = v_cur > 0.0f ? v_cur / vp : 1.0f;     // keep O in units of this page's scale
      v_cur = vp;
    }
    const uint32_t* ksc = nullptr;
    const uint32_t* vsc = nullptr;
    if constexpr (kFmt == MSA_KV_NVFP4) { ksc = R.ks; vsc = R.vs; }

#pragma unroll
    for (int c = 0; c < 4; ++c) {
      if (c >= nchunks) break;
      // ---- scores of 32 tokens for 16 heads
      float x[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = mfma16x16x32(dequant8<kFmt>(R.k, ksc, 2 * c + u, j), Qop[j], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int tok = 32 * c + 16 * u + 4 * q + i;
          x[u][i] = tok < n_vis ? acc[i] * cs : -INFINITY;
        }
      }
      // ---- online softmax (per lane: one head)
      float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mx = xor_max(xor_max(mx, 16), 32);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      float psum = 0.0f;
      half8_t Pt;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = exp2f(x[u][i] - m_new);
          psum += p;
          Pt[4 * u + i] = static_cast<half_t>(p);
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      const float ao = c == 0 ? alpha * ratio : alpha;
#pragma unroll
      for (int d = 0; d < 8; ++d) O[d] *= ao;
      // ---- V chunk to LDS (natural [token][d] layout, fp16)
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<half8_t*>(vb + (16 * u + n) * kVRowHalves + 32 * q + 8 * j) =
              dequant8<kFmt>(R.v, vsc, 2 * c + u, j);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      // ---- O^T += V^T . P^T over the 32 tokens, 8 tiles of 16 dims
      typedef __attribute__((address_space(3))) short4_t lds_s4;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const half_t* p0 = vb + (4 * q + (n >> 2)) * kVRowHalves + 16 * d + 4 * (n & 3);
        const half_t* p1 = p0 + 16 * kVRowHalves;
        const short4_t r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0));
        const short4_t r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1));
        half8_t Vt;
        const half4_t h0 = __builtin_bit_cast(half4_t, r0), h1 = __builtin_bit_cast(half4_t, r1);
        Vt[0] = h0[0]; Vt[1] = h0[1]; Vt[2] = h0[2]; Vt[3] = h0[3];
        Vt[4] = h1[0]; Vt[5] = h1[1]; Vt[6] = h1[2]; Vt[7] = h1[3];
        O[d] = mfma16x16x32(Vt, Pt, O[d]);
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
  }

  float l_tot = xor_add(xor_add(l_run, 16), 32);
  float oscale;
  if constexpr (kFmt == MSA_KV_NVFP4) oscale = a.v_t; else oscale = v_cur;
  const int64_t head = static_cast<int64_t>(r) * hq + kHeadsPerKv * g;
  if constexpr (kW == 1) {
    float* po = a.part_o + ((head + n) * a.num_splits + s) * kHeadDim + 4 * q;
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<float4_t*>(po + 16 * d) = O[d] * oscale;
    if (q == 0) {
      float* pm = a.part_ml + ((head + n) * a.num_splits + s) * 2;
      pm[0] = m_run;
      pm[1] = l_tot;
    }
  } else {
    __syncthreads();                               // every wave is done with vbuf
    float* ob = reinterpret_cast<float*>(vbuf[wave]);   // [16 heads][128 d] fp32 = 8 KiB
#pragma unroll
    for (int d = 0; d < 8; ++d) *reinterpret_cast<float4_t*>(ob + n * kHeadDim + 16 * d + 4 * q) = O[d] * oscale;
    if (q == 0) { mbuf[wave][n] = m_run; lbuf[wave][n] = l_tot; }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * (kHeadDim / 4); idx += 64 * kW) {
      const int h = idx / (kHeadDim / 4), d4 = idx % (kHeadDim / 4);
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < kW; ++w) M = fmaxf(M, mbuf[w][h]);
      float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
      float l = 0.0f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          const float wt = exp2f(mbuf[w][h] - M);
          acc += wt * *reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(vbuf[w]) +
                                                         h * kHeadDim + 4 * d4);
          l += wt * lbuf[w][h];
        }
      }
      float* po = a.part_o + ((head + h) * a.num_splits + s) * kHeadDim + 4 * d4;
      *reinterpret_cast<float4_t*>(po) = acc;
      if (d4 == 0) {
        float* pm = a.part_ml + ((head + h) * a.num_splits + s) * 2;
        pm[0] = M;
        pm[1] = l;
      }
    }
  }
}

template <int kFmt, int kW>
void launch(const DecodeArgs& a, dim3 grid, hipStream_t s) {
  sparse_decode_kernel<kFmt, kW><<<grid, dim3(64 * kW), 0, s>>>(a);
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_sparse_decode(const msa_kv_pool_t* pool, const msa_step_t* step,
                                          int32_t num_q_heads, const void* q, const int32_t* sel,
                                          int32_t k, float softmax_scale, int32_t num_splits,
                                          float* part_o, float* part_ml, void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (num_q_heads != MSA_HEADS_PER_KV * pool->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  if (k < 1 || k > MSA_MAX_TOPK || num_splits < 1 || num_splits > k) return MSA_ERR_UNSUPPORTED;
  if (!(softmax_scale > 0.0f)) return MSA_ERR_INVALID_ARG;
  if (step->num_rows == 0) return MSA_OK;
  if (q == nullptr || sel == nullptr || part_o == nullptr || part_ml == nullptr) return MSA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(part_o) || (reinterpret_cast<uintptr_t>(part_ml) & 7u))
    return MSA_ERR_INVALID_ARG;
  if (step->num_rows > 65535) return MSA_ERR_UNSUPPORTED;
  DecodeArgs a;
  a.k_codes = static_cast<const uint8_t*>(pool->k_codes);
  a.v_codes = static_cast<const uint8_t*>(pool->v_codes);
  a.k_scales = static_cast<const uint8_t*>(pool->k_scales);
  a.v_scales = static_cast<const uint8_t*>(pool->v_scales);
  a.k_t = pool->k_tensor_scale;
  a.v_t = pool->v_tensor_scale;
  a.hkv = pool->num_kv_heads;
  a.block_table = step->block_table;
  a.row_seq = step->row_seq;
  a.row_pos = step->row_pos;
  a.max_blocks = step->max_blocks_per_seq;
  a.q = static_cast<const uint16_t*>(q);
  a.sel = sel;
  a.k = k;
  a.softmax_scale = softmax_scale;
  a.num_splits = num_splits;
  a.part_o = part_o;
  a.part_ml = part_ml;
  // waves per workgroup: one per selected page of the split, up to 4
  const int per_split = (k + num_splits - 1) / num_splits;
  const int W = per_split >= 4 ? 4 : per_split >= 2 ? 2 : 1;
  dim3 grid(num_splits, pool->num_kv_heads, step->num_rows);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (pool->fmt == MSA_KV_NVFP4) {
    if (W == 4) launch<MSA_KV_NVFP4, 4>(a, grid, s);
    else if (W == 2) launch<MSA_KV_NVFP4, 2>(a, grid, s);
    else launch<MSA_KV_NVFP4, 1>(a, grid, s);
  } else {
    if (W == 4) launch<MSA_KV_FP8_E4M3, 4>(a, grid, s);
    else if (W == 2) launch<MSA_KV_FP8_E4M3, 2>(a, grid, s);
    else launch<MSA_KV_FP8_E4M3, 1>(a, grid, s);
  }
  return launch_status();
}
