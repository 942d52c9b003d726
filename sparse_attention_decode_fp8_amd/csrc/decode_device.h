// Decode building blocks shared by the sparse decode kernels (one query row per
// workgroup, or a group of rows over the union of their selections): the per-lane
// registers of one 32-token chunk of one (page, KV head), its loads through buffer
// resources, its exact dequantisation to fp16 MFMA operands, and the LDS staging of V.
//
// MFMA layout (v_mfma_f32_16x16x32_f16, see msa_device.h): all 16 query heads of a KV
// head ride in the N dimension, so "head" is lane % 16 in both contractions:
//   S^T[token][head] = K[token][d] . Q^T[d][head]      A = K  (dequantised in registers)
//   O^T[d][head]    += V^T[d][token] . P^T[token][head] A = V^T (LDS, transposing read)
#pragma once

#include "msa_device.h"

namespace msa {

constexpr int kVRowHalves = 144;   // 128 fp16 + 16 pad: 288-byte rows keep 4 rows on disjoint banks
constexpr int kVBufBytes = 32 * kVRowHalves * 2;   // one wave's 32-token V chunk
// A wave's O tile, [16 heads][128 d] fp32, reuses its V buffer. Rows are 132 floats
// (33 16-byte quads, an odd count) so the 16 heads a quarter-wave writes at once fall
// on distinct banks; 128-float rows would put all 16 on the same banks.
constexpr int kORowFloats = kHeadDim + 4;
static_assert(16 * kORowFloats * 4 <= kVBufBytes, "O tile must fit in a V buffer");

// The pool arrays a decode reads (layout of msa_kv_pool_t).
struct KvArrays {
  const uint8_t* k_codes;
  const uint8_t* v_codes;
  const uint8_t* k_scales;
  const uint8_t* v_scales;
};

__device__ __forceinline__ half2_t bcast_lo(half2_t v) { return half2_t{v[0], v[0]}; }
__device__ __forceinline__ half2_t bcast_hi(half2_t v) { return half2_t{v[1], v[1]}; }

// One 32-token chunk of one page, as held by a lane: tile u (tokens 16u .. 16u+15 of
// the chunk), token 16u + (lane % 16), dims 32q .. 32q+31.
template <int kFmt>
struct ChunkRegs;
template <>
struct ChunkRegs<MSA_KV_NVFP4> {
  uint4 k[2], v[2];        // 32 E2M1 codes
  uint32_t ks[2], vs[2];   // the two E4M3 scales of those 32 dims
};
template <>
struct ChunkRegs<MSA_KV_FP8_E4M3> {
  uint4 k[4], v[4];        // [tile * 2 + half]: 32 E4M3 codes
};

// Loads of one 32-token chunk (chunk c of the page's 128 tokens) of one (page, KV head)
// through buffer resources whose base is that (page, head)'s region of each array (a
// wave-uniform address: the page comes from the selection table in scalar registers).
// An empty chunk (valid = false) gets resources of zero bytes: its loads return zero
// without touching memory, and every chunk issues the same loads, so the compiler
// knows how many are in flight and can consume earlier loads (Q) without waiting for
// the page data.
template <int kFmt>
__device__ __forceinline__ void load_chunk(ChunkRegs<kFmt>& R, const KvArrays& a, int64_t ph, bool valid,
                                           int c, int n, int q) {
  const uint32_t t0 = 32u * c + n;   // this lane's token in tile 0; tile 1 is 16 tokens on
  if constexpr (kFmt == MSA_KV_NVFP4) {
    constexpr uint32_t kCodeBytes = kPage * kHeadDim / 2, kScaleBytes = kPage * kHeadDim / 16;
    const __amdgpu_buffer_rsrc_t kc = make_rsrc(uniform_ptr(a.k_codes + ph * kCodeBytes), valid ? kCodeBytes : 0u);
    const __amdgpu_buffer_rsrc_t vc = make_rsrc(uniform_ptr(a.v_codes + ph * kCodeBytes), valid ? kCodeBytes : 0u);
    const __amdgpu_buffer_rsrc_t ks = make_rsrc(uniform_ptr(a.k_scales + ph * kScaleBytes), valid ? kScaleBytes : 0u);
    const __amdgpu_buffer_rsrc_t vs = make_rsrc(uniform_ptr(a.v_scales + ph * kScaleBytes), valid ? kScaleBytes : 0u);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t t = t0 + 16u * u;
      R.k[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, static_cast<int>(t * (kHeadDim / 2) + 16 * q), 0, 0));
      R.v[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vc, static_cast<int>(t * (kHeadDim / 2) + 16 * q), 0, 0));
      R.ks[u] = __builtin_amdgcn_raw_buffer_load_b16(ks, static_cast<int>(t * (kHeadDim / 16) + 2 * q), 0, 0);
      R.vs[u] = __builtin_amdgcn_raw_buffer_load_b16(vs, static_cast<int>(t * (kHeadDim / 16) + 2 * q), 0, 0);
    }
  } else {
    constexpr uint32_t kCodeBytes = kPage * kHeadDim;
    const __amdgpu_buffer_rsrc_t kc = make_rsrc(uniform_ptr(a.k_codes + ph * kCodeBytes), valid ? kCodeBytes : 0u);
    const __amdgpu_buffer_rsrc_t vc = make_rsrc(uniform_ptr(a.v_codes + ph * kCodeBytes), valid ? kCodeBytes : 0u);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t t = t0 + 16u * u;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        R.k[2 * u + h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, static_cast<int>(t * kHeadDim + 32 * q + 16 * h), 0, 0));
        R.v[2 * u + h] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(vc, static_cast<int>(t * kHeadDim + 32 * q + 16 * h), 0, 0));
      }
    }
  }
}

// Dims 32q + 8j .. +7 of tile u as an fp16 MFMA operand.
template <int kFmt>
__device__ __forceinline__ half8_t dequant8(const uint4* codes, const uint32_t* scales, int u, int j) {
  if constexpr (kFmt == MSA_KV_NVFP4) {
    const uint4 c = codes[u];
    const uint32_t w = j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
    const half2_t sc = e4m3x2_to_f16(scales[u]);
    return e2m1x8_to_f16(w, j < 2 ? bcast_lo(sc) : bcast_hi(sc));
  } else {
    const uint4 c = codes[2 * u + (j >> 1)];
    return (j & 1) ? e4m3x8_to_f16(c.z, c.w) : e4m3x8_to_f16(c.x, c.y);
  }
}

// Q^T operand of one (row, KV head): lane (n, q) holds head 16g + n, dims 32q + 8j .. +7
// for k-step j. `qh` points at dims 32q of that head's bf16 row.
__device__ __forceinline__ void load_q_raw(uint4 (&qraw)[4], const uint16_t* qh) {
  const uint4* qp = reinterpret_cast<const uint4*>(qh);
#pragma unroll
  for (int i = 0; i < 4; ++i) qraw[i] = qp[i];
}

// Exact fp16 operand: each head is scaled by a power of two 2^e that brings its bf16
// values into fp16's normal range; cscale = 2^-e * base * mult is the logit scale that
// undoes it (base: softmax scale * log2(e); mult: the NVFP4 K tensor scale, or 1).
__device__ __forceinline__ void convert_q_op(const uint4 (&qraw)[4], half8_t (&Qop)[4], float& cscale, float base,
                                             float mult) {
  float qf[32];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t wv[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qf[8 * i + 2 * t] = __uint_as_float(wv[t] << 16);
      qf[8 * i + 2 * t + 1] = __uint_as_float(wv[t] & 0xffff0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(qf[i]));
  amax = rows_max(amax);
  const int e = f16_prescale_exp(amax);
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) Qop[j][i] = static_cast<half_t>(ldexpf(qf[8 * j + i], e));
  cscale = ldexpf(base, -e) * mult;
}

}  // namespace msa
