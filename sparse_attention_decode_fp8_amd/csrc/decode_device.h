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

#include "append_device.h"
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
      R.k[u] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(kc, static_cast<int>(t * (kHeadDim / 2) + 16 * q), 0, kStreamPolicy));
      R.v[u] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(vc, static_cast<int>(t * (kHeadDim / 2) + 16 * q), 0, kStreamPolicy));
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

// The new tokens' K and V of one KV head as the append encodes them, held in LDS by the
// single-launch step (at most 64 tokens): NVFP4 codes [token][K, V][group of 16 dims]
// (8 bytes) and scale codes; FP8 codes [token][K, V][group] (16 bytes).
template <int kFmt>
struct NewKv;
template <>
struct NewKv<MSA_KV_NVFP4> {
  uint2 codes[64][2][8];
  uint8_t scales[64][2][8];
};
template <>
struct NewKv<MSA_KV_FP8_E4M3> {
  uint4 codes[64][2][8];
};

// Encode group `grp` of KV head g into `nk`: new token grp / 16, K (or V when
// (grp / 8) is odd), dims 16 (grp % 8) .. +15, by the append's rules (NVFP4 at the
// tensor scale; FP8 at the scale of the token's page); with `owner`, also write it to
// the token's slot in the pool (msa_kv_append's layout). A token with a negative slot,
// or a null source, is not appended and is skipped.
// Position of the k-th set bit (k from 0) of m; k < popcount(m).
__device__ __forceinline__ int nth_set_bit(uint64_t m, int k) {
  int pos = 0;
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) {
    const int c = __popcll(m & ((1ull << w) - 1));
    if (k >= c) {
      k -= c;
      m >>= w;
      pos += w;
    }
  }
  return pos;
}

// One 16-element group encoded by the 16 lanes of a row, lane l holding element l:
// the same arithmetic per element as nvfp4_encode16 / fp8_encode16 / encode_index16
// (the group maximum by exact max operations, from max(|x|, 0) in every lane, so a NaN
// is ignored as there), so the codes are bit-identical. The packed codes are returned
// in lane 0 of the row (and the NVFP4 scale code in every lane).
// NVFP4 at tensor scale t: codes as w0 | w1 << 32 (element 2j in the low nibble of byte j).
__device__ __forceinline__ uint32_t nvfp4_encode_row(float x, float t, uint2& codes) {
#pragma clang fp contract(off)
  const int l = threadIdx.x & 15;
  float amax = fmaxf(fabsf(x), 0.0f);
#pragma unroll
  for (int m = 1; m < 16; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 16));
  const float six_t = 6.0f * t;
  const uint32_t sc = f32_to_e4m3_sat(amax / six_t);
  const float dec = e4m3_to_f32(sc);
  uint32_t v = 0;
  if (dec != 0.0f) {
    const float d = dec * t;
    v = f32_to_e2m1_sat(x / d) << (4 * (l & 7));
  }
#pragma unroll
  for (int m = 1; m < 8; m <<= 1) v |= __shfl_xor(v, m, 16);   // each half row's 8 nibbles
  codes = make_uint2(v, __shfl_down(v, 8, 16));
  return sc;
}
// E4M3 codes of x / s (s = 1: the index-key rule), bytes in element order.
__device__ __forceinline__ uint4 e4m3_encode_row(float x, float s) {
#pragma clang fp contract(off)
  const int l = threadIdx.x & 15;
  uint32_t v = f32_to_e4m3_sat(x / s) << (8 * (l & 3));
#pragma unroll
  for (int m = 1; m < 4; m <<= 1) v |= __shfl_xor(v, m, 16);   // each quarter row's 4 bytes
  return make_uint4(v, __shfl_down(v, 4, 16), __shfl_down(v, 8, 16), __shfl_down(v, 12, 16));
}

// The new tokens that land in chunk c of `page` (bit i: new token i; slot0: lane i <
// n_new holds new token i's slot, else -1).
__device__ __forceinline__ uint64_t new_tokens_in_chunk(int64_t slot0, int64_t page, int c) {
  return __ballot(slot0 >= 0 && (slot0 >> 7) == page && ((slot0 & (kPage - 1)) >> 5) == c);
}

// Tokens appended by the same launch (the single-launch step): the lanes that hold one
// of the chunk's new tokens (`hits`, from new_tokens_in_chunk) replace its codes and
// scales with the token's encoding, so the decode never depends on when the append's
// stores to the pool land. Tokens in `in_lds` (bit i: new token i) take it from `nk`;
// any other is encoded here from its bf16 source, by the append's rules, by the lanes
// that hold it (KV head g; FP8 at the page's scales kps / vps). Called once the chunk's
// loads have arrived (the registers it writes are those loads' destinations). A K or V
// source that is null is not appended, and the loaded bytes stay.
template <int kFmt>
__device__ __forceinline__ void patch_new_tokens(ChunkRegs<kFmt>& R, const NewKv<kFmt>& nk, const AppendArgs& app,
                                                 int64_t slot0, uint64_t hits, uint64_t in_lds, int g, int n, int q,
                                                 float kps, float vps) {
  while (hits != 0u) {
    const int i = __ffsll(static_cast<unsigned long long>(hits)) - 1;
    hits &= hits - 1;
    const int off = __builtin_amdgcn_readlane(static_cast<int>(slot0 & 31), i);   // token in the chunk
    if ((off & 15) != n) continue;
    const int u = off >> 4;
    const bool from_lds = (in_lds >> i) & 1u;
#pragma unroll
    for (int kv = 0; kv < 2; ++kv) {
      const uint16_t* src = kv == 0 ? app.k_new : app.v_new;
      if (src == nullptr) continue;
      uint4* codes = kv == 0 ? R.k : R.v;
      if constexpr (kFmt == MSA_KV_NVFP4) {   // dims 32q .. 32q+31: groups 2q and 2q+1
        uint2 a, b;
        uint32_t sc;
        if (from_lds) {
          a = nk.codes[i][kv][2 * q];
          b = nk.codes[i][kv][2 * q + 1];
          sc = nk.scales[i][kv][2 * q] | (static_cast<uint32_t>(nk.scales[i][kv][2 * q + 1]) << 8);
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(src + (static_cast<int64_t>(i) * app.hkv + g) * kHeadDim + 32 * q);
          const float t = kv == 0 ? app.k_t : app.v_t;
          const uint32_t sa = nvfp4_encode16_bits(p[0], p[1], t, a.x, a.y);
          const uint32_t sb = nvfp4_encode16_bits(p[2], p[3], t, b.x, b.y);
          sc = sa | (sb << 8);
        }
        uint32_t* scales = kv == 0 ? R.ks : R.vs;
        if (u == 0) { codes[0] = make_uint4(a.x, a.y, b.x, b.y); scales[0] = sc; }
        else { codes[1] = make_uint4(a.x, a.y, b.x, b.y); scales[1] = sc; }
      } else {
        uint4 a, b;
        if (from_lds) {
          a = nk.codes[i][kv][2 * q];
          b = nk.codes[i][kv][2 * q + 1];
        } else {
          const uint4* p = reinterpret_cast<const uint4*>(src + (static_cast<int64_t>(i) * app.hkv + g) * kHeadDim + 32 * q);
          const float ps = kv == 0 ? kps : vps;
          float x[16];
          bf16x16_to_f32(p[0], p[1], x);
          a = fp8_encode16(x, ps);
          bf16x16_to_f32(p[2], p[3], x);
          b = fp8_encode16(x, ps);
        }
        if (u == 0) { codes[0] = a; codes[1] = b; }
        else { codes[2] = a; codes[3] = b; }
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
