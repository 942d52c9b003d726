// Append encoder shared by msa_kv_append and the fused append/score/select kernel.
//
// One call encodes one group of 16 contiguous elements of one new token: an NVFP4
// scale group, or 16 FP8 / index-key codes. A token never touches another token's
// bytes, so no atomics are needed. [GB300] "Step-loop runtime hooks" names the KV
// update as its own step; [Rubin] Description requires saturating FP8 casts.
#pragma once

#include "msa_device.h"
#include "msa_host.h"

namespace msa {

struct AppendArgs {
  const int64_t* slot;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* idx_new;
  uint8_t* k_codes;
  uint8_t* v_codes;
  uint8_t* k_scales;   // NVFP4: e4m3 bytes; FP8: fp32 page scales
  uint8_t* v_scales;
  uint8_t* index_k;
  uint8_t* index_scales;   // NVFP4 index keys: e4m3 bytes [pages][128][index_dim / 16]
  float k_t, v_t, idx_t;
  int index_nvfp4;
  int n_new, hkv;
  int num_pages;
  int32_t* err;        // debug library: the error word of failed metadata checks
  int kv_groups;       // groups of 16 per token for K (and for V): hkv * 8
  int groups_per_tok;  // K groups + V groups + index groups
};

__device__ __forceinline__ void load16_bf16(const uint16_t* src, float x[16]) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
  uint4 a = p[0], b = p[1];
  uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(w[i] << 16);
    x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// 16 bf16 values (as loaded: two 16-byte words) -> 16 saturating E4M3 codes (no
// scale), packed little-endian.
__device__ __forceinline__ uint4 encode_index16_bits(uint4 a, uint4 b) {
  const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float x[16];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(wv[i] << 16);
    x[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
  }
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) w[i] = f32x4_to_e4m3_sat(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ uint4 encode_index16(const uint16_t* src) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
  return encode_index16_bits(p[0], p[1]);
}

// One NVFP4 group: 16 values at tensor scale t -> 16 E2M1 codes (element 2j in the low
// nibble of byte j, as w0 | w1 << 32) and the E4M3 scale code. amax = max|x|,
// sc = E4M3(amax / (6 t)); a zero decoded scale gives all codes +0; otherwise
// d = E4M3(sc) * t and code_i = E2M1(x_i / d). Every operation is a correctly rounded
// fp32 operation (contraction off).
__device__ __forceinline__ uint32_t nvfp4_encode16(const float x[16], float t, uint32_t& w0, uint32_t& w1) {
#pragma clang fp contract(off)
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const float six_t = 6.0f * t;
  const uint32_t sc = f32_to_e4m3_sat(amax / six_t);
  const float dec = e4m3_to_f32(sc);
  w0 = 0;
  w1 = 0;
  if (dec != 0.0f) {
    const float d = dec * t;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      w0 |= f32_to_e2m1_sat(x[i] / d) << (4 * i);
      w1 |= f32_to_e2m1_sat(x[8 + i] / d) << (4 * i);
    }
  }
  return sc;
}

// 16 bf16 values as loaded (two 16-byte words) -> fp32.
__device__ __forceinline__ void bf16x16_to_f32(uint4 a, uint4 b, float x[16]) {
  const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[2 * i] = __uint_as_float(wv[i] << 16);
    x[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
  }
}

// 16 bf16 values (two 16-byte words as loaded) -> one NVFP4 group.
__device__ __forceinline__ uint32_t nvfp4_encode16_bits(uint4 a, uint4 b, float t, uint32_t& w0, uint32_t& w1) {
  float x[16];
  bf16x16_to_f32(a, b, x);
  return nvfp4_encode16(x, t, w0, w1);
}

// 16 values -> 16 saturating E4M3 codes of x / s, packed little-endian (the FP8 KV
// encoding at page scale s; one correctly rounded fp32 division per value).
__device__ __forceinline__ uint4 fp8_encode16(const float x[16], float s) {
#pragma clang fp contract(off)
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = f32x4_to_e4m3_sat(x[4 * i] / s, x[4 * i + 1] / s, x[4 * i + 2] / s, x[4 * i + 3] / s);
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Encode group `gid` (token gid / groups_per_tok) of the new tokens into the pool.
template <int kFmt>
__device__ __forceinline__ void append_group(const AppendArgs& a, int64_t gid) {
#pragma clang fp contract(off)
  const int tok = static_cast<int>(gid / a.groups_per_tok);
  int grp = static_cast<int>(gid % a.groups_per_tok);
  const int64_t slot = a.slot[tok];
  if (slot < 0) return;
  const int64_t page = slot / kPage;
  const int off = static_cast<int>(slot % kPage);
  if (!dcheck(page < a.num_pages, MSA_DEBUG_BAD_SLOT, a.err)) return;

  if (grp >= 2 * a.kv_groups) {                    // index-K: E4M3, no scale, or NVFP4
    if (a.idx_new == nullptr) return;
    const int g = grp - 2 * a.kv_groups;             // 0..3
    const uint16_t* src = a.idx_new + static_cast<int64_t>(tok) * kIndexDim + 16 * g;
    const int64_t row = page * kPage + off;
    if (a.index_nvfp4) {
      // group-major page layout: group g of token 16 t + n at [g][n][t]
      const uint4* p = reinterpret_cast<const uint4*>(src);
      uint32_t w0, w1;
      const uint32_t sc = nvfp4_encode16_bits(p[0], p[1], a.idx_t, w0, w1);
      const int64_t at = (page * (kIndexDim / 16) + g) * kPage + (off % 16) * 8 + off / 16;
      *reinterpret_cast<uint2*>(a.index_k + at * 8) = make_uint2(w0, w1);
      a.index_scales[at] = static_cast<uint8_t>(sc);
    } else {
      *reinterpret_cast<uint4*>(a.index_k + row * kIndexDim + 16 * g) = encode_index16(src);
    }
    return;
  }
  const bool is_v = grp >= a.kv_groups;
  if (is_v) grp -= a.kv_groups;
  const uint16_t* src = is_v ? a.v_new : a.k_new;
  if (src == nullptr) return;
  const int h = grp >> 3, g = grp & 7;
  float x[16];
  load16_bf16(src + (static_cast<int64_t>(tok) * a.hkv + h) * kHeadDim + 16 * g, x);
  const int64_t row = (page * a.hkv + h) * kPage + off;   // token row inside the pool

  if constexpr (kFmt == MSA_KV_NVFP4) {
    uint32_t w0, w1;
    const uint32_t sc = nvfp4_encode16(x, is_v ? a.v_t : a.k_t, w0, w1);
    uint8_t* codes = is_v ? a.v_codes : a.k_codes;
    uint8_t* scales = is_v ? a.v_scales : a.k_scales;
    *reinterpret_cast<uint2*>(codes + row * (kHeadDim / 2) + 8 * g) = make_uint2(w0, w1);
    scales[row * (kHeadDim / 16) + g] = static_cast<uint8_t>(sc);
  } else {
    const float s = reinterpret_cast<const float*>(is_v ? a.v_scales : a.k_scales)[page];
    uint8_t* codes = is_v ? a.v_codes : a.k_codes;
    *reinterpret_cast<uint4*>(codes + row * kHeadDim + 16 * g) = fp8_encode16(x, s);
  }
}

// Fill the append arguments from a pool and the new tokens.
inline AppendArgs make_append_args(const msa_kv_pool_t* pool, int32_t n_new, const int64_t* slot,
                                   const void* k_new, const void* v_new, const void* idx_k_new) {
  AppendArgs a;
  a.slot = slot;
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.idx_new = static_cast<const uint16_t*>(idx_k_new);
  a.k_codes = static_cast<uint8_t*>(pool->k_codes);
  a.v_codes = static_cast<uint8_t*>(pool->v_codes);
  a.k_scales = static_cast<uint8_t*>(pool->k_scales);
  a.v_scales = static_cast<uint8_t*>(pool->v_scales);
  a.index_k = static_cast<uint8_t*>(pool->index_k);
  a.index_scales = static_cast<uint8_t*>(pool->index_scales);
  a.index_nvfp4 = pool->index_fmt == MSA_INDEX_NVFP4;
  a.k_t = pool->k_tensor_scale;
  a.v_t = pool->v_tensor_scale;
  a.idx_t = pool->index_tensor_scale;
  a.n_new = n_new;
  a.hkv = pool->num_kv_heads;
  a.num_pages = pool->num_pages;
  a.err = debug_error_word();
  a.kv_groups = pool->num_kv_heads * (MSA_HEAD_DIM / 16);
  a.groups_per_tok = 2 * a.kv_groups + MSA_INDEX_DIM / 16;
  return a;
}

}  // namespace msa
