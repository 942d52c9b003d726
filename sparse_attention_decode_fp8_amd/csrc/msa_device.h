// Device helpers shared by the libmsadecode kernels (gfx950 / CDNA4, wave64).
//
// Lane layouts used throughout (v_mfma_f32_16x16x32_f16, measured on gfx950):
//   A operand: lane l holds A[l % 16][8 * (l / 16) + i], i = 0..7
//   B operand: lane l holds B[8 * (l / 16) + i][l % 16], i = 0..7
//   C/D:       lane l holds C[4 * (l / 16) + j][l % 16], j = 0..3
// ds_read_b64_tr_b16: within each 16-lane group, lanes 4j..4j+3 each point at 4
// consecutive 16-bit elements that together form row j (16 elements); lane i then
// receives element i of rows j = 0..3.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_decode.h"

namespace msa {

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half4_t __attribute__((ext_vector_type(4)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float float2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint2_t __attribute__((ext_vector_type(2)));
typedef uint32_t uint4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));

constexpr int kPage = MSA_PAGE_SIZE;
constexpr int kHeadDim = MSA_HEAD_DIM;
constexpr int kIndexDim = MSA_INDEX_DIM;
constexpr int kHeadsPerKv = MSA_HEADS_PER_KV;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even fp32 -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// 2^x as the hardware instruction alone (exp2f adds a range fix-up for results below
// 2^-126). Used for softmax and merge weights, whose arguments are <= 0: a weight
// below 2^-126 of the largest one may come out as zero, which changes no sum.
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x, 0) as one instruction: the median of (x, 0, +inf). Written as fmaxf, the
// compiler first canonicalises x (a second instruction) to honour signalling NaNs,
// which the matrix-core results fed here never are. (Not inline asm: the compiler
// cannot see an asm's register reads, so it would not insert the wait states a
// matrix-core result needs before a vector instruction may read it, once it keeps that
// result in vector rather than accumulator registers.)
// +inf that the compiler cannot see as a constant (an asm with no instruction that only
// claims to rewrite its register): with a constant bound it would rewrite the median
// into a max and canonicalise the operand again.
__device__ __forceinline__ float opaque_inf() {
  float v = __builtin_inff();
  asm("" : "+v"(v));
  return v;
}
__device__ __forceinline__ float relu_raw(float x) { return __builtin_amdgcn_fmed3f(x, 0.0f, opaque_inf()); }

// max(a, b) as one instruction, the median of (a, b, +inf) (no canonicalisation of the
// operands first; for values that are never NaN).
__device__ __forceinline__ float max_raw(float a, float b) { return __builtin_amdgcn_fmed3f(a, b, opaque_inf()); }

// Max / sum over the four lanes l, l^16, l^32, l^48 (the rows of 16 lanes), in every
// lane, with the row swaps of gfx950 (vector ALU; no LDS round trip). The sums pair
// the operands as (row0 + row1) + (row2 + row3), in every lane.
__device__ __forceinline__ float rows_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = max_raw(__uint_as_float(r[0]), __uint_as_float(r[1]));
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return max_raw(__uint_as_float(t[0]), __uint_as_float(t[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float a = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  const auto t = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
  return __uint_as_float(t[0]) + __uint_as_float(t[1]);
}
// Max over each row of 16 lanes, delivered to the row's first lane (DPP row shifts
// towards lane 0; lanes a shift has no source for keep -inf).
__device__ __forceinline__ float row_max_to_first(float x) {
  constexpr int kNegInf = static_cast<int>(0xff800000u);
  x = max_raw(x, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(x), 0x101, 0xf, 0xf, false)));
  x = max_raw(x, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(x), 0x102, 0xf, 0xf, false)));
  x = max_raw(x, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(x), 0x104, 0xf, 0xf, false)));
  x = max_raw(x, __int_as_float(__builtin_amdgcn_update_dpp(kNegInf, __float_as_int(x), 0x108, 0xf, 0xf, false)));
  return x;
}

// Two OCP E4M3FN codes (bytes 0 and 1 of `v`, or bytes 2 and 3 with kHi) -> two exact
// fp16 values. The convert picks the half word itself, so no shift or extract first.
template <bool kHi = false>
__device__ __forceinline__ half2_t e4m3x2_to_f16(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, 1.0f, kHi);
}

// Two E2M1 codes (byte `sel` of `v`: low nibble first) -> two exact fp16 values.
template <int kSel>
__device__ __forceinline__ half2_t e2m1x2_to_f16(uint32_t v) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(v, 1.0f, kSel);
}

// One E4M3 code (byte 0 of v) -> exact fp32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t v) {
  return __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(v & 0xffu), false)[0];
}

__device__ __forceinline__ float4_t mfma16x16x32(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 8 E4M3 codes (two dwords) -> 8 fp16 values in one MFMA operand.
__device__ __forceinline__ half8_t e4m3x8_to_f16(uint32_t lo, uint32_t hi) {
  half2_t a = e4m3x2_to_f16<false>(lo), b = e4m3x2_to_f16<true>(lo);
  half2_t c = e4m3x2_to_f16<false>(hi), d = e4m3x2_to_f16<true>(hi);
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// 8 E2M1 codes (one dword, element 0 in the low nibble) times an fp16 scale.
__device__ __forceinline__ half8_t e2m1x8_to_f16(uint32_t v, half2_t scale2) {
  half2_t a = e2m1x2_to_f16<0>(v) * scale2;
  half2_t b = e2m1x2_to_f16<1>(v) * scale2;
  half2_t c = e2m1x2_to_f16<2>(v) * scale2;
  half2_t d = e2m1x2_to_f16<3>(v) * scale2;
  return half8_t{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Power-of-two exponent e such that amax * 2^e lies in [2^14, 2^15): converting
// bf16 values times 2^e to fp16 is then exact down to amax * 2^-28.
__device__ __forceinline__ int f16_prescale_exp(float amax) {
  if (!(amax > 0.0f) || !(amax < 3.0e38f)) return 0;
  int ex;
  frexpf(amax, &ex);           // amax = m * 2^ex, m in [0.5, 1)
  return 15 - ex;
}

// Wave-wide OR / AND / max of a 32-bit value with DPP moves (row shifts 1, 2, 4, 8 within each
// row of 16 lanes, then the row broadcasts of lanes 15 and 31), read back from lane 63:
// vector ALU only, no LDS round trips. Lanes a move has no source for keep the
// identity (0 for OR, all ones for AND).
__device__ __forceinline__ uint32_t wave_or(uint32_t v) {
  int x = static_cast<int>(v);
  x |= __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x |= __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x |= __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x |= __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x |= __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x |= __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}
__device__ __forceinline__ uint32_t wave_and(uint32_t v) {
  int x = static_cast<int>(v);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x111, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x112, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x114, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x118, 0xf, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x142, 0xa, 0xf, false);
  x &= __builtin_amdgcn_update_dpp(-1, x, 0x143, 0xc, 0xf, false);
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}
// Inclusive prefix sum over the wave's lanes in lane order, the same moves (identity 0):
// lane L gets v(0) + ... + v(L), lane 63 the total. Counts from several registers per
// lane summed this way replace one ballot and popcount per register.
__device__ __forceinline__ uint32_t wave_scan_add_u32(uint32_t v) {
  int x = static_cast<int>(v);
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31
  return static_cast<uint32_t>(x);
}
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wave_scan_add_u32(v)), 63));
}
// Wave-wide unsigned maximum, the same moves (identity 0).
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t x = v;
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x111, 0xf, 0xf, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x112, 0xf, 0xf, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x114, 0xf, 0xf, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x118, 0xf, 0xf, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x142, 0xa, 0xf, false)));
  x = max(x, static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), 0x143, 0xc, 0xf, false)));
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(x), 63));
}

// Agent-scope coherent 16- and 8-byte accesses through a buffer resource: the sc1
// cache-policy bit makes them coherent across the XCDs (each has its own L2), so one
// workgroup can read what another wrote in the same launch once the writer's wait on
// the vector memory counter and a device-scope atomic order the two. Offsets are in
// bytes from the resource's base; the range is [base, base + bytes).
constexpr int kCoherentPolicy = 16;   // sc1
// Non-temporal cache policy (nt) for data read once per step: the NVFP4 page codes of
// the decode and the index keys of the scorer. Measured: the scorer 6.6 -> 6.1 us and
// the decode 10.1 -> 9.8 us at the 8 x 32k NVFP4 workload (the FP8 page loads keep the
// default policy, which measured faster for them).
constexpr int kStreamPolicy = 2;
// A 16-byte load with the non-temporal policy.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(x[0], x[1], x[2], x[3]);
}
// A pointer the caller knows to be the same in every lane, moved to scalar registers
// (a resource built from it then needs no per-lane loop).
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<T*>((static_cast<uint64_t>(hi) << 32) | lo);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(uint4_t, v), r, static_cast<int>(off), 0,
                                         kCoherentPolicy);
}
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off, float2_t v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(uint2_t, v), r, static_cast<int>(off), 0,
                                        kCoherentPolicy);
}
__device__ __forceinline__ float4_t load_coherent4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float4_t, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0,
                                                                          kCoherentPolicy));
}
__device__ __forceinline__ float load_coherent1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(off), 0, kCoherentPolicy));
}
__device__ __forceinline__ float2_t load_coherent2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2_t, __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(off), 0,
                                                                         kCoherentPolicy));
}

// Split-merge slots hold MSA_MERGE_IDLE_BITS (a signalling NaN) until written. A
// written value is canonicalised first, which turns a signalling NaN into a quiet one
// and leaves every other value as it is, so no written word carries the pattern.
__device__ __forceinline__ float not_idle(float v) { return __builtin_canonicalizef(v); }
// min over the words of (word ^ pattern): zero exactly when some word still holds the
// pattern. Plain vector arithmetic, no compares into scalar masks.
__device__ __forceinline__ uint32_t idle_key(uint32_t acc, float v) {
  return min(acc, __float_as_uint(v) ^ MSA_MERGE_IDLE_BITS);
}
__device__ __forceinline__ uint32_t idle_key(uint32_t acc, float2_t v) { return idle_key(idle_key(acc, v[0]), v[1]); }
__device__ __forceinline__ uint32_t idle_key(uint32_t acc, float4_t v) {
  return idle_key(idle_key(idle_key(idle_key(acc, v[0]), v[1]), v[2]), v[3]);
}
// Zero that the compiler must treat as differing between lanes (an asm result): added
// to an address, it keeps a load's result in a vector register.
// Device-side metadata check of the debug library (built with MSA_DEBUG_CHECKS): a
// failed check records its msa_debug_error_t code in the caller's error word (if it is
// still 0) and returns false, and the caller skips the access the check guards. The
// release library trusts the metadata: the check is always true and compiles away.
__device__ __forceinline__ bool dcheck(bool ok, int32_t code, int32_t* err) {
#ifdef MSA_DEBUG_CHECKS
  if (!ok && err != nullptr) atomicCAS(err, 0, code);
  return ok;
#else
  (void)code;
  (void)err;
  return true;
#endif
}

// Checked metadata of the debug library: a value out of range is recorded and replaced
// by 0, which keeps every access in bounds (the results are then meaningless).
__device__ __forceinline__ int checked_seq(int seq, int num_seqs, int32_t* err) {
  return dcheck(seq >= 0 && seq < num_seqs, MSA_DEBUG_BAD_SEQ, err) ? seq : 0;
}
__device__ __forceinline__ int64_t checked_page(int64_t page, int num_pages, int32_t* err) {
  return dcheck(page >= 0 && page < num_pages, MSA_DEBUG_BAD_PAGE, err) ? page : 0;
}
// A row position is valid when it is not negative and its block is inside the table.
__device__ __forceinline__ void check_pos(int pos, int max_blocks, int32_t* err) {
  dcheck(pos >= 0 && pos / MSA_PAGE_SIZE < max_blocks, MSA_DEBUG_BAD_POS, err);
}

__device__ __forceinline__ int lane_varying_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}

// Most splits the combining decode merges in one launch.
constexpr int kMaxMergeSplits = 16;

// Merge state word of one (row, KV head) pair in the combining decode's workspace: bit
// 31 = which of the two exchange buffers the next launch uses, bits 26..30 = the split
// count the workspace was set up for, bit 25 = kMergeTimeoutBit (which makes the word
// invalid), bits 8..22 = slices handed to the last split by merging splits that gave up
// waiting for it (kMergeHandoffShift), bits 0..7 = splits arrived in the current launch.
__host__ __device__ __forceinline__ uint32_t merge_state(int buffer, int num_splits) {
  return (static_cast<uint32_t>(buffer) << 31) | (static_cast<uint32_t>(num_splits) << 26);
}
constexpr uint32_t kMergeArrivalMask = 0xffu;
constexpr int kMergeHandoffShift = 8;
constexpr uint32_t kMergeHandoffMask = 0x7fffu << kMergeHandoffShift;
// Set for good by a merger that gave up polling: every later launch finds the word
// invalid until the workspace is set up again.
constexpr uint32_t kMergeTimeoutBit = 1u << 25;
__device__ __forceinline__ bool merge_state_ok(uint32_t w, int num_splits) {
  return ((w >> 26) & 0x1fu) == static_cast<uint32_t>(num_splits) && (w & kMergeTimeoutBit) == 0u &&
         (w & kMergeArrivalMask) < static_cast<uint32_t>(num_splits);
}
// The split merge of a pair's 16 heads is shared by its last merge_slices(S) splits to
// arrive, each taking 16 / merge_slices(S) heads: the largest power of two not above S
// (at most 16, one head each; the handoff field holds one bit for each slice but the
// last).
__host__ __device__ __forceinline__ int merge_slices(int num_splits) {
  int k = 1;
  while (2 * k <= num_splits && 2 * k <= kMaxMergeSplits) k *= 2;
  return k;
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS accesses, not for
// its outstanding global stores.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Request a row belongs to when every request has the same number of rows (the
// multiplier comes from seq_guess_mul on the host); callers check it against row_seq.
__device__ __forceinline__ int seq_guess(int r, uint64_t mul) {
  return static_cast<int>((static_cast<uint64_t>(r) * mul) >> 32);
}

// Order-preserving map of fp32 onto uint32 (larger float -> larger key).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- encoders
// Saturating round-to-nearest-even fp32 -> OCP E4M3 (largest finite 448). The input is
// clamped to +-448 first, so the hardware conversion (which rounds to nearest even)
// never overflows; every magnitude above 448 becomes 448. The sign of zero is kept.
__device__ __forceinline__ float e4m3_clamp(float x) { return __builtin_amdgcn_fmed3f(x, -448.0f, 448.0f); }
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const float c = e4m3_clamp(x);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false)) & 0xffu;
}
// Four values -> four E4M3 codes, first value in the low byte.
__device__ __forceinline__ uint32_t f32x4_to_e4m3_sat(float a, float b, float c, float d) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), 0, false);
  return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(c), e4m3_clamp(d), lo, true));
}

// Saturating round-to-nearest-even fp32 -> E2M1 (sign bit 3). Grid
// {0, .5, 1, 1.5, 2, 3, 4, 6}; each comparison is one decision boundary, with the
// tie at the boundary going to the even code.
__device__ __forceinline__ uint32_t f32_to_e2m1_sat(float x) {
  uint32_t sign = (__float_as_uint(x) >> 28) & 0x8u;
  float a = fabsf(x);
  uint32_t c = (a > 0.25f) + (a >= 0.75f) + (a > 1.25f) + (a >= 1.75f) + (a > 2.5f) +
               (a >= 3.5f) + (a > 5.0f);
  return sign | c;
}

}  // namespace msa
