// msa_index_score: per-token index score, max-pooled over 128-token blocks; and
// msa_append_score_select: KV append + index score + top-k select in one launch.
//
// The scorer streams every visible token's 64-byte E4M3 index key once per request
// ([GB300] "The TP4 decode target": an index scorer reading index-K pages; [Rubin]
// commit messages: a proxy max-score pass producing one score per block). The
// per-block contraction is [128 tokens x 64] . [64 x (rows * heads)], done on the
// matrix cores with fp16 operands (E4M3 keys convert exactly; bf16 queries are
// pre-scaled by a power of two per (row, head) so the conversion is exact) and fp32
// accumulation.
//
// Work split: one wave per (group of rows of one request, block). A group holds up
// to 16 / Hi consecutive rows of the same request, so a request's index keys are read
// once for all of its query rows. MFMA A = queries (M = row * Hi + head), B = keys
// (N = 16 tokens), so lane (n, q) ends up with all heads of row-slot q for token n:
// the head sum is in-lane and its order never depends on the token's position.
//
// Fused launch ([GB300] "The TP4 decode target" fuses long-context block selection and
// the KV update into its attention megakernels; the TP8 target fuses index scoring
// with block selection): extra workgroups append the new tokens; scoring waves whose
// page receives a new token encode that token's index key themselves (same encoder)
// instead of waiting for the append; the scores are stored write-through (agent
// coherent) and the last scoring workgroup of a row group, found with a counter,
// runs the selection for those rows.
#include <type_traits>

#include "append_device.h"
#include "msa_host.h"
#include "score_device.h"
#include "select_device.h"

namespace msa {
namespace {

// Waves (blocks) per scoring workgroup: 2, or 4 where the launch's last workgroup of a
// row group runs the block radix select (which takes 256 threads). Smaller workgroups
// measured slightly faster at every workload (scores are identical).
constexpr int score_waves(bool selects) { return selects ? 4 : 2; }

struct ScoreArgs {
  const uint8_t* index_k;
  const uint8_t* index_scales;   // NVFP4 index keys: e4m3 [pages][128][4]
  float idx_t;                   // NVFP4 index tensor scale
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_pos;
  const uint16_t* q_idx;
  const float* w;
  float* scores;
  int num_rows, max_blocks;
  int num_seqs, num_pages;
  int32_t* err;       // debug library: the error word of failed metadata checks
  uint64_t seq_mul;   // seq_guess multiplier
  // fused launch only
  AppendArgs app;
  int k, n_init, n_local;
  int32_t* sel;
  int32_t* sel_pages;
  int32_t* counters;
  int score_wgs_x;   // workgroups along x that score blocks
  int append_row;    // fused launch: 1 if grid row 0 holds the append workgroups
  // > 0: every request has this many rows, and the grid has one row per group of
  // rows (groups_per_seq per request) instead of one per query row
  int rows_per_seq, groups_per_seq;
};

// kG score tables per row: table t sums the index heads [t * kHi / kG, (t + 1) * kHi / kG).
template <int kHi, int kG, int kFmt, bool kFused, bool kIdxNv, int kWaves>
__global__ void __launch_bounds__(64 * kWaves) score_kernel(ScoreArgs a) {
  static_assert(kHi % kG == 0, "index heads split evenly into the tables");
  constexpr int kHpg = kHi / kG;
  extern __shared__ uint32_t sel_keys[];        // fused: selection scratch [max_blocks]
  __shared__ SelectSmem sm;
  __shared__ int s_last;
  constexpr int kRowsPerGroup = 16 / kHi;
  constexpr int kRowsPerLane = 4 / kHi;
  if constexpr (kFused) {
    // The append workgroups form grid row 0 (when there is anything to append), so
    // they are dispatched first and run alongside the scoring.
    if (a.append_row && blockIdx.y == 0) {
      const int64_t gid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
      if (gid < static_cast<int64_t>(a.app.n_new) * a.app.groups_per_tok) append_group<kFmt>(a.app, gid);
      return;
    }
    if (static_cast<int>(blockIdx.x) >= a.score_wgs_x) return;
  }
  // The group's first row: grid row y - append_row is row r0 itself, or, with a stated
  // row count per request, group (request, i) of that request's rows.
  int r0 = static_cast<int>(blockIdx.y) - a.append_row;
  if (a.rows_per_seq > 0) r0 = (r0 / a.groups_per_seq) * a.rows_per_seq + (r0 % a.groups_per_seq) * kRowsPerGroup;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 15, q = lane >> 4;
  const int b = blockIdx.x * kWaves + wave;

  // Row metadata in one round of loads: lanes 0..31 read row_seq of rows r0-32 .. r0-1,
  // lanes 32..47 row_seq and row_pos of rows r0 .. r0+15, and every lane the block-table
  // entry of block b for the request r0 belongs to when every request has the same
  // number of rows (checked below, and read again if wrong).
  const int rr = r0 - 32 + lane;
  const bool in_rows = lane < 48 && rr >= 0 && rr < a.num_rows;
  const int seq_l = in_rows ? a.row_seq[rr] : -1;
  const int pos_l = in_rows && lane >= 32 ? a.row_pos[rr] : -1;
  const int guess = seq_guess(r0, a.seq_mul);
  const int page_g = b < a.max_blocks ? a.block_table[static_cast<int64_t>(guess) * a.max_blocks + b] : -1;
  // fused launch: the first 64 new tokens' slots, so that matching them against the
  // page below waits for no further load
  int64_t slot0 = -1;
  if constexpr (kFused)
    if (a.app.idx_new != nullptr && lane < a.app.n_new) slot0 = a.app.slot[lane];
  const int seq_raw = __builtin_amdgcn_readlane(seq_l, 32);
  const uint64_t same = __ballot(seq_l == seq_raw);
  // Is r0 the first row of a group? Count the earlier rows of the same request.
  const uint32_t before = ~static_cast<uint32_t>(same);            // lanes 0..31: a different request
  int j = before != 0 ? __builtin_clz(before) : 32;               // run of equal rows ending at r0-1
  if (j == 32)
    while (r0 - j - 1 >= 0 && a.row_seq[r0 - j - 1] == seq_raw) ++j;
  // (a stated row count per request puts r0 at a group's start: checked by the debug
  // library, trusted by the release one)
  dcheck(a.rows_per_seq == 0 || (j % kRowsPerGroup == 0 && seq_raw == r0 / a.rows_per_seq), MSA_DEBUG_BAD_SEQ,
         a.err);
  if (j % kRowsPerGroup != 0) return;
  // rows r0 .. r0+nr-1 of the same request form the group
  const uint32_t after = ~static_cast<uint32_t>(same >> 32);       // bit i: row r0+i differs
  const int nr = min(kRowsPerGroup, __builtin_ctz(after | (1u << 16)));
  int max_pos = lane >= 32 && lane < 32 + nr ? pos_l : -1;
  if (lane >= 32 && lane < 32 + nr && blockIdx.x == 0) check_pos(pos_l, a.max_blocks, a.err);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) max_pos = max(max_pos, __shfl_xor(max_pos, m, 64));
  const int last_block = max_pos / kPage;
  const int seq = checked_seq(seq_raw, a.num_seqs, a.err);

  const bool active = b < a.max_blocks && b <= last_block;   // this wave scores block b
  const bool fill = b < a.max_blocks && b > last_block;      // past every row: -inf only

  if (active) {
    // The query-side loads go out before the key loads: the vector memory counter
    // retires in order, so converting the queries waits for them alone.
    // A operand: lane (m, q) holds query row-slot m / Hi, head m % Hi, dims
    // 16q + 8ks .. +7, times 2^e (e per (row, head), from the amax over 64 dims).
    const int m = n;
    const int rs = m / kHi, hd = m % kHi;
    uint4 qa0 = make_uint4(0u, 0u, 0u, 0u), qa1 = qa0;
    if (rs < nr) {
      const uint16_t* qp = a.q_idx + (static_cast<int64_t>(r0 + rs) * kHi + hd) * kIndexDim + 16 * q;
      qa0 = reinterpret_cast<const uint4*>(qp)[0];
      qa1 = reinterpret_cast<const uint4*>(qp)[1];
    }
    // After the MFMA, lane (n, q) holds M = 4q + jj: the matching (row, head) weight.
    float wj[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int mm = 4 * q + jj;
      const int rr = mm / kHi, hh = mm % kHi;
      wj[jj] = rr < nr ? a.w[static_cast<int64_t>(r0 + rr) * kHi + hh] : 0.0f;
    }
    int rowslot[kRowsPerLane], pos[kRowsPerLane];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
      rowslot[i] = q * kRowsPerLane + i;
      pos[i] = rowslot[i] < nr ? a.row_pos[r0 + rowslot[i]] : -1;
    }

    // All key loads of the block: lane (n, q) reads its share of tokens 16t + n, dims
    // 16q .. 16q+15 (k-step 0 uses the first 8, k-step 1 the last 8): 16 E4M3 bytes per
    // t, or (NVFP4) 8 code bytes and the group's scale byte per t. They are issued from the
    // guessed request's page (an unused entry reads page 0) and issued again from the
    // right page if the guess was wrong.
    int64_t page = page_g;
    uint4 key[8];
    auto load_keys = [&]() {
      const int64_t tok0 = page * kPage + n;
      if constexpr (kIdxNv) {
        // group-major page: lane (n, q)'s 8 token rows are 64 contiguous code bytes and
        // 8 contiguous scale bytes
        const int64_t at = (page * (kIndexDim / 16) + q) * kPage + n * 8;
        const uint4* kp = reinterpret_cast<const uint4*>(a.index_k + at * 8);
        const uint4 c0 = load_stream16(kp), c1 = load_stream16(kp + 1), c2 = load_stream16(kp + 2),
                    c3 = load_stream16(kp + 3);
        const uint2 sc = *reinterpret_cast<const uint2*>(a.index_scales + at);
        const uint4 c[4] = {c0, c1, c2, c3};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const uint4 ct = c[t >> 1];
          const uint32_t sw = t < 4 ? sc.x : sc.y;
          key[t] = (t & 1) ? make_uint4(ct.z, ct.w, (sw >> (8 * (t & 3))) & 0xffu, 0u)
                           : make_uint4(ct.x, ct.y, (sw >> (8 * (t & 3))) & 0xffu, 0u);
        }
      } else {
        const uint8_t* kp = a.index_k + tok0 * kIndexDim + 16 * q;
#pragma unroll
        for (int t = 0; t < 8; ++t) key[t] = load_stream16(kp + t * 16 * kIndexDim);
      }
    };
    if (seq != guess) page = a.block_table[static_cast<int64_t>(seq) * a.max_blocks + b];
    page = checked_page(page, a.num_pages, a.err);
    if (page < 0) page = 0;   // (an entry of -1 here is invalid input: read page 0, not before the pool)
    // New tokens landing in this page (fused launch): their keys are encoded here from
    // the bf16 source instead of waiting for the append. The first one's source is
    // read together with the page's keys and its code replaces the stale key as the
    // operand is formed; any further ones (several new tokens in one page, or more than
    // 64 new tokens) overwrite the key registers afterwards.
    int pt = -1;                                   // token row (0..7) this lane patches
    uint4 pv = make_uint4(0u, 0u, 0u, 0u), pv1 = pv;
    bool patch_more = false;
    if constexpr (kFused) {
      if (a.app.idx_new != nullptr) {
        const uint64_t h0 = __ballot(slot0 >= 0 && slot0 / kPage == page);
        patch_more = a.app.n_new > 64 || (h0 & (h0 - 1)) != 0;
        if (h0 != 0) {
          const int first = __ffsll(static_cast<unsigned long long>(h0)) - 1;
          const int off0 = __builtin_amdgcn_readlane(static_cast<int>(slot0 % kPage), first);
          if ((off0 & 15) == n) {
            const uint4* src = reinterpret_cast<const uint4*>(
                a.app.idx_new + static_cast<int64_t>(first) * kIndexDim + 16 * q);
            pv = src[0];
            pv1 = src[1];
            pt = off0 >> 4;
          }
        }
      }
    }
    load_keys();
    if (pt >= 0) pv = encode_key16<kIdxNv>(pv, pv1, a.idx_t);

    float qa[16];
    {
      const uint32_t wv[8] = {qa0.x, qa0.y, qa0.z, qa0.w, qa1.x, qa1.y, qa1.z, qa1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        qa[2 * i] = __uint_as_float(wv[i] << 16);
        qa[2 * i + 1] = __uint_as_float(wv[i] & 0xffff0000u);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(qa[i]));
    amax = rows_max(amax);
    const int e = f16_prescale_exp(amax);
    half8_t A0, A1;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      A0[i] = static_cast<half_t>(ldexpf(qa[i], e));
      A1[i] = static_cast<half_t>(ldexpf(qa[8 + i], e));
    }
    // Head weight times the inverse pre-scale of the (row, head) that lane (n, q)'s
    // result M = 4q + jj has: the scale is positive, so w * relu(x * inv) =
    // (w * inv) * relu(x) (exactly for E4M3 keys, whose scale is a power of two; up to
    // rounding with the NVFP4 keys' tensor scale folded in).
    float wi[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float inv = ldexpf(1.0f, -__shfl(e, 4 * q + jj, 64));
      if constexpr (kIdxNv) inv *= a.idx_t;   // NVFP4 keys: their tensor scale (> 0)
      wi[jj] = wj[jj] * inv;
    }

    if constexpr (kFused) {
      // New tokens landing in this page: encode their keys here (the append runs
      // concurrently in other workgroups).
      if (patch_more) {
        for (int base = 0; base < a.app.n_new; base += 64) {
          const int i = base + lane;
          const int64_t sl = base == 0 ? slot0 : i < a.app.n_new ? a.app.slot[i] : -1;
          uint64_t hits = __ballot(sl >= 0 && sl / kPage == page);
          if (base == 0) hits &= hits - 1;         // the first one is patched at the operand
          while (hits) {
            const int jj = __ffsll(static_cast<unsigned long long>(hits)) - 1;
            hits &= hits - 1;
            const int off = __builtin_amdgcn_readlane(static_cast<int>(sl % kPage), jj);
            if ((off & 15) == n) {
              const uint4* src = reinterpret_cast<const uint4*>(
                  a.app.idx_new + static_cast<int64_t>(base + jj) * kIndexDim + 16 * q);
              const uint4 v = encode_key16<kIdxNv>(src[0], src[1], a.idx_t);
#pragma unroll
              for (int t = 0; t < 8; ++t)
                if (t == (off >> 4)) key[t] = v;
            }
          }
        }
      }
    }

    // The first new token's key replaces its stale row, in the waves that have one.
    if (__ballot(pt >= 0) != 0) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (t == pt) key[t] = pv;
    }
    float best[kRowsPerLane][kG];
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i)
#pragma unroll
      for (int t = 0; t < kG; ++t) best[i][t] = -INFINITY;
    // Tokens past a row's position are masked only in a block that holds one (the
    // last visible block of some row of the group); elsewhere the loop skips the test.
    bool ends_here = false;
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) ends_here |= rowslot[i] < nr && b * kPage + kPage - 1 > pos[i];
    auto score_tokens = [&](auto masked) {
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        half8_t B0, B1;
        key_operands<kIdxNv>(key[t], B0, B1);
        float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
        acc = mfma16x16x32(A0, B0, acc);
        acc = mfma16x16x32(A1, B1, acc);
        const int p = b * kPage + 16 * t + n;      // absolute position of this lane's token
#pragma unroll
        for (int i = 0; i < kRowsPerLane; ++i) {
#pragma unroll
          for (int t = 0; t < kG; ++t) {
            float s = 0.0f;
#pragma unroll
            for (int hh = t * kHpg; hh < (t + 1) * kHpg; ++hh) {
              const int jj = i * kHi + hh;
              s = fmaf(wi[jj], relu_raw(acc[jj]), s);
            }
            if constexpr (decltype(masked)::value) {
              if (p <= pos[i]) best[i][t] = max_raw(best[i][t], s);
            } else {
              best[i][t] = max_raw(best[i][t], s);
            }
          }
        }
      }
    };
    if (__ballot(ends_here) != 0) score_tokens(std::true_type{});
    else score_tokens(std::false_type{});
#pragma unroll
    for (int i = 0; i < kRowsPerLane; ++i) {
#pragma unroll
      for (int t = 0; t < kG; ++t) {
        const float v = row_max_to_first(best[i][t]);   // the block maximum, in lane n == 0
        if (n == 0 && rowslot[i] < nr) {
          float* dst = a.scores + (static_cast<int64_t>(r0 + rowslot[i]) * kG + t) * a.max_blocks + b;
          // write-through only when this launch's last workgroup selects from the scores;
          // a later kernel sees plain stores after the kernel boundary
          if (kFused && a.counters != nullptr) __hip_atomic_store(dst, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else *dst = v;
        }
      }
    }
  } else if (fill) {
    // the group's rows' tables are consecutive: (r0 + i) * kG + t = r0 * kG + lane
    if (lane < nr * kG) a.scores[(static_cast<int64_t>(r0) * kG + lane) * a.max_blocks + b] = -INFINITY;
  }

  // (the selecting launch has 256-thread workgroups; smaller ones never select)
  if constexpr (kFused && 64 * kWaves >= kSelectThreads) {
    if (a.counters == nullptr) return;                 // append + score only
    // The last scoring workgroup of this row group selects for its rows.
    const int nwg = (last_block + kWaves) / kWaves;   // workgroups holding blocks 0..last_block
    if (static_cast<int>(blockIdx.x) >= nwg) return;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's score stores are done
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(a.counters + r0, 1) == nwg - 1;
    __syncthreads();
    if (!s_last) return;
    const int32_t* bt = a.block_table + static_cast<int64_t>(seq) * a.max_blocks;
    for (int i = 0; i < nr * kG; ++i) {
      const int r = r0 + i / kG;
      const int64_t tr = static_cast<int64_t>(r0) * kG + i;      // table row (r, i % kG)
      const int nb = min(a.row_pos[r] / kPage + 1, a.max_blocks);
      block_select_row<true>(a.scores + tr * a.max_blocks, nb, a.k, a.n_init, a.n_local, bt,
                             a.sel + tr * a.k, a.sel_pages ? a.sel_pages + tr * a.k : nullptr,
                             sel_keys, sm);
    }
    if (threadIdx.x == 0) a.counters[r0] = 0;
  }
}

// Per-KV-head score tables: one per KV head, each over an equal share of the index heads.
bool tables_ok(const msa_kv_pool_t* pool, int tables, int n_idx_heads) {
  return tables == 1 || (tables == pool->num_kv_heads && n_idx_heads % tables == 0);
}

ScoreArgs make_score_args(const msa_kv_pool_t* pool, const msa_step_t* step, const void* q_idx,
                          const float* w, float* block_scores) {
  ScoreArgs a{};
  a.index_k = static_cast<const uint8_t*>(pool->index_k);
  a.index_scales = static_cast<const uint8_t*>(pool->index_scales);
  a.idx_t = pool->index_tensor_scale;
  a.block_table = step->block_table;
  a.row_seq = step->row_seq;
  a.row_pos = step->row_pos;
  a.q_idx = static_cast<const uint16_t*>(q_idx);
  a.w = w;
  a.scores = block_scores;
  a.num_rows = step->num_rows;
  a.seq_mul = seq_guess_mul(step->num_seqs, step->num_rows);
  a.max_blocks = step->max_blocks_per_seq;
  a.num_seqs = step->num_seqs;
  a.num_pages = pool->num_pages;
  a.err = debug_error_word();
  return a;
}

// Grid rows of the scoring workgroups: one per query row, or, with a stated row count
// per request, one per group of a request's rows (16 / n_idx_heads rows per group).
void set_score_rows(ScoreArgs& a, const msa_step_t* step, int n_idx_heads) {
  const int per_group = 16 / n_idx_heads;
  a.rows_per_seq = step->rows_per_seq;
  a.groups_per_seq = a.rows_per_seq > 0 ? (a.rows_per_seq + per_group - 1) / per_group : 0;
}
int score_rows(const ScoreArgs& a, const msa_step_t* step) {
  return a.rows_per_seq > 0 ? step->num_seqs * a.groups_per_seq : step->num_rows;
}

template <int kFmt, bool kFused, bool kIdxNv, int kWaves>
void launch_score_fmt(const ScoreArgs& a, int hi, int tables, dim3 grid, size_t lds, hipStream_t s) {
  const dim3 block(64 * kWaves);
#define MSA_SCORE_LAUNCH(HI, G) score_kernel<HI, G, kFmt, kFused, kIdxNv, kWaves><<<grid, block, lds, s>>>(a)
  if (hi == 1) MSA_SCORE_LAUNCH(1, 1);
  else if (hi == 2) {
    if (tables == 1) MSA_SCORE_LAUNCH(2, 1);
    else MSA_SCORE_LAUNCH(2, 2);
  } else {
    if (tables == 1) MSA_SCORE_LAUNCH(4, 1);
    else if (tables == 2) MSA_SCORE_LAUNCH(4, 2);
    else MSA_SCORE_LAUNCH(4, 4);
  }
#undef MSA_SCORE_LAUNCH
}

// hi in {1, 2, 4} and tables dividing hi are checked by the caller.
template <bool kFused, int kWaves>
msa_status_t launch_score(const ScoreArgs& a, const msa_kv_pool_t* pool, int hi, int tables, dim3 grid,
                          size_t lds, hipStream_t s) {
  const bool nv = index_nvfp4(pool);
  if (pool->fmt == MSA_KV_NVFP4) {
    if (nv) launch_score_fmt<MSA_KV_NVFP4, kFused, true, kWaves>(a, hi, tables, grid, lds, s);
    else launch_score_fmt<MSA_KV_NVFP4, kFused, false, kWaves>(a, hi, tables, grid, lds, s);
  } else {
    if (nv) launch_score_fmt<MSA_KV_FP8_E4M3, kFused, true, kWaves>(a, hi, tables, grid, lds, s);
    else launch_score_fmt<MSA_KV_FP8_E4M3, kFused, false, kWaves>(a, hi, tables, grid, lds, s);
  }
  return launch_status();
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_index_score(const msa_kv_pool_t* pool, const msa_step_t* step,
                                        int32_t n_idx_heads, const void* q_idx, const float* w,
                                        float* block_scores, void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (n_idx_heads != 1 && n_idx_heads != 2 && n_idx_heads != 4) return MSA_ERR_UNSUPPORTED;
  const int tables = sel_tables(step);
  if (!tables_ok(pool, tables, n_idx_heads)) return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0) return MSA_OK;
  if (q_idx == nullptr || w == nullptr || block_scores == nullptr || !aligned16(q_idx))
    return MSA_ERR_INVALID_ARG;
  if (step->num_rows > 65535) return MSA_ERR_UNSUPPORTED;
  ScoreArgs a = make_score_args(pool, step, q_idx, w, block_scores);
  set_score_rows(a, step, n_idx_heads);
  constexpr int kW = score_waves(false);
  a.score_wgs_x = (step->max_blocks_per_seq + kW - 1) / kW;
  dim3 grid(a.score_wgs_x, score_rows(a, step));
  return launch_score<false, kW>(a, pool, n_idx_heads, tables, grid, 0, static_cast<hipStream_t>(stream));
}

extern "C" msa_status_t msa_append_score_select(
    const msa_kv_pool_t* pool, const msa_step_t* step, int32_t n_new, const int64_t* slot,
    const void* k_new, const void* v_new, const void* idx_k_new, int32_t n_idx_heads,
    const void* q_idx, const float* w, int32_t k, int32_t n_init, int32_t n_local,
    float* block_scores, int32_t* sel, int32_t* sel_pages, int32_t* counters, void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (n_idx_heads != 1 && n_idx_heads != 2 && n_idx_heads != 4) return MSA_ERR_UNSUPPORTED;
  const int tables = sel_tables(step);
  if (!tables_ok(pool, tables, n_idx_heads)) return MSA_ERR_UNSUPPORTED;
  if (k < 1 || k > MSA_MAX_TOPK || n_init < 0 || n_local < 0 || n_init + n_local > k)
    return MSA_ERR_UNSUPPORTED;
  if (n_new < 0) return MSA_ERR_INVALID_ARG;
  if (n_new > 4096) return MSA_ERR_UNSUPPORTED;
  if (n_new > 0 && slot == nullptr) return MSA_ERR_INVALID_ARG;
  for (const void* p : {k_new, v_new, idx_k_new})
    if (p != nullptr && !aligned16(p)) return MSA_ERR_INVALID_ARG;
  if (step->num_rows == 0) {
    return n_new > 0 ? msa_kv_append(pool, n_new, slot, k_new, v_new, idx_k_new, stream) : MSA_OK;
  }
  if (q_idx == nullptr || w == nullptr || block_scores == nullptr || !aligned16(q_idx))
    return MSA_ERR_INVALID_ARG;
  if ((sel == nullptr) != (counters == nullptr)) return MSA_ERR_INVALID_ARG;
  if (step->num_rows >= 65535) return MSA_ERR_UNSUPPORTED;
  ScoreArgs a = make_score_args(pool, step, q_idx, w, block_scores);
  set_score_rows(a, step, n_idx_heads);
  a.app = make_append_args(pool, n_new, slot, k_new, v_new, idx_k_new);
  a.k = k;
  a.n_init = n_init;
  a.n_local = n_local;
  a.sel = sel;
  a.sel_pages = sel_pages;
  a.counters = counters;
  const int waves = score_waves(sel != nullptr);
  a.score_wgs_x = (step->max_blocks_per_seq + waves - 1) / waves;
  const int64_t app_wgs = (static_cast<int64_t>(n_new) * a.app.groups_per_tok + 64 * waves - 1) / (64 * waves);
  a.append_row = n_new > 0 ? 1 : 0;
  dim3 grid(static_cast<unsigned>(std::max<int64_t>(a.score_wgs_x, app_wgs)), score_rows(a, step) + a.append_row);
  const size_t lds = sel ? static_cast<size_t>(step->max_blocks_per_seq) * sizeof(uint32_t) : 0;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  if (sel != nullptr) return launch_score<true, score_waves(true)>(a, pool, n_idx_heads, tables, grid, lds, hs);
  return launch_score<true, score_waves(false)>(a, pool, n_idx_heads, tables, grid, lds, hs);
}
