// Sparse GQA decode of groups of query rows over the union of their selections:
//   msa_sparse_decode_union
//
// On the pages: [Rubin] commit messages list query pairing among the tuned parameters
// of the NVFP4 sparse decode at a verify length of 4 query rows per request. Reading:
// the rows of one request that select the same block read that page once, and each
// row applies its own causal mask and keeps its own softmax state.
//
// MI355X design. One workgroup per (split, group, KV head), a group being 1..4 rows of
// one request. The workgroup first builds the union of the group's selection tables
// in LDS: a bitmap over the request's blocks, 4 bits per block (one per row), marks
// which rows picked each block; the first pick of a block (rows in order, each table in
// order) becomes a union entry (block, page, row mask). Split s of S takes the union
// entries [s N / S, (s + 1) N / S) of the N entries. As in the one-row decode, each
// wave takes one 32-token chunk per round and stages V in its LDS buffer; here it does
// so once for every row of the entry's mask, and then, for each of those rows that sees
// a token of the chunk, computes the row's scores (K dequantised from the same
// registers, Q read from LDS), its online softmax and its O update. The rounds are
// software-pipelined: the next round's chunk is loaded into a second register set while
// the current one is computed. Every wave holds the softmax state and O of all the
// group's rows (32 fp32 per row and lane), so the four-row variant runs two waves per
// SIMD. The waves' states are merged row by row through LDS. One split writes the bf16
// output itself; several write partials in msa_sparse_decode's layout, which
// msa_combine merges.
#include <algorithm>

#include "msa_device.h"
#include "msa_host.h"
#include "decode_device.h"

namespace msa {
namespace {

constexpr int kUnionWaves = 8;
constexpr int kMaxGroupRows = MSA_MAX_GROUP_ROWS;
static_assert(kMaxGroupRows <= 4, "the union bitmap holds 4 row bits per block");

struct UnionArgs {
  KvArrays kv;
  float k_t, v_t;
  int hkv;
  const int32_t* block_table;
  const int32_t* row_seq;
  const int32_t* row_pos;
  int max_blocks;
  int num_rows, num_seqs, num_pages;
  const uint16_t* q;
  int sel_tables;
  const int32_t* sel;
  const int32_t* sel_pages;   // may be null: translate through the block table
  const int32_t* group_rows;  // [groups + 1] row offsets
  int max_group_rows;
  int k;
  float softmax_scale;
  int num_splits;
  float* part_o;              // several splits: partials [rows][hq][S][128]
  float* part_ml;
  uint16_t* out;              // one split: bf16 [rows][hq][128]
  int32_t* err;
};

// kR: the rows of a group the kernel is compiled for (1, 2 or 4). kPipe: the next
// round's chunk is loaded while the wave computes the current one (a second set of
// chunk registers; off where those registers would not fit beside four rows' state).
template <int kFmt, int kR, bool kDirect>
constexpr bool union_pipelined() { return !(kFmt == MSA_KV_FP8_E4M3 && kR == 4); }

template <int kFmt, int kR, bool kDirect>
__global__ void __launch_bounds__(64 * kUnionWaves) union_decode_kernel(UnionArgs a) {
  constexpr int kW = kUnionWaves;
  constexpr bool kPipe = union_pipelined<kFmt, kR, kDirect>();
  // Dynamic LDS: the union bitmap while the union is built, then the per-wave V staging
  // buffers and, at the end, the per-wave O tiles of one row at a time.
  extern __shared__ __attribute__((aligned(16))) uint8_t dyn_lds[];
  __shared__ int32_t ublk[kR * MSA_MAX_TOPK], upage[kR * MSA_MAX_TOPK], umask[kR * MSA_MAX_TOPK];
  __shared__ int32_t s_pos[kR];
  __shared__ int32_t s_cnt[kW];
  __shared__ half8_t qlds[kR][4][64];
  __shared__ float qcs[kR][64];
  __shared__ float mbuf[kW][16], lbuf[kW][16];

  const int grp = blockIdx.y / a.hkv, g = blockIdx.y % a.hkv, s = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63, n = lane & 15, q = lane >> 4;
  const int hq = a.hkv * kHeadsPerKv;

  // ---- the group's rows [r0, r0 + nr), kept inside [0, num_rows) and kR rows
  int r0 = a.group_rows[grp], r1 = a.group_rows[grp + 1];
  const bool group_ok = r0 >= 0 && r0 <= r1 && r1 <= a.num_rows && r1 - r0 <= a.max_group_rows;
  if (threadIdx.x == 0) dcheck(group_ok, MSA_DEBUG_BAD_GROUP, a.err);
  r0 = min(max(r0, 0), a.num_rows);
  const int nr = __builtin_amdgcn_readfirstlane(min(max(r1 - r0, 0), min(kR, a.num_rows - r0)));
  if (nr == 0) return;
  r0 = __builtin_amdgcn_readfirstlane(r0);

  // ---- Q of row rho, converted by wave kW - 1 - rho (its load goes out first)
  const int qrow = kW - 1 - wave;
  uint4 qraw[4];
  if (qrow < nr)
    load_q_raw(qraw, a.q + (static_cast<int64_t>(r0 + qrow) * hq + kHeadsPerKv * g + n) * kHeadDim + 32 * q);

  // ---- picks: thread t < nr * k holds entry t % k of row t / k
  const int t = threadIdx.x;
  const int rho = t / a.k, e = t - rho * a.k;
  int b = -1, page = -1;
  const int seq0 = checked_seq(a.row_seq[r0], a.num_seqs, a.err);
  if (rho < nr) {
    const int r = r0 + rho;
    const int64_t trow = static_cast<int64_t>(r) * a.sel_tables + (a.sel_tables > 1 ? g : 0);
    b = a.sel[trow * a.k + e];
    const int pos = a.row_pos[r];
    // an entry that is neither -1 nor a visible block of its row is dropped (the debug
    // library reports it); this also keeps the bitmap update below in bounds
    if (!dcheck(b >= -1 && b < min(pos / kPage + 1, a.max_blocks), MSA_DEBUG_BAD_SEL, a.err)) b = -1;
    if (b >= 0)
      page = a.sel_pages ? a.sel_pages[trow * a.k + e] : a.block_table[static_cast<int64_t>(seq0) * a.max_blocks + b];
    // (a negative page, e.g. a -1 table entry reached through a group that mixes
    // requests, is dropped rather than read before the pool)
    if (page < 0) b = -1;
    if (e == 0) {
      s_pos[rho] = pos;
      dcheck(a.row_seq[r] == a.row_seq[r0], MSA_DEBUG_BAD_GROUP, a.err);
      if (s == 0) check_pos(pos, a.max_blocks, a.err);
    }
  }
  uint32_t* bits = reinterpret_cast<uint32_t*>(dyn_lds);
  const int nwords = (a.max_blocks + 7) >> 3;
  for (int i = t; i < nwords; i += 64 * kW) bits[i] = 0u;
  __syncthreads();
  uint32_t old = 0u;
  const int sh = 4 * (b & 7) + rho;
  if (b >= 0) old = atomicOr(bits + (b >> 3), 1u << sh);
  // Q conversion runs while the bitmap settles
  half8_t Qop[4];
  float cscale;
  if (qrow < nr) {
    convert_q_op(qraw, Qop, cscale, a.softmax_scale * kLog2e, kFmt == MSA_KV_NVFP4 ? a.k_t : 1.0f);
#pragma unroll
    for (int j = 0; j < 4; ++j) qlds[qrow][j][lane] = Qop[j];
    qcs[qrow][lane] = cscale;
  }
  __syncthreads();
  // A pick is a union entry if no earlier row picked its block and it is the row's only
  // pick of it (of two equal picks in one row, the one whose update came first).
  bool owner = false;
  int mask = 0;
  if (b >= 0) {
    mask = static_cast<int>((bits[b >> 3] >> (4 * (b & 7))) & 0xfu);
    const bool dup = (old >> sh) & 1u;
    dcheck(!dup, MSA_DEBUG_BAD_SEL, a.err);
    owner = !dup && (mask & ((1 << rho) - 1)) == 0;
  }
  // compaction in pick order: rows in order, each table in order
  const uint64_t bal = __ballot(owner);
  if (lane == 0) s_cnt[wave] = __popcll(bal);
  __syncthreads();
  int base = 0, total = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const int c = s_cnt[w];
    base += w < wave ? c : 0;
    total += c;
  }
  if (owner) {
    const int at = base + __popcll(bal & ((1ull << lane) - 1ull));
    ublk[at] = b;
    upage[at] = page;
    umask[at] = mask;
  }
  __syncthreads();

  int pos_r[kR];
#pragma unroll
  for (int i = 0; i < kR; ++i) pos_r[i] = __builtin_amdgcn_readfirstlane(s_pos[i < nr ? i : 0]);
  const int N = __builtin_amdgcn_readfirstlane(total);
  const int lo = (s * N) / a.num_splits, hi = ((s + 1) * N) / a.num_splits;
  const int n_items = (hi - lo) * 4;

  float m_run[kR], l_run[kR], v_cur[kR];
  float4_t O[kR][8];
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    m_run[i] = -INFINITY;
    l_run[i] = 0.0f;
    v_cur[i] = 0.0f;
#pragma unroll
    for (int d = 0; d < 8; ++d) O[i][d] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  }
  half_t* vb = reinterpret_cast<half_t*>(dyn_lds + wave * kVBufBytes);
  typedef __attribute__((address_space(3))) short4_t lds_s4;
  const KvArrays kv = a.kv;

  // One chunk of a round as a wave holds it: its registers and per-row visible tokens.
  struct Item {
    ChunkRegs<kFmt> R;
    int nvis[kR];
    bool valid;
    float kps, vps;
  };
  // Issue every load of this wave's chunk of the round at `round`: union entry
  // lo + it / 4, 32-token chunk it % 4 (past the split: zero-byte loads, not valid).
  auto issue = [&](Item& X, int round) {
    const int it = round + wave;
    const int ue = lo + min(it, n_items - 1) / 4, c = it & 3;
    const int blk = __builtin_amdgcn_readfirstlane(ublk[ue]);
    const int msk = __builtin_amdgcn_readfirstlane(umask[ue]);
    int nv_any = 0;
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      const int nv = min(pos_r[i] - blk * kPage + 1, kPage) - 32 * c;
      X.nvis[i] = (it < n_items && i < nr && ((msk >> i) & 1)) ? min(max(nv, 0), 32) : 0;
      nv_any = max(nv_any, X.nvis[i]);
    }
    X.valid = nv_any > 0;
    int64_t pg = X.valid ? checked_page(upage[ue], a.num_pages, a.err) : 0;
    pg = static_cast<int64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(pg))));
    load_chunk<kFmt>(X.R, kv, pg * a.hkv + g, X.valid, c, n, q);
    X.kps = X.vps = 1.0f;
    if constexpr (kFmt == MSA_KV_FP8_E4M3) {
      X.kps = reinterpret_cast<const float*>(a.kv.k_scales)[pg];
      X.vps = reinterpret_cast<const float*>(a.kv.v_scales)[pg];
    }
  };
  auto compute = [&](Item& X) {
    if (!X.valid) return;
    const float kps = X.kps, vps = X.vps;
    const uint32_t* ksc = nullptr;
    const uint32_t* vsc = nullptr;
    if constexpr (kFmt == MSA_KV_NVFP4) { ksc = X.R.ks; vsc = X.R.vs; }
    // ---- V chunk to LDS once for every row (natural [token][d] layout, fp16)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        *reinterpret_cast<half8_t*>(vb + (16 * u + n) * kVRowHalves + 32 * q + 8 * kk) = dequant8<kFmt>(X.R.v, vsc, u, kk);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < kR; ++i) {
      if (X.nvis[i] <= 0) continue;
      half8_t Qi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) Qi[j] = qlds[i][j][lane];
      const float cs = qcs[i][lane] * kps;
      float ratio = 1.0f;
      if constexpr (kFmt == MSA_KV_FP8_E4M3) {
        ratio = v_cur[i] > 0.0f ? v_cur[i] / vps : 1.0f;   // keep the row's O in units of this page's scale
        v_cur[i] = vps;
      }
      float4_t acc[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        acc[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) acc[u] = mfma16x16x32(dequant8<kFmt>(X.R.k, ksc, u, kk), Qi[kk], acc[u]);
      }
      float x[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[u][j] = (16 * u + 4 * q + j) < X.nvis[i] ? acc[u][j] * cs : -INFINITY;
      float mx = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                       fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
      mx = rows_max(mx);
      const float m_new = fmaxf(m_run[i], mx);
      const float alpha = exp2_raw(m_run[i] - m_new);
      float psum = 0.0f;
      half8_t Pt;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p = exp2_raw(x[u][j] - m_new);
          psum += p;
          Pt[4 * u + j] = static_cast<half_t>(p);
        }
      if (m_run[i] != -INFINITY) {
        const float ao = alpha * ratio;
#pragma unroll
        for (int d = 0; d < 8; ++d) O[i][d] *= ao;
      }
      l_run[i] = l_run[i] * alpha + psum;
      m_run[i] = m_new;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const half_t* p0 = vb + (4 * q + (n >> 2)) * kVRowHalves + 16 * d + 4 * (n & 3);
        const half_t* p1 = p0 + 16 * kVRowHalves;
        const half4_t h0 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p0)));
        const half4_t h1 = __builtin_bit_cast(half4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p1)));
        const half8_t Vt = {h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
        O[i][d] = mfma16x16x32(Vt, Pt, O[i][d]);
      }
    }
    asm volatile("" ::: "memory");   // (the next chunk's V writes stay behind these reads)
  };

  if constexpr (kPipe) {
    // Two register sets: a round's loads are in flight while the wave computes the
    // round before (every chunk issues the same loads, so the wait before each compute
    // leaves exactly the later round's loads outstanding).
    Item A, B;
    issue(A, 0);
    for (int round = 0; round < n_items; round += 2 * kW) {
      issue(B, round + kW);
      compute(A);
      issue(A, round + 2 * kW);
      compute(B);
    }
  } else {
    Item A;
    for (int round = 0; round < n_items; round += kW) {
      issue(A, round);
      compute(A);
    }
  }

  // ---- per row: merge the waves' states through LDS, write the output or the partial
  constexpr int kTasks = 16 * (kHeadDim / 4);
  static_assert(kTasks == 64 * kW, "one (head, 4 dims) item per thread");
  const int h = threadIdx.x / (kHeadDim / 4), d4 = threadIdx.x % (kHeadDim / 4);
  float* ob = reinterpret_cast<float*>(dyn_lds + wave * kVBufBytes);   // [16 heads][kORowFloats]
#pragma unroll
  for (int i = 0; i < kR; ++i) {
    if (i >= nr) break;
    const float l_tot = rows_sum(l_run[i]);
    float oscale;
    if constexpr (kFmt == MSA_KV_NVFP4) oscale = a.v_t; else oscale = v_cur[i];
    __syncthreads();   // (every wave is done with the LDS it overwrites)
#pragma unroll
    for (int d = 0; d < 8; ++d)
      *reinterpret_cast<float4_t*>(ob + n * kORowFloats + 16 * d + 4 * q) = O[i][d] * oscale;
    if (q == 0) { mbuf[wave][n] = m_run[i]; lbuf[wave][n] = l_tot; }
    __syncthreads();
    float mw[kW], lw[kW];
    float4_t tw[kW];
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      mw[w] = mbuf[w][h];
      lw[w] = lbuf[w][h];
      tw[w] = *reinterpret_cast<const float4_t*>(reinterpret_cast<const float*>(dyn_lds + w * kVBufBytes) +
                                                 h * kORowFloats + 4 * d4);
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, mw[w]);
    float4_t acc = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        const float wt = exp2_raw(mw[w] - M);
        acc += wt * tw[w];
        l += wt * lw[w];
      }
    }
    const int64_t head = static_cast<int64_t>(r0 + i) * hq + kHeadsPerKv * g + h;
    if constexpr (kDirect) {
      uint16_t o[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = l > 0.0f ? f32_to_bf16_rne(acc[j] / l) : 0;
      *reinterpret_cast<uint2*>(a.out + head * kHeadDim + 4 * d4) =
          make_uint2(o[0] | (static_cast<uint32_t>(o[1]) << 16), o[2] | (static_cast<uint32_t>(o[3]) << 16));
    } else {
      *reinterpret_cast<float4_t*>(a.part_o + (head * a.num_splits + s) * kHeadDim + 4 * d4) = acc;
      if (d4 == 0) {
        float* pm = a.part_ml + (head * a.num_splits + s) * 2;
        pm[0] = M;
        pm[1] = l;
      }
    }
  }
}

template <int kFmt, int kR, bool kDirect>
void launch(const UnionArgs& a, dim3 grid, hipStream_t st) {
  const size_t lds = std::max(static_cast<size_t>(kUnionWaves) * kVBufBytes,
                              static_cast<size_t>((a.max_blocks + 7) >> 3) * sizeof(uint32_t));
  union_decode_kernel<kFmt, kR, kDirect><<<grid, dim3(64 * kUnionWaves), lds, st>>>(a);
}

template <int kFmt, bool kDirect>
void dispatch_rows(const UnionArgs& a, dim3 grid, hipStream_t st) {
  if (a.max_group_rows <= 1) launch<kFmt, 1, kDirect>(a, grid, st);
  else if (a.max_group_rows <= 2) launch<kFmt, 2, kDirect>(a, grid, st);
  else launch<kFmt, 4, kDirect>(a, grid, st);
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_sparse_decode_union(const msa_kv_pool_t* pool, const msa_step_t* step,
                                                int32_t num_q_heads, const void* q, const int32_t* sel,
                                                const int32_t* sel_pages, int32_t k, int32_t num_groups,
                                                const int32_t* group_rows, int32_t max_group_rows,
                                                float softmax_scale, int32_t num_splits, float* part_o,
                                                float* part_ml, void* out, void* stream) {
  using namespace msa;
  msa_status_t st = check_pool(pool);
  if (st != MSA_OK) return st;
  if ((st = check_step(step)) != MSA_OK) return st;
  if (num_q_heads != MSA_HEADS_PER_KV * pool->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  // (as many splits as msa_combine merges)
  if (k < 1 || k > MSA_MAX_TOPK || num_splits < 1 || num_splits > MSA_MAX_TOPK) return MSA_ERR_UNSUPPORTED;
  if (max_group_rows < 1 || max_group_rows > kMaxGroupRows) return MSA_ERR_UNSUPPORTED;
  if (num_groups < 0) return MSA_ERR_INVALID_ARG;
  if (!(softmax_scale > 0.0f)) return MSA_ERR_INVALID_ARG;
  const int tables = sel_tables(step);
  if (tables != 1 && tables != pool->num_kv_heads) return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0 || num_groups == 0) return MSA_OK;
  if (q == nullptr || sel == nullptr || group_rows == nullptr || !aligned16(q)) return MSA_ERR_INVALID_ARG;
  if (num_splits == 1 ? (out == nullptr || (reinterpret_cast<uintptr_t>(out) & 7u))
                      : (part_o == nullptr || part_ml == nullptr || !aligned16(part_o) ||
                         (reinterpret_cast<uintptr_t>(part_ml) & 7u)))
    return MSA_ERR_INVALID_ARG;
  if (static_cast<int64_t>(num_groups) * pool->num_kv_heads > 65535) return MSA_ERR_UNSUPPORTED;
  UnionArgs a{};
  a.kv = KvArrays{static_cast<const uint8_t*>(pool->k_codes), static_cast<const uint8_t*>(pool->v_codes),
                  static_cast<const uint8_t*>(pool->k_scales), static_cast<const uint8_t*>(pool->v_scales)};
  a.k_t = pool->k_tensor_scale;
  a.v_t = pool->v_tensor_scale;
  a.hkv = pool->num_kv_heads;
  a.block_table = step->block_table;
  a.row_seq = step->row_seq;
  a.row_pos = step->row_pos;
  a.max_blocks = step->max_blocks_per_seq;
  a.num_rows = step->num_rows;
  a.num_seqs = step->num_seqs;
  a.num_pages = pool->num_pages;
  a.q = static_cast<const uint16_t*>(q);
  a.sel_tables = tables;
  a.sel = sel;
  a.sel_pages = sel_pages;
  a.group_rows = group_rows;
  a.max_group_rows = max_group_rows;
  a.k = k;
  a.softmax_scale = softmax_scale;
  a.num_splits = num_splits;
  a.part_o = part_o;
  a.part_ml = part_ml;
  a.out = static_cast<uint16_t*>(out);
  a.err = debug_error_word();
  const dim3 grid(num_splits, num_groups * pool->num_kv_heads);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool direct = num_splits == 1;
  if (pool->fmt == MSA_KV_NVFP4) {
    if (direct) dispatch_rows<MSA_KV_NVFP4, true>(a, grid, s); else dispatch_rows<MSA_KV_NVFP4, false>(a, grid, s);
  } else {
    if (direct) dispatch_rows<MSA_KV_FP8_E4M3, true>(a, grid, s); else dispatch_rows<MSA_KV_FP8_E4M3, false>(a, grid, s);
  }
  return launch_status();
}
