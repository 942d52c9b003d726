// msa_select_topk: deterministic top-k block selection per query row.
//
// Contract ([Rubin] commit messages; [GB300] "The TP4 decode target", numerics):
// forced init/local blocks, the best other blocks by (score desc, index asc), output
// ascending and -1 padded. Ties are resolved by block index at any tie width, never
// by arrival order. Rows of up to 2048 candidates: one wave per row runs the ballot
// threshold search of the fused decode. Longer rows: the k'-th largest score is found
// with an MSB-first radix select (LDS histograms, whose counts do not depend on atomic
// order), then blocks tied at that score are ranked by an exclusive scan in block order.
// With T selection tables per row (one per KV head) each (row, table) pair is selected
// on its own, as table row r * T + t of the scores and of the outputs.
#include "msa_device.h"
#include "msa_host.h"
#include "select_device.h"

namespace msa {
namespace {

__global__ void __launch_bounds__(kSelectThreads)
select_topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ row_pos,
                   const int32_t* __restrict__ row_seq, const int32_t* __restrict__ block_table,
                   int32_t* __restrict__ sel, int32_t* __restrict__ sel_pages, int max_blocks, int k,
                   int n_init, int n_local, int tables, int num_seqs, int32_t* err) {
  extern __shared__ uint32_t keys[];            // [candidates]
  __shared__ SelectSmem sm;
  const int64_t tr = blockIdx.x;                // table row
  const int r = static_cast<int>(tr / tables);
  if (threadIdx.x == 0) check_pos(row_pos[r], max_blocks, err);
  const int nb = min(row_pos[r] / kPage + 1, max_blocks);   // the table covers nb blocks
  block_select_row<false>(scores + tr * max_blocks, nb, k, n_init, n_local,
                          block_table + static_cast<int64_t>(checked_seq(row_seq[r], num_seqs, err)) * max_blocks,
                          sel + tr * k, sel_pages ? sel_pages + tr * k : nullptr, keys, sm);
}

// Rows with at most kWaveSelectMax candidates: one wave per row, the wave-level search
// of the fused decode (same contract, same table). Its block-table reads go out with the
// score reads, from the row of the request the row would belong to if every request
// had the same number of rows; the pages are read again if row_seq says otherwise.
constexpr int kRowsPerSelectWg = 4;
__global__ void __launch_bounds__(64 * kRowsPerSelectWg)
select_topk_wave_kernel(const float* __restrict__ scores, const int32_t* __restrict__ row_pos,
                        const int32_t* __restrict__ row_seq, const int32_t* __restrict__ block_table,
                        int32_t* __restrict__ sel, int32_t* __restrict__ sel_pages, int num_rows,
                        int max_blocks, int k, int n_init, int n_local, uint64_t seq_mul, int tables,
                        int num_seqs, int32_t* err) {
  __shared__ int32_t lsel[kRowsPerSelectWg][MSA_MAX_TOPK], lpage[kRowsPerSelectWg][MSA_MAX_TOPK];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int tr = blockIdx.x * kRowsPerSelectWg + wave;      // table row
  if (tr >= num_rows * tables) return;
  const int r = tr / tables;
  const int guess = seq_guess(r, seq_mul);
  const int seq = checked_seq(row_seq[r], num_seqs, err);
  if (lane == 0) check_pos(row_pos[r], max_blocks, err);
  wave_select(scores + static_cast<int64_t>(tr) * max_blocks, block_table + static_cast<int64_t>(guess) * max_blocks,
              max_blocks, row_pos + r, k, n_init, n_local, lsel[wave], lpage[wave]);
  const int b = lsel[wave][lane];
  int page = lpage[wave][lane];
  if (seq != guess) page = b >= 0 ? block_table[static_cast<int64_t>(seq) * max_blocks + b] : -1;
  if (lane < k) {
    sel[static_cast<int64_t>(tr) * k + lane] = b;
    if (sel_pages) sel_pages[static_cast<int64_t>(tr) * k + lane] = page;
  }
}

}  // namespace
}  // namespace msa

extern "C" msa_status_t msa_select_topk(const msa_step_t* step, const float* block_scores,
                                        int32_t k, int32_t n_init, int32_t n_local, int32_t* sel,
                                        int32_t* sel_pages, void* stream) {
  using namespace msa;
  msa_status_t st = check_step(step);
  if (st != MSA_OK) return st;
  if (k < 1 || k > MSA_MAX_TOPK || n_init < 0 || n_local < 0 || n_init + n_local > k)
    return MSA_ERR_UNSUPPORTED;
  if (step->num_rows == 0) return MSA_OK;
  if (block_scores == nullptr || sel == nullptr) return MSA_ERR_INVALID_ARG;
  const int tables = sel_tables(step);
  const int64_t table_rows = static_cast<int64_t>(step->num_rows) * tables;
  if (table_rows > 0x7fffffff) return MSA_ERR_UNSUPPORTED;
  // (the request guess is exact, and so in range, for up to 65535 rows)
  if (step->max_blocks_per_seq - n_init - n_local <= kWaveSelectMax && step->num_rows <= 65535) {
    const unsigned wgs = static_cast<unsigned>((table_rows + kRowsPerSelectWg - 1) / kRowsPerSelectWg);
    select_topk_wave_kernel<<<dim3(wgs), dim3(64 * kRowsPerSelectWg), 0, static_cast<hipStream_t>(stream)>>>(
        block_scores, step->row_pos, step->row_seq, step->block_table, sel, sel_pages, step->num_rows,
        step->max_blocks_per_seq, k, n_init, n_local, seq_guess_mul(step->num_seqs, step->num_rows), tables,
        step->num_seqs, debug_error_word());
    return launch_status();
  }
  const size_t lds = static_cast<size_t>(step->max_blocks_per_seq) * sizeof(uint32_t);
  select_topk_kernel<<<dim3(static_cast<unsigned>(table_rows)), dim3(kSelectThreads), lds,
                       static_cast<hipStream_t>(stream)>>>(
      block_scores, step->row_pos, step->row_seq, step->block_table, sel, sel_pages,
      step->max_blocks_per_seq, k, n_init, n_local, tables, step->num_seqs, debug_error_word());
  return launch_status();
}
