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
#include "select_device.h"

namespace msa {
namespace {

__global__ void __launch_bounds__(kSelectThreads)
select_topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ row_pos,
                   const int32_t* __restrict__ row_seq, const int32_t* __restrict__ block_table,
                   int32_t* __restrict__ sel, int32_t* __restrict__ sel_pages, int max_blocks, int k,
                   int n_init, int n_local) {
  extern __shared__ uint32_t keys[];            // [candidates]
  __shared__ SelectSmem sm;
  const int r = blockIdx.x;
  const int nb = min(row_pos[r] / kPage + 1, max_blocks);   // the table covers nb blocks
  block_select_row<false>(scores + static_cast<int64_t>(r) * max_blocks, nb, k, n_init, n_local,
                          block_table + static_cast<int64_t>(row_seq[r]) * max_blocks,
                          sel + static_cast<int64_t>(r) * k,
                          sel_pages ? sel_pages + static_cast<int64_t>(r) * k : nullptr, keys, sm);
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
  const size_t lds = static_cast<size_t>(step->max_blocks_per_seq) * sizeof(uint32_t);
  select_topk_kernel<<<dim3(step->num_rows), dim3(kSelectThreads), lds, static_cast<hipStream_t>(stream)>>>(
      block_scores, step->row_pos, step->row_seq, step->block_table, sel, sel_pages,
      step->max_blocks_per_seq, k, n_init, n_local);
  return launch_status();
}
