// Host-side argument validation shared by the libmsadecode entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msa_decode.h"

namespace msa {

// The debug library's error word (null in the release library, or when unset).
int32_t* debug_error_word();
// Bound on the last split's merge poll rounds: kMergePollLimit, or the debug library's
// setting.
constexpr int32_t kMergePollLimit = 1 << 16;
int32_t merge_poll_limit();
// Bound on the poll rounds of a merging split that is not the last to arrive, before it
// hands its slice to the last one: kMergeHelperPolls, or the debug library's setting.
// (A poll round is one agent-coherent load round trip, about a microsecond.)
constexpr int32_t kMergeHelperPolls = 32;
int32_t merge_helper_poll_limit();

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

inline msa_status_t check_pool(const msa_kv_pool_t* pool) {
  if (pool == nullptr) return MSA_ERR_INVALID_ARG;
  if (pool->fmt != MSA_KV_FP8_E4M3 && pool->fmt != MSA_KV_NVFP4) return MSA_ERR_UNSUPPORTED;
  if (pool->head_dim != MSA_HEAD_DIM || pool->page_size != MSA_PAGE_SIZE ||
      pool->index_dim != MSA_INDEX_DIM)
    return MSA_ERR_UNSUPPORTED;
  if (pool->num_pages <= 0 || pool->num_kv_heads <= 0) return MSA_ERR_INVALID_ARG;
  if (pool->num_kv_heads > 64) return MSA_ERR_UNSUPPORTED;
  const void* arr[5] = {pool->k_codes, pool->v_codes, pool->k_scales, pool->v_scales,
                        pool->index_k};
  for (const void* p : arr)
    if (p == nullptr || !aligned16(p)) return MSA_ERR_INVALID_ARG;
  if (pool->fmt == MSA_KV_NVFP4 && !(pool->k_tensor_scale > 0.0f && pool->v_tensor_scale > 0.0f))
    return MSA_ERR_INVALID_ARG;
  if (pool->index_fmt == MSA_INDEX_NVFP4) {
    if (pool->index_scales == nullptr || !aligned16(pool->index_scales) || !(pool->index_tensor_scale > 0.0f))
      return MSA_ERR_INVALID_ARG;
  } else if (pool->index_fmt != 0 && pool->index_fmt != MSA_INDEX_E4M3) {
    return MSA_ERR_UNSUPPORTED;
  }
  return MSA_OK;
}

inline bool index_nvfp4(const msa_kv_pool_t* pool) { return pool->index_fmt == MSA_INDEX_NVFP4; }

inline msa_status_t check_step(const msa_step_t* step) {
  if (step == nullptr) return MSA_ERR_INVALID_ARG;
  if (step->num_seqs < 0 || step->num_rows < 0 || step->max_blocks_per_seq <= 0)
    return MSA_ERR_INVALID_ARG;
  if (step->max_blocks_per_seq > MSA_MAX_BLOCKS) return MSA_ERR_UNSUPPORTED;
  if (step->sel_tables < 0) return MSA_ERR_INVALID_ARG;
  if (step->sel_tables > MSA_MAX_SEL_TABLES) return MSA_ERR_UNSUPPORTED;
  if (step->num_rows > 0 && (step->num_seqs == 0 || step->block_table == nullptr ||
                             step->row_seq == nullptr || step->row_pos == nullptr))
    return MSA_ERR_INVALID_ARG;
  if (step->rows_per_seq < 0 ||
      (step->rows_per_seq > 0 &&
       static_cast<int64_t>(step->num_seqs) * step->rows_per_seq != static_cast<int64_t>(step->num_rows)))
    return MSA_ERR_INVALID_ARG;
  return MSA_OK;
}

// Selection tables per query row: 1 (0 in the struct) or one per KV head.
inline int sel_tables(const msa_step_t* step) { return step->sel_tables > 1 ? step->sel_tables : 1; }

// Multiplier for the device-side guess of a row's request, r * num_seqs / num_rows,
// as (r * mul) >> 32 with mul = ceil(2^32 * num_seqs / num_rows). For r < num_rows <=
// 65535 this equals the exact floor quotient (the excess r * (ceil - exact) / 2^32 stays
// below 1 / num_rows, the smallest nonzero distance to the next integer).
inline uint64_t seq_guess_mul(int32_t num_seqs, int32_t num_rows) {
  if (num_rows <= 0) return 0;
  const uint64_t n = static_cast<uint64_t>(num_seqs) << 32;
  return n / static_cast<uint64_t>(num_rows) + (n % static_cast<uint64_t>(num_rows) != 0);
}

inline msa_status_t launch_status() {
  return hipGetLastError() == hipSuccess ? MSA_OK : MSA_ERR_LAUNCH;
}

}  // namespace msa
