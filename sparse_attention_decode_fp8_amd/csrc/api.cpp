// Host-only entry points of libmsadecode: sizes and status strings.
#include <stddef.h>
#include <stdint.h>

#include "msa_decode.h"
#include "msa_host.h"

extern "C" size_t msa_decode_workspace_bytes(int32_t rows, int32_t num_q_heads, int32_t head_dim,
                                             int32_t num_splits) {
  if (rows < 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  const size_t n = static_cast<size_t>(rows) * num_q_heads * num_splits;
  size_t o = n * head_dim * sizeof(float);
  o = (o + 255) / 256 * 256;
  return o + n * 2 * sizeof(float);
}

extern "C" msa_status_t msa_pool_bytes(int32_t fmt, int32_t num_pages, int32_t num_kv_heads,
                                       int32_t head_dim, int32_t index_dim, size_t out[5]) {
  if (out == nullptr || num_pages <= 0 || num_kv_heads <= 0) return MSA_ERR_INVALID_ARG;
  if (head_dim != MSA_HEAD_DIM || index_dim != MSA_INDEX_DIM) return MSA_ERR_UNSUPPORTED;
  const size_t tok = static_cast<size_t>(num_pages) * num_kv_heads * MSA_PAGE_SIZE;
  if (fmt == MSA_KV_NVFP4) {
    out[0] = out[1] = tok * (head_dim / 2);
    out[2] = out[3] = tok * (head_dim / 16);
  } else if (fmt == MSA_KV_FP8_E4M3) {
    out[0] = out[1] = tok * head_dim;
    out[2] = out[3] = static_cast<size_t>(num_pages) * sizeof(float);
  } else {
    return MSA_ERR_UNSUPPORTED;
  }
  out[4] = static_cast<size_t>(num_pages) * MSA_PAGE_SIZE * index_dim;
  return MSA_OK;
}

extern "C" msa_status_t msa_index_bytes(int32_t index_fmt, int32_t num_pages, int32_t index_dim,
                                        size_t out[2]) {
  if (out == nullptr || num_pages <= 0) return MSA_ERR_INVALID_ARG;
  if (index_dim != MSA_INDEX_DIM) return MSA_ERR_UNSUPPORTED;
  const size_t tok = static_cast<size_t>(num_pages) * MSA_PAGE_SIZE;
  if (index_fmt == 0 || index_fmt == MSA_INDEX_E4M3) {
    out[0] = tok * index_dim;
    out[1] = 0;
  } else if (index_fmt == MSA_INDEX_NVFP4) {
    out[0] = tok * (index_dim / 2);
    out[1] = tok * (index_dim / 16);
  } else {
    return MSA_ERR_UNSUPPORTED;
  }
  return MSA_OK;
}

namespace msa {
// The error word of the debug library's device-side checks (see msa_debug_set_error_word).
static int32_t* g_debug_error_word = nullptr;
int32_t* debug_error_word() { return g_debug_error_word; }
// The debug library's bound on a merging split's poll rounds (< 0: the release bound).
static int32_t g_merge_poll_limit = -1;
int32_t merge_poll_limit() { return g_merge_poll_limit < 0 ? kMergePollLimit : g_merge_poll_limit; }
static int32_t g_merge_helper_poll_limit = -1;
int32_t merge_helper_poll_limit() {
  return g_merge_helper_poll_limit < 0 ? kMergeHelperPolls : g_merge_helper_poll_limit;
}
}  // namespace msa

extern "C" msa_status_t msa_debug_set_error_word(int32_t* word) {
#ifdef MSA_DEBUG_CHECKS
  msa::g_debug_error_word = word;
  return MSA_OK;
#else
  (void)word;
  return MSA_ERR_UNSUPPORTED;
#endif
}

extern "C" msa_status_t msa_debug_set_merge_poll_limit(int32_t polls) {
#ifdef MSA_DEBUG_CHECKS
  msa::g_merge_poll_limit = polls;
  return MSA_OK;
#else
  (void)polls;
  return MSA_ERR_UNSUPPORTED;
#endif
}

extern "C" msa_status_t msa_debug_set_merge_helper_poll_limit(int32_t polls) {
#ifdef MSA_DEBUG_CHECKS
  msa::g_merge_helper_poll_limit = polls;
  return MSA_OK;
#else
  (void)polls;
  return MSA_ERR_UNSUPPORTED;
#endif
}

extern "C" int32_t msa_debug_checks_enabled(void) {
#ifdef MSA_DEBUG_CHECKS
  return 1;
#else
  return 0;
#endif
}

extern "C" const char* msa_status_string(msa_status_t status) {
  switch (status) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_INVALID_ARG: return "MSA_ERR_INVALID_ARG: null, misaligned or negative argument";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: geometry or format outside the contract";
    case MSA_ERR_LAUNCH: return "MSA_ERR_LAUNCH: kernel launch failed";
    case MSA_ERR_TOO_LARGE: return "MSA_ERR_TOO_LARGE: the call needs more than the allocation-free entry's fixed scratch";
  }
  return "MSA_ERR_UNKNOWN";
}
