"""libmsadecode: block-sparse FP8/NVFP4 attention decode for AMD MI355X (gfx950).

The decode path lives in hand-written HIP kernels behind the C ABI declared in
include/msa_decode.h; this package is the ctypes binding (marshalling only) plus
the in-tree build script. Importing it loads the HIP library and fails loudly if
it has not been built.
"""
from ._lib import (FMT_FP8, FMT_NVFP4, IDX_E4M3, IDX_NVFP4, KVPool, MsaError, Step, msa_combine,  # noqa: F401
                   msa_decode_workspace_bytes, msa_index_score, msa_kv_append, msa_select_topk,
                   msa_sparse_decode, msa_sparse_decode_combine, msa_sparse_decode_union, group_rows_of,
                   msa_sparse_decode_combine_noalloc,
                   msa_append_score_select, msa_select_decode_combine, msa_merge_workspace_init,
                   msa_decode_step, msa_step_workspace_init,
                   MERGE_IDLE_BITS, msa_debug_set_error_word, msa_debug_set_merge_poll_limit,
                   msa_debug_set_merge_helper_poll_limit,
                   load_library, use_library,
                   RELEASE_LIB_PATH, DEBUG_LIB_PATH)
from .pipeline import DecodeBuffers, default_num_splits, run_step  # noqa: F401
