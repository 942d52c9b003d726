"""ctypes binding of libmsadecode (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch tensors
that already live on the GPU; it passes their device pointers and the current HIP
stream to the library and raises MsaError on a non-OK status. No computation of
the decode path happens in Python, and there is no fallback: if the HIP library is
not built, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
RELEASE_LIB_PATH = os.path.join(_HERE, "libmsadecode.so")
# The same library with device-side metadata checks (msa_debug_set_error_word);
# MSA_DEBUG_CHECKS=1 in the environment selects it at import.
DEBUG_LIB_PATH = os.path.join(_HERE, "libmsadecode_debug.so")
LIB_PATH = DEBUG_LIB_PATH if os.environ.get("MSA_DEBUG_CHECKS", "0") not in ("", "0") else RELEASE_LIB_PATH

FMT_FP8 = 1
FMT_NVFP4 = 2
IDX_E4M3 = 1
IDX_NVFP4 = 2
PAGE = 128
HEAD_DIM = 128
INDEX_DIM = 64

MSA_OK = 0
MSA_ERR_UNSUPPORTED = -2
MERGE_IDLE_BITS = 0x7fbadbad   # every fp32 word of an idle merge workspace


class MsaError(RuntimeError):
    pass


class MsaKvPool(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("index_dim", ctypes.c_int32),
                ("k_codes", ctypes.c_void_p), ("v_codes", ctypes.c_void_p),
                ("k_scales", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("k_tensor_scale", ctypes.c_float), ("v_tensor_scale", ctypes.c_float),
                ("index_k", ctypes.c_void_p), ("index_fmt", ctypes.c_int32),
                ("index_scales", ctypes.c_void_p), ("index_tensor_scale", ctypes.c_float)]


class MsaStep(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("max_blocks_per_seq", ctypes.c_int32), ("block_table", ctypes.c_void_p),
                ("row_seq", ctypes.c_void_p), ("row_pos", ctypes.c_void_p),
                ("sel_tables", ctypes.c_int32), ("rows_per_seq", ctypes.c_int32)]


EXPORTS = ["msa_kv_append", "msa_index_score", "msa_select_topk", "msa_append_score_select",
           "msa_sparse_decode", "msa_sparse_decode_union", "msa_sparse_decode_combine_noalloc",
           "msa_sparse_decode_combine", "msa_select_decode_combine", "msa_decode_step", "msa_combine",
           "msa_merge_workspace_init", "msa_step_workspace_init",
           "msa_decode_workspace_bytes", "msa_pool_bytes", "msa_index_bytes", "msa_status_string",
           "msa_debug_set_error_word", "msa_debug_set_merge_poll_limit", "msa_debug_set_merge_helper_poll_limit",
           "msa_debug_checks_enabled"]


def load_library(path: str):
    """Load one build of the library (release or debug) with its C signatures set."""
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python sparse_attention_decode_fp8_amd/build.py`")
    lib = ctypes.CDLL(path)
    P, I32, F32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "msa_kv_append": (I32, [P, I32, P, P, P, P, P]),
        "msa_index_score": (I32, [P, P, I32, P, P, P, P]),
        "msa_select_topk": (I32, [P, P, I32, I32, I32, P, P, P]),
        "msa_append_score_select": (I32, [P, P, I32, P, P, P, P, I32, P, P, I32, I32, I32, P, P, P, P, P]),
        "msa_sparse_decode": (I32, [P, P, I32, P, P, P, I32, F32, I32, P, P, P]),
        "msa_sparse_decode_union": (I32, [P, P, I32, P, P, P, I32, I32, P, I32, F32, I32, P, P, P, P]),
        "msa_sparse_decode_combine": (I32, [P, P, I32, P, P, P, I32, F32, I32, P, P, P, P, P]),
        "msa_sparse_decode_combine_noalloc": (I32, [P, P, I32, P, P, P, I32, F32, I32, P, P]),
        "msa_select_decode_combine": (I32, [P, P, I32, P, P, I32, I32, I32, F32, I32, P, P, P, P, P, P, P]),
        "msa_decode_step": (I32, [P, P, I32, P, P, P, P, I32, P, P, I32, P, I32, I32, I32, F32, I32, P, P, P, P, P,
                                  P, P, P, P, P]),
        "msa_step_workspace_init": (I32, [I32, I32, P, P, P]),
        "msa_combine": (I32, [I32, I32, I32, I32, P, P, P, P]),
        "msa_merge_workspace_init": (I32, [I32, I32, I32, I32, P, P, P, P]),
        "msa_decode_workspace_bytes": (SZ, [I32, I32, I32, I32]),
        "msa_pool_bytes": (I32, [I32, I32, I32, I32, I32, ctypes.POINTER(SZ)]),
        "msa_index_bytes": (I32, [I32, I32, I32, ctypes.POINTER(SZ)]),
        "msa_status_string": (ctypes.c_char_p, [I32]),
        "msa_debug_set_error_word": (I32, [P]),
        "msa_debug_set_merge_poll_limit": (I32, [I32]),
        "msa_debug_set_merge_helper_poll_limit": (I32, [I32]),
        "msa_debug_checks_enabled": (I32, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    return lib


LIB = load_library(LIB_PATH)


class use_library:
    """Context manager: the wrappers of this module call `lib` (from load_library)
    inside the block, e.g. the debug build in a test next to the release one."""

    def __init__(self, lib):
        self.lib = lib

    def __enter__(self):
        global LIB
        self.prev, LIB = LIB, self.lib
        return self.lib

    def __exit__(self, *exc):
        global LIB
        LIB = self.prev
        return False


def msa_debug_set_error_word(word):
    """Debug library: device int32 word (a 1-element tensor, or None) that failed
    metadata checks report to. The release library raises MsaError."""
    _check(LIB.msa_debug_set_error_word(_ptr(word, torch.int32, "word")), "msa_debug_set_error_word")


def msa_debug_set_merge_poll_limit(polls: int):
    """Debug library: poll rounds after which a merging split gives up (< 0: the release
    bound; 0: at once, to force the failure path). The release library raises MsaError."""
    _check(LIB.msa_debug_set_merge_poll_limit(int(polls)), "msa_debug_set_merge_poll_limit")


def msa_debug_set_merge_helper_poll_limit(polls: int):
    """Debug library: poll rounds after which a merging split other than the last to
    arrive hands its slice to the last one (< 0: the release bound; 0: at once, to force
    the handoff path). The release library raises MsaError."""
    _check(LIB.msa_debug_set_merge_helper_poll_limit(int(polls)), "msa_debug_set_merge_helper_poll_limit")


def _check(status: int, what: str):
    if status != MSA_OK:
        raise MsaError(f"{what}: {LIB.msa_status_string(status).decode()}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise MsaError(f"{name} must be a CUDA (HIP) tensor")
    if dtype is not None and t.dtype != dtype:
        raise MsaError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise MsaError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


class KVPool:
    """One layer's paged pool on the GPU (layout documented in include/msa_decode.h)."""

    def __init__(self, fmt, num_pages, num_kv_heads, device="cuda", k_tensor_scale=1.0,
                 v_tensor_scale=1.0, k_page_scale=None, v_page_scale=None, index_fmt=IDX_E4M3,
                 index_tensor_scale=1.0):
        sizes = (ctypes.c_size_t * 5)()
        _check(LIB.msa_pool_bytes(fmt, num_pages, num_kv_heads, HEAD_DIM, INDEX_DIM, sizes),
               "msa_pool_bytes")
        isizes = (ctypes.c_size_t * 2)()
        _check(LIB.msa_index_bytes(index_fmt, num_pages, INDEX_DIM, isizes), "msa_index_bytes")
        self.fmt, self.num_pages, self.num_kv_heads = fmt, num_pages, num_kv_heads
        self.k_tensor_scale, self.v_tensor_scale = float(k_tensor_scale), float(v_tensor_scale)
        self.index_fmt, self.index_tensor_scale = index_fmt, float(index_tensor_scale)
        z = lambda n: torch.zeros(n, dtype=torch.uint8, device=device)   # pools start zeroed
        self.k_codes, self.v_codes = z(sizes[0]), z(sizes[1])
        self.index_k = z(isizes[0])
        self.index_scales = z(isizes[1]) if isizes[1] else None
        if fmt == FMT_FP8:
            mk = lambda s: (torch.ones(num_pages, dtype=torch.float32) if s is None
                            else torch.as_tensor(s, dtype=torch.float32)).to(device)
            self.k_scales, self.v_scales = mk(k_page_scale), mk(v_page_scale)
        else:
            self.k_scales, self.v_scales = z(sizes[2]), z(sizes[3])

    def arrays(self):
        a = {"k_codes": self.k_codes, "v_codes": self.v_codes, "k_scales": self.k_scales,
             "v_scales": self.v_scales, "index_k": self.index_k}
        if self.index_scales is not None:
            a["index_scales"] = self.index_scales
        return a

    def cstruct(self) -> MsaKvPool:
        return MsaKvPool(self.fmt, self.num_pages, self.num_kv_heads, HEAD_DIM, PAGE, INDEX_DIM,
                         self.k_codes.data_ptr(), self.v_codes.data_ptr(), self.k_scales.data_ptr(),
                         self.v_scales.data_ptr(), self.k_tensor_scale, self.v_tensor_scale,
                         self.index_k.data_ptr(), self.index_fmt,
                         self.index_scales.data_ptr() if self.index_scales is not None else None,
                         self.index_tensor_scale)

    def clone(self) -> "KVPool":
        c = object.__new__(KVPool)
        c.__dict__.update(self.__dict__)
        for k, v in self.arrays().items():
            setattr(c, k, v.clone())
        return c


def rows_per_seq_of(row_seq, num_seqs: int) -> int:
    """R if the request-major `row_seq` (host array) gives every one of the num_seqs
    requests exactly R consecutive rows, else 0 (not stated)."""
    rs = np.asarray(row_seq, dtype=np.int64).reshape(-1)
    if num_seqs <= 0 or rs.size == 0 or rs.size % num_seqs != 0:
        return 0
    r = rs.size // num_seqs
    return r if np.array_equal(rs, np.repeat(np.arange(num_seqs), r)) else 0


class Step:
    """Per-step metadata on the GPU: block table, row -> request, row -> position, and
    the number of selection tables per row (1: shared by the KV heads; the pool's KV-head
    count: one per KV head, with a table axis after the row in scores and selections).
    rows_per_seq (see msa_step_t): None derives it from a host `row_seq` (0 when
    row_seq is already a device tensor); an int states it."""

    def __init__(self, block_table, row_seq, row_pos, device="cuda", sel_tables=1, rows_per_seq=None):
        bt = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.block_table = bt
        self.num_seqs, self.max_blocks = bt.shape
        if rows_per_seq is None:
            on_device = isinstance(row_seq, torch.Tensor) and row_seq.device.type != "cpu"
            rows_per_seq = 0 if on_device else rows_per_seq_of(row_seq, self.num_seqs)
        self.rows_per_seq = int(rows_per_seq)
        self.row_seq = torch.as_tensor(row_seq, dtype=torch.int32).to(device).contiguous()
        self.row_pos = torch.as_tensor(row_pos, dtype=torch.int32).to(device).contiguous()
        self.num_rows = self.row_pos.numel()
        self.sel_tables = sel_tables

    def cstruct(self) -> MsaStep:
        return MsaStep(self.num_seqs, self.num_rows, self.max_blocks, self.block_table.data_ptr(),
                       self.row_seq.data_ptr(), self.row_pos.data_ptr(), self.sel_tables, self.rows_per_seq)


def msa_kv_append(pool: KVPool, slot, k_new=None, v_new=None, idx_k_new=None, stream=None):
    n = slot.numel()
    ps = pool.cstruct()
    _check(LIB.msa_kv_append(ctypes.byref(ps), n, _ptr(slot, torch.int64, "slot"),
                             _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
                             _ptr(idx_k_new, torch.bfloat16, "idx_k_new"), _stream(stream)),
           "msa_kv_append")


def msa_index_score(pool: KVPool, step: Step, q_idx, w, block_scores, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_index_score(ctypes.byref(ps), ctypes.byref(ss), q_idx.shape[1],
                               _ptr(q_idx, torch.bfloat16, "q_idx"), _ptr(w, torch.float32, "w"),
                               _ptr(block_scores, torch.float32, "block_scores"), _stream(stream)),
           "msa_index_score")


def msa_select_topk(step: Step, block_scores, k, n_init, n_local, sel, sel_pages=None, stream=None):
    ss = step.cstruct()
    _check(LIB.msa_select_topk(ctypes.byref(ss), _ptr(block_scores, torch.float32, "block_scores"),
                               k, n_init, n_local, _ptr(sel, torch.int32, "sel"),
                               _ptr(sel_pages, torch.int32, "sel_pages"), _stream(stream)),
           "msa_select_topk")


def msa_append_score_select(pool: KVPool, step: Step, q_idx, w, k, n_init, n_local, block_scores,
                            sel=None, sel_pages=None, counters=None, slot=None, k_new=None, v_new=None,
                            idx_k_new=None, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    n = 0 if slot is None else slot.numel()
    _check(LIB.msa_append_score_select(
        ctypes.byref(ps), ctypes.byref(ss), n, _ptr(slot, torch.int64, "slot"),
        _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
        _ptr(idx_k_new, torch.bfloat16, "idx_k_new"), q_idx.shape[1],
        _ptr(q_idx, torch.bfloat16, "q_idx"), _ptr(w, torch.float32, "w"), k, n_init, n_local,
        _ptr(block_scores, torch.float32, "block_scores"), _ptr(sel, torch.int32, "sel"),
        _ptr(sel_pages, torch.int32, "sel_pages"), _ptr(counters, torch.int32, "counters"),
        _stream(stream)),
        "msa_append_score_select")


def msa_sparse_decode(pool: KVPool, step: Step, q, sel, k, softmax_scale, num_splits, part_o,
                      part_ml, sel_pages=None, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_sparse_decode(ctypes.byref(ps), ctypes.byref(ss), q.shape[1],
                                 _ptr(q, torch.bfloat16, "q"), _ptr(sel, torch.int32, "sel"),
                                 _ptr(sel_pages, torch.int32, "sel_pages"), k, float(softmax_scale),
                                 num_splits, _ptr(part_o, torch.float32, "part_o"),
                                 _ptr(part_ml, torch.float32, "part_ml"), _stream(stream)),
           "msa_sparse_decode")


def group_rows_of(row_seq, max_group_rows=4):
    """Row groups for msa_sparse_decode_union: each request's consecutive rows, cut into
    groups of at most max_group_rows. Returns the int32 offsets [groups + 1]."""
    import numpy as np
    rs = np.asarray(row_seq).ravel()
    starts = [0]
    for i in range(1, len(rs) + 1):
        if i == len(rs) or rs[i] != rs[i - 1] or i - starts[-1] == max_group_rows:
            starts.append(i)
    return np.asarray(starts, dtype=np.int32)


def msa_sparse_decode_union(pool: KVPool, step: Step, q, sel, k, group_rows, max_group_rows,
                            softmax_scale, num_splits, part_o=None, part_ml=None, out=None,
                            sel_pages=None, stream=None):
    """group_rows: device int32 [groups + 1] offsets (see group_rows_of)."""
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_sparse_decode_union(
        ctypes.byref(ps), ctypes.byref(ss), q.shape[1], _ptr(q, torch.bfloat16, "q"),
        _ptr(sel, torch.int32, "sel"), _ptr(sel_pages, torch.int32, "sel_pages"), k,
        group_rows.numel() - 1, _ptr(group_rows, torch.int32, "group_rows"), max_group_rows,
        float(softmax_scale), num_splits, _ptr(part_o, torch.float32, "part_o"),
        _ptr(part_ml, torch.float32, "part_ml"), _ptr(out, torch.bfloat16, "out"), _stream(stream)),
        "msa_sparse_decode_union")


def msa_sparse_decode_combine(pool: KVPool, step: Step, q, sel, k, softmax_scale, num_splits,
                              part_o, part_ml, counters, out, sel_pages=None, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_sparse_decode_combine(
        ctypes.byref(ps), ctypes.byref(ss), q.shape[1], _ptr(q, torch.bfloat16, "q"),
        _ptr(sel, torch.int32, "sel"), _ptr(sel_pages, torch.int32, "sel_pages"), k,
        float(softmax_scale), num_splits, _ptr(part_o, torch.float32, "part_o"),
        _ptr(part_ml, torch.float32, "part_ml"), _ptr(counters, torch.int32, "counters"),
        _ptr(out, torch.bfloat16, "out"), _stream(stream)),
        "msa_sparse_decode_combine")


def msa_sparse_decode_combine_noalloc(pool: KVPool, step: Step, q, sel, k, softmax_scale, num_splits, out,
                                      sel_pages=None, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_sparse_decode_combine_noalloc(
        ctypes.byref(ps), ctypes.byref(ss), q.shape[1], _ptr(q, torch.bfloat16, "q"),
        _ptr(sel, torch.int32, "sel"), _ptr(sel_pages, torch.int32, "sel_pages"), k,
        float(softmax_scale), num_splits, _ptr(out, torch.bfloat16, "out"), _stream(stream)),
        "msa_sparse_decode_combine_noalloc")


def msa_select_decode_combine(pool: KVPool, step: Step, q, block_scores, k, n_init, n_local,
                              softmax_scale, num_splits, part_o, part_ml, counters, out, sel=None,
                              sel_pages=None, stream=None):
    ps, ss = pool.cstruct(), step.cstruct()
    _check(LIB.msa_select_decode_combine(
        ctypes.byref(ps), ctypes.byref(ss), q.shape[1], _ptr(q, torch.bfloat16, "q"),
        _ptr(block_scores, torch.float32, "block_scores"), k, n_init, n_local, float(softmax_scale),
        num_splits, _ptr(part_o, torch.float32, "part_o"), _ptr(part_ml, torch.float32, "part_ml"),
        _ptr(counters, torch.int32, "counters"), _ptr(out, torch.bfloat16, "out"),
        _ptr(sel, torch.int32, "sel"), _ptr(sel_pages, torch.int32, "sel_pages"), _stream(stream)),
        "msa_select_decode_combine")


def msa_decode_step(pool: KVPool, step: Step, q_idx, w, q, k, n_init, n_local, softmax_scale, num_splits,
                    score_x, score_words, part_o, part_ml, counters, out, block_scores=None, sel=None,
                    sel_pages=None, slot=None, k_new=None, v_new=None, idx_k_new=None, stream=None,
                    unsupported_ok=False) -> bool:
    """The whole step in one launch. Returns True when launched; with unsupported_ok,
    False (nothing launched) for a shape outside the single-launch contract."""
    ps, ss = pool.cstruct(), step.cstruct()
    n = 0 if slot is None else slot.numel()
    st = LIB.msa_decode_step(
        ctypes.byref(ps), ctypes.byref(ss), n, _ptr(slot, torch.int64, "slot"),
        _ptr(k_new, torch.bfloat16, "k_new"), _ptr(v_new, torch.bfloat16, "v_new"),
        _ptr(idx_k_new, torch.bfloat16, "idx_k_new"), q_idx.shape[1], _ptr(q_idx, torch.bfloat16, "q_idx"),
        _ptr(w, torch.float32, "w"), q.shape[1], _ptr(q, torch.bfloat16, "q"), k, n_init, n_local,
        float(softmax_scale), num_splits, _ptr(score_x, torch.float32, "score_x"),
        _ptr(score_words, torch.int32, "score_words"), _ptr(part_o, torch.float32, "part_o"),
        _ptr(part_ml, torch.float32, "part_ml"), _ptr(counters, torch.int32, "counters"),
        _ptr(out, torch.bfloat16, "out"), _ptr(block_scores, torch.float32, "block_scores"),
        _ptr(sel, torch.int32, "sel"), _ptr(sel_pages, torch.int32, "sel_pages"), _stream(stream))
    if unsupported_ok and st == MSA_ERR_UNSUPPORTED:
        return False
    _check(st, "msa_decode_step")
    return True


def msa_step_workspace_init(rows, max_blocks, score_x, score_words, stream=None):
    _check(LIB.msa_step_workspace_init(rows, max_blocks, _ptr(score_x, torch.float32, "score_x"),
                                       _ptr(score_words, torch.int32, "score_words"), _stream(stream)),
           "msa_step_workspace_init")


def msa_combine(rows, num_q_heads, head_dim, num_splits, part_o, part_ml, out, stream=None):
    _check(LIB.msa_combine(rows, num_q_heads, head_dim, num_splits,
                           _ptr(part_o, torch.float32, "part_o"), _ptr(part_ml, torch.float32, "part_ml"),
                           _ptr(out, torch.bfloat16, "out"), _stream(stream)),
           "msa_combine")


def msa_merge_workspace_init(rows, num_q_heads, head_dim, num_splits, part_o, part_ml, counters,
                             stream=None):
    _check(LIB.msa_merge_workspace_init(rows, num_q_heads, head_dim, num_splits,
                                        _ptr(part_o, torch.float32, "part_o"),
                                        _ptr(part_ml, torch.float32, "part_ml"),
                                        _ptr(counters, torch.int32, "counters"), _stream(stream)),
           "msa_merge_workspace_init")


def msa_decode_workspace_bytes(rows, num_q_heads, head_dim, num_splits) -> int:
    return int(LIB.msa_decode_workspace_bytes(rows, num_q_heads, head_dim, num_splits))
