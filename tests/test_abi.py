"""The C-ABI library loads and exports every declared symbol; host-side validation
rejects out-of-contract calls before any launch (no GPU work happens here)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

from sparse_attention_decode_fp8_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for f in os.listdir(inc):
        if f.endswith(".h"):
            src = open(os.path.join(inc, f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(msa_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert {"msa_kv_append", "msa_index_score", "msa_select_topk", "msa_sparse_decode",
            "msa_combine"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", L.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (msa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(L.LIB, n) is not None


def test_debug_library_exports_the_same_entry_points_and_its_setter():
    """libmsadecode_debug.so (MSA_DEBUG_CHECKS) exports every declared symbol too; only
    it accepts an error word, and each build reports which one it is."""
    names = declared_symbols()
    assert {"msa_debug_set_error_word", "msa_debug_checks_enabled"} <= set(names)
    out = subprocess.run(["nm", "-D", "--defined-only", L.DEBUG_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (msa_\w+)", out))
    assert set(names) <= exported
    rel, dbg = L.load_library(L.RELEASE_LIB_PATH), L.load_library(L.DEBUG_LIB_PATH)
    assert rel.msa_debug_checks_enabled() == 0 and dbg.msa_debug_checks_enabled() == 1
    assert rel.msa_debug_set_error_word(ctypes.c_void_p(16)) == -2
    assert dbg.msa_debug_set_error_word(ctypes.c_void_p(16)) == 0
    assert dbg.msa_debug_set_error_word(None) == 0
    assert rel.msa_debug_set_merge_poll_limit(0) == -2
    assert dbg.msa_debug_set_merge_poll_limit(0) == 0 and dbg.msa_debug_set_merge_poll_limit(-1) == 0
    assert rel.msa_debug_set_merge_helper_poll_limit(0) == -2
    assert dbg.msa_debug_set_merge_helper_poll_limit(0) == 0 and dbg.msa_debug_set_merge_helper_poll_limit(-1) == 0
    # host-side validation is the same in both builds
    B, P = ctypes.byref, ctypes.c_void_p
    pool, step = _fake_pool(), _fake_step()
    for lib in (rel, dbg):
        assert lib.msa_index_score(B(pool), B(step), 3, P(16), P(16), P(16), None) == -2
        assert lib.msa_sparse_decode(B(pool), B(step), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16), None) == 0


def test_read_probe_library_loads_and_validates():
    """The bench's read references (libmsaprobe.so: a streaming read and a read of the
    step's selected pages) are exported and reject bad arguments before any launch."""
    lib = ctypes.CDLL(os.path.join(os.path.dirname(L.LIB_PATH), "libmsaprobe.so"))
    f = lib.msa_probe_stream_read
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p]
    assert f(None, 16, 16, 1, None) == -1            # null buffer
    assert f(16, 24, 16, 1, None) == -1              # not a multiple of 16 bytes
    assert f(16, 16, None, 1, None) == -1            # null sink
    assert f(16, 16, 16, 0, None) == -1              # no workgroups
    assert f(8, 16, 16, 1, None) == -1               # misaligned
    assert f(16, 0, 16, 1, None) == 0                # nothing to read: no launch
    g = lib.msa_probe_page_read                      # the bench's page-list read floor
    g.restype = ctypes.c_int
    g.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32] + [ctypes.c_void_p] * 4 + \
        [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    assert g(16, -1, 2, 16, 16, 16, 16, 4, 16, None) == -1   # negative unit count
    assert g(16, 1, 3, 16, 16, 16, 16, 4, 16, None) == -1    # unknown format
    assert g(16, 1, 2, 16, 16, 16, 16, 0, 16, None) == -1    # no KV heads
    assert g(16, 1, 2, None, 16, 16, 16, 4, 16, None) == -1  # null array
    assert g(16, 1, 2, 16, 16, 16, 16, 4, None, None) == -1  # null sink
    assert g(None, 0, 2, 16, 16, 16, 16, 4, 16, None) == 0   # nothing to read: no launch


def test_binding_names_match_c_entry_points():
    import sparse_attention_decode_fp8_amd as M
    for n in ("msa_kv_append", "msa_index_score", "msa_select_topk", "msa_sparse_decode",
              "msa_combine", "msa_decode_workspace_bytes"):
        assert callable(getattr(M, n))


def test_status_strings():
    for st, tag in ((0, "MSA_OK"), (-1, "INVALID_ARG"), (-2, "UNSUPPORTED"), (-3, "LAUNCH")):
        assert tag in L.LIB.msa_status_string(st).decode()


def test_pool_bytes_and_workspace():
    sz = (ctypes.c_size_t * 5)()
    assert L.LIB.msa_pool_bytes(2, 10, 4, 128, 64, sz) == 0
    assert list(sz) == [10 * 4 * 128 * 64] * 2 + [10 * 4 * 128 * 8] * 2 + [10 * 128 * 64]
    assert L.LIB.msa_pool_bytes(1, 10, 4, 128, 64, sz) == 0
    assert list(sz) == [10 * 4 * 128 * 128] * 2 + [40, 40, 10 * 128 * 64]
    assert L.LIB.msa_pool_bytes(3, 10, 4, 128, 64, sz) == -2
    assert L.LIB.msa_pool_bytes(2, 10, 4, 64, 64, sz) == -2
    ws = L.LIB.msa_decode_workspace_bytes(8, 64, 128, 4)
    assert ws == 8 * 64 * 4 * 128 * 4 + 8 * 64 * 4 * 2 * 4
    assert L.LIB.msa_decode_workspace_bytes(-1, 64, 128, 4) == 0
    isz = (ctypes.c_size_t * 2)()
    assert L.LIB.msa_index_bytes(1, 10, 64, isz) == 0 and list(isz) == [10 * 128 * 64, 0]
    assert L.LIB.msa_index_bytes(0, 10, 64, isz) == 0 and list(isz) == [10 * 128 * 64, 0]
    assert L.LIB.msa_index_bytes(2, 10, 64, isz) == 0 and list(isz) == [10 * 128 * 32, 10 * 128 * 4]
    assert L.LIB.msa_index_bytes(3, 10, 64, isz) == -2
    assert L.LIB.msa_index_bytes(2, 10, 32, isz) == -2
    assert L.LIB.msa_index_bytes(2, 0, 64, isz) == -1


def _fake_pool(fmt=2, head_dim=128, k_t=1.0, index_fmt=0, index_scales=None, index_t=0.0):
    # 16-byte aligned non-null host addresses: validation only, never dereferenced
    a = 1 << 20
    return L.MsaKvPool(fmt, 4, 2, head_dim, 128, 64, a, a, a, a, k_t, 1.0, a, index_fmt,
                       index_scales, index_t)


def _fake_step(rows=0, max_blocks=8, tables=0, rows_per_seq=0):
    a = 1 << 20
    return L.MsaStep(1, rows, max_blocks, a, a, a, tables, rows_per_seq)


def test_validation_rejects_before_launch():
    B = ctypes.byref
    P = ctypes.c_void_p
    pool, step = _fake_pool(), _fake_step()
    # empty work is OK and launches nothing
    assert L.LIB.msa_kv_append(B(pool), 0, None, None, None, None, None) == 0
    assert L.LIB.msa_index_score(B(pool), B(step), 4, P(16), P(16), P(16), None) == 0
    assert L.LIB.msa_select_topk(B(step), P(16), 8, 0, 1, P(16), None, None) == 0
    assert L.LIB.msa_sparse_decode(B(pool), B(step), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16), None) == 0
    assert L.LIB.msa_combine(0, 32, 128, 2, P(16), P(16), P(16), None) == 0
    # unsupported geometry
    assert L.LIB.msa_kv_append(B(_fake_pool(head_dim=64)), 1, P(16), None, None, None, None) == -2
    assert L.LIB.msa_kv_append(B(_fake_pool(fmt=7)), 1, P(16), None, None, None, None) == -2
    assert L.LIB.msa_index_score(B(pool), B(step), 3, P(16), P(16), P(16), None) == -2
    assert L.LIB.msa_select_topk(B(step), P(16), 0, 0, 1, P(16), None, None) == -2
    assert L.LIB.msa_select_topk(B(step), P(16), 65, 0, 1, P(16), None, None) == -2
    assert L.LIB.msa_select_topk(B(step), P(16), 4, 3, 2, P(16), None, None) == -2
    assert L.LIB.msa_select_topk(B(_fake_step(max_blocks=12289)), P(16), 4, 0, 1, P(16), None, None) == -2
    assert L.LIB.msa_sparse_decode(B(pool), B(step), 48, P(16), P(16), None, 8, 0.1, 2, P(16), P(16), None) == -2
    assert L.LIB.msa_sparse_decode(B(pool), B(step), 32, P(16), P(16), None, 8, 0.1, 9, P(16), P(16), None) == -2
    assert L.LIB.msa_combine(1, 32, 64, 2, P(16), P(16), P(16), None) == -2
    # invalid arguments
    assert L.LIB.msa_kv_append(None, 1, P(16), None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(pool), -1, P(16), None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(pool), 1, None, None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(pool), 1, P(16), P(18), None, None, None) == -1   # misaligned
    assert L.LIB.msa_kv_append(B(_fake_pool(k_t=0.0)), 1, P(16), None, None, None, None) == -1
    bad = _fake_pool()
    bad.k_codes = None
    assert L.LIB.msa_kv_append(B(bad), 1, P(16), None, None, None, None) == -1
    s1 = _fake_step(rows=1)
    assert L.LIB.msa_index_score(B(pool), B(s1), 4, None, P(16), P(16), None) == -1
    # a stated row count per request must be exact (num_rows == num_seqs * R) and >= 0
    for rps in (-1, 2):
        sr = _fake_step(rows=1, rows_per_seq=rps)
        assert L.LIB.msa_index_score(B(pool), B(sr), 4, P(16), P(16), P(16), None) == -1
        assert L.LIB.msa_select_topk(B(sr), P(16), 4, 0, 1, P(16), None, None) == -1
        assert L.LIB.msa_sparse_decode(B(pool), B(sr), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16),
                                       None) == -1
    assert L.LIB.msa_select_topk(B(s1), None, 4, 0, 1, P(16), None, None) == -1
    assert L.LIB.msa_sparse_decode(B(pool), B(s1), 32, P(16), P(16), None, 8, 0.0, 2, P(16), P(16), None) == -1
    assert L.LIB.msa_sparse_decode(B(pool), B(s1), 32, P(24), P(16), None, 8, 0.1, 2, P(16), P(16), None) == -1
    assert L.LIB.msa_combine(1, 32, 128, 2, None, P(16), P(16), None) == -1
    # the combining decode needs both its counters and its output
    assert L.LIB.msa_sparse_decode_combine(B(pool), B(s1), 32, P(16), P(16), None, 8, 0.1, 2, P(16),
                                           P(16), None, P(16), None) == -1
    assert L.LIB.msa_sparse_decode_combine(B(pool), B(s1), 32, P(16), P(16), None, 8, 0.1, 2, P(16),
                                           P(16), P(16), None, None) == -1
    assert L.LIB.msa_sparse_decode_combine(B(pool), B(step), 32, P(16), P(16), None, 8, 0.1, 2, P(16),
                                           P(16), P(16), P(16), None) == 0
    # the merge workspace fill: empty is OK; geometry and pointers are checked
    assert L.LIB.msa_merge_workspace_init(0, 32, 128, 2, None, None, None, None) == 0
    assert L.LIB.msa_merge_workspace_init(1, 32, 64, 2, P(16), P(16), P(16), None) == -2
    assert L.LIB.msa_merge_workspace_init(1, 24, 128, 2, P(16), P(16), P(16), None) == -2
    assert L.LIB.msa_merge_workspace_init(-1, 32, 128, 2, P(16), P(16), P(16), None) == -1
    assert L.LIB.msa_merge_workspace_init(1, 32, 128, 0, P(16), P(16), P(16), None) == -1
    assert L.LIB.msa_merge_workspace_init(1, 32, 128, 17, P(16), P(16), P(16), None) == -2
    assert L.LIB.msa_merge_workspace_init(1, 32, 128, 2, P(16), None, P(16), None) == -1
    # fused append + score + select
    assert L.LIB.msa_append_score_select(B(pool), B(step), 0, None, None, None, None, 4, P(16), P(16),
                                         8, 0, 1, P(16), P(16), None, P(16), None) == 0
    assert L.LIB.msa_append_score_select(B(pool), B(s1), 4097, P(16), None, None, None, 4, P(16),
                                         P(16), 8, 0, 1, P(16), P(16), None, P(16), None) == -2
    assert L.LIB.msa_append_score_select(B(pool), B(s1), 1, None, None, None, None, 4, P(16), P(16),
                                         8, 0, 1, P(16), P(16), None, P(16), None) == -1
    assert L.LIB.msa_append_score_select(B(pool), B(s1), 0, None, None, None, None, 4, P(16), P(16),
                                         8, 0, 1, P(16), P(16), None, None, None) == -1
    assert L.LIB.msa_append_score_select(B(pool), B(s1), 0, None, None, None, None, 3, P(16), P(16),
                                         8, 0, 1, P(16), P(16), None, P(16), None) == -2
    # index-key formats: E4M3 (0 or 1) needs nothing more; NVFP4 needs its scales and
    # a positive tensor scale; anything else is unsupported
    a16 = 1 << 20
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=1)), 0, None, None, None, None, None) == 0
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=2, index_scales=a16, index_t=0.5)), 0, None,
                               None, None, None, None) == 0
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=2, index_t=0.5)), 0, None, None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=2, index_scales=a16)), 0, None, None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=2, index_scales=a16 + 4, index_t=0.5)), 0, None,
                               None, None, None, None) == -1
    assert L.LIB.msa_kv_append(B(_fake_pool(index_fmt=5)), 0, None, None, None, None, None) == -2
    nullstep = L.MsaStep(1, 1, 8, None, None, None, 0)
    assert L.LIB.msa_index_score(B(pool), B(nullstep), 4, P(16), P(16), P(16), None) == -1
    # rows need at least one request
    noseq = L.MsaStep(0, 1, 8, P(16), P(16), P(16), 0)
    assert L.LIB.msa_index_score(B(pool), B(noseq), 4, P(16), P(16), P(16), None) == -1
    assert L.LIB.msa_select_topk(B(noseq), P(16), 4, 0, 1, P(16), None, None) == -1
    assert L.LIB.msa_sparse_decode(B(pool), B(noseq), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16), None) == -1


def test_selection_table_count_is_validated():
    """One table per row (0 or 1) or one per KV head (the fake pool has 2 KV heads);
    the scorer also needs the index heads to split evenly into the tables."""
    B, P = ctypes.byref, ctypes.c_void_p
    pool = _fake_pool()
    for T in (0, 1, 2):
        st = _fake_step(tables=T)
        assert L.LIB.msa_index_score(B(pool), B(st), 4, P(16), P(16), P(16), None) == 0
        assert L.LIB.msa_index_score(B(pool), B(st), 2, P(16), P(16), P(16), None) == 0
        assert L.LIB.msa_select_topk(B(st), P(16), 8, 0, 1, P(16), None, None) == 0
        assert L.LIB.msa_sparse_decode(B(pool), B(st), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16),
                                       None) == 0
        assert L.LIB.msa_append_score_select(B(pool), B(st), 0, None, None, None, None, 4, P(16), P(16),
                                             8, 0, 1, P(16), P(16), None, P(16), None) == 0
    t2 = _fake_step(tables=2)
    assert L.LIB.msa_index_score(B(pool), B(t2), 1, P(16), P(16), P(16), None) == -2   # 1 head, 2 tables
    t4 = _fake_step(tables=4)                        # 4 tables, 2 KV heads
    assert L.LIB.msa_index_score(B(pool), B(t4), 4, P(16), P(16), P(16), None) == -2
    assert L.LIB.msa_sparse_decode(B(pool), B(t4), 32, P(16), P(16), None, 8, 0.1, 2, P(16), P(16), None) == -2
    assert L.LIB.msa_select_decode_combine(B(pool), B(t4), 32, P(16), P(16), 8, 0, 1, 0.1, 2, P(16), P(16),
                                           P(16), P(16), None, None, None) == -2
    assert L.LIB.msa_append_score_select(B(pool), B(t4), 0, None, None, None, None, 4, P(16), P(16),
                                         8, 0, 1, P(16), P(16), None, P(16), None) == -2
    assert L.LIB.msa_select_topk(B(_fake_step(tables=5)), P(16), 8, 0, 1, P(16), None, None) == -2
    assert L.LIB.msa_select_topk(B(_fake_step(tables=-1)), P(16), 8, 0, 1, P(16), None, None) == -1


def test_binding_rejects_host_tensors():
    import torch
    with pytest.raises(L.MsaError):
        L._ptr(torch.zeros(4), torch.float32, "x")


def test_environment_selects_the_debug_library():
    """MSA_DEBUG_CHECKS=1 at import makes the binding load libmsadecode_debug.so."""
    code = ("import sparse_attention_decode_fp8_amd._lib as L; "
            "print(L.LIB_PATH.endswith('libmsadecode_debug.so'), L.LIB.msa_debug_checks_enabled())")
    env = dict(os.environ, MSA_DEBUG_CHECKS="1")
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True, env=env,
                         cwd=ROOT).stdout.split()
    assert out == ["True", "1"]
    env["MSA_DEBUG_CHECKS"] = "0"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, check=True, env=env,
                         cwd=ROOT).stdout.split()
    assert out == ["False", "0"]


def test_use_library_switches_and_restores():
    dbg = L.load_library(L.DEBUG_LIB_PATH)
    before = L.LIB
    with L.use_library(dbg) as lib:
        assert L.LIB is dbg and lib.msa_debug_checks_enabled() == 1
    assert L.LIB is before


def test_union_decode_validation_rejects_before_launch():
    B = ctypes.byref
    P = ctypes.c_void_p
    U = L.LIB.msa_sparse_decode_union
    pool, step, s1 = _fake_pool(), _fake_step(), _fake_step(rows=1)
    # args: pool, step, hq, q, sel, sel_pages, k, groups, group_rows, max_rows, scale, S, po, pm, out, stream
    assert U(B(pool), B(step), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 1, None, None, P(16), None) == 0
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 0, P(16), 4, 0.1, 1, None, None, P(16), None) == 0
    # geometry: heads, k, split count (up to 64, as msa_combine), group size
    assert U(B(pool), B(s1), 48, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 1, None, None, P(16), None) == -2
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 65, 1, P(16), 4, 0.1, 1, None, None, P(16), None) == -2
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 65, P(16), P(16), None, None) == -2
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 5, 0.1, 1, None, None, P(16), None) == -2
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 0, 0.1, 1, None, None, P(16), None) == -2
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 65536 // 2, P(16), 4, 0.1, 1, None, None, P(16),
             None) == -2
    # arguments: one split needs out, several need both partial arrays; group_rows, q, sel
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 1, P(16), P(16), None, None) == -1
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 2, None, P(16), P(16), None) == -1
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.1, 2, P(24), P(16), None, None) == -1
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, None, 4, 0.1, 1, None, None, P(16), None) == -1
    assert U(B(pool), B(s1), 32, None, P(16), None, 8, 1, P(16), 4, 0.1, 1, None, None, P(16), None) == -1
    assert U(B(pool), B(s1), 32, P(16), None, None, 8, 1, P(16), 4, 0.1, 1, None, None, P(16), None) == -1
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, -1, P(16), 4, 0.1, 1, None, None, P(16), None) == -1
    assert U(B(pool), B(s1), 32, P(16), P(16), None, 8, 1, P(16), 4, 0.0, 1, None, None, P(16), None) == -1


def test_no_alloc_entry_refuses_oversized_calls_on_the_host():
    """The allocation-free decode checks its fixed scratch limit before any HIP call."""
    B = ctypes.byref
    P = ctypes.c_void_p
    N = L.LIB.msa_sparse_decode_combine_noalloc
    pool = _fake_pool()
    # pool, step, hq, q, sel, sel_pages, k, scale, S, out, stream
    assert N(B(pool), B(_fake_step()), 32, P(16), P(16), None, 8, 0.1, 2, P(16), None) == 0
    # 8 MiB holds 16 rows x 32 heads x 16 splits x 130 fp32 (4.3 MB) but not 64 rows
    assert N(B(pool), B(_fake_step(rows=64)), 32, P(16), P(16), None, 8, 0.1, 16, P(16), None) == -4
    assert L.LIB.msa_status_string(-4).decode().startswith("MSA_ERR_TOO_LARGE")
    assert N(B(pool), B(_fake_step(rows=1)), 32, P(16), P(16), None, 8, 0.1, 17, P(16), None) == -2
    assert N(B(pool), B(_fake_step(rows=1)), 32, P(16), P(16), None, 8, 0.1, 0, P(16), None) == -1
    assert N(B(pool), B(_fake_step(rows=1)), 32, P(16), P(16), None, 8, 0.1, 2, None, None) == -1
    assert N(None, B(_fake_step(rows=1)), 32, P(16), P(16), None, 8, 0.1, 2, P(16), None) == -1


def test_single_launch_step_validation_rejects_before_launch():
    """msa_decode_step: arguments and the single-launch contract are checked on the host
    (nothing reaches a launch here: every call below returns before it)."""
    B, P = ctypes.byref, ctypes.c_void_p
    pool = _fake_pool()
    one = _fake_step(rows=1, rows_per_seq=1)

    def call(pool_=pool, step_=one, n_new=0, slot=None, n_idx=4, k=8, n_init=0, n_local=1, splits=2,
             counters=P(16), out=P(16), score_x=P(16), words=P(16), q_idx=P(16)):
        return L.LIB.msa_decode_step(B(pool_), B(step_), n_new, slot, None, None, None, n_idx, q_idx, P(16), 32,
                                     P(16), k, n_init, n_local, 0.1, splits, score_x, words, P(16), P(16),
                                     counters, out, None, None, None, None)

    # an empty step launches nothing
    assert call(step_=_fake_step(rows=0, rows_per_seq=0)) == 0
    # outside the single-launch contract: MSA_ERR_UNSUPPORTED, so the caller takes the
    # two-launch entries
    assert call(n_idx=2) == -2                                       # index heads other than 4
    assert call(pool_=_fake_pool(index_fmt=2, index_scales=1 << 20, index_t=0.5)) == -2   # NVFP4 keys
    assert call(step_=_fake_step(rows=1, tables=2, rows_per_seq=1)) == -2                  # per-KV-head tables
    assert call(step_=_fake_step(rows=1, rows_per_seq=0)) == -2      # row count per request not stated
    assert call(n_new=65, slot=P(16)) == -2                          # more than 64 new tokens
    assert call(k=8, splits=1) == -2                                 # one split of 8 blocks: 16-wave workgroups
    assert call(step_=_fake_step(rows=1, max_blocks=200, rows_per_seq=1), k=4, splits=4) == -2   # 200 blocks > 2 x 32 waves
    # invalid arguments
    assert call(n_new=-1) == -1
    assert call(n_new=1, slot=None) == -1
    assert call(counters=None) == -1
    assert call(out=None) == -1
    assert call(score_x=None) == -1
    assert call(words=None) == -1
    assert call(q_idx=None) == -1
    # the exchange set-up: empty is OK; geometry and pointers are checked
    assert L.LIB.msa_step_workspace_init(0, 8, None, None, None) == 0
    assert L.LIB.msa_step_workspace_init(-1, 8, P(16), P(16), None) == -1
    assert L.LIB.msa_step_workspace_init(1, 0, P(16), P(16), None) == -1
    assert L.LIB.msa_step_workspace_init(1, 12289, P(16), P(16), None) == -2
    assert L.LIB.msa_step_workspace_init(1, 8, None, P(16), None) == -1
