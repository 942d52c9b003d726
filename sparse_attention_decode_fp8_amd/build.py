"""Build libmsadecode.so in-tree with hipcc for gfx950.

    python sparse_attention_decode_fp8_amd/build.py [--jobs N]

Every HIP source is compiled to an object with `hipcc --offload-arch=gfx950`, then
linked into sparse_attention_decode_fp8_amd/libmsadecode.so next to this file; the same
sources built with -DMSA_DEBUG_CHECKS (device-side metadata checks) into
libmsadecode_debug.so; and the bench's read references (a streaming read and a read of
the step's selected pages) into libmsaprobe.so.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmsadecode.so")
# The same sources with the device-side metadata checks (MSA_DEBUG_CHECKS).
DEBUG_LIB = os.path.join(PKG, "libmsadecode_debug.so")
SOURCES = ["kv_append.hip", "index_score.hip", "select_topk.hip", "sparse_decode.hip", "union_decode.hip", "decode_no_alloc.hip",
           "combine.hip", "api.cpp"]
# The bench's read references, a library of their own (not part of the decode path).
PROBE_LIB = os.path.join(PKG, "libmsaprobe.so")
PROBE_SOURCES = ["stream_read.hip", "page_read.hip"]

COMMON = ["-O3", "-fPIC", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
          "-Wall", "-Wno-unused-function"]
# gfx950 only; packed-fp32 VALU ops are disabled for all device code.
HIP_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-fno-gpu-rdc", "-munsafe-fp-atomics"]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Per-source extras. sparse_decode.hip: its split-arrival counter update must not be
# rewritten into a wave-reduced form whose result is consumed at once (the workgroup
# reads the old count only after it has issued its partial's stores).
EXTRA = {"sparse_decode.hip": ["-mllvm", "-amdgpu-atomic-optimizer-strategy=None"]}


def _compile(src: str, debug: bool = False) -> str:
    out = os.path.join(BUILD, "debug") if debug else BUILD
    obj = os.path.join(out, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *HIP_FLAGS, *EXTRA.get(src, []), *(["-DMSA_DEBUG_CHECKS"] if debug else []),
           "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(jobs: int = 6, verbose: bool = False) -> str:
    os.makedirs(os.path.join(BUILD, "debug"), exist_ok=True)
    jobs_list = [(f, False) for f in SOURCES + PROBE_SOURCES] + [(f, True) for f in SOURCES]
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda fd: _compile(*fd), jobs_list))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    _link(objs[n:n + len(PROBE_SOURCES)], PROBE_LIB)
    _link(objs[n + len(PROBE_SOURCES):], DEBUG_LIB)
    if verbose:
        print(f"built {LIB}, {DEBUG_LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=6)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
