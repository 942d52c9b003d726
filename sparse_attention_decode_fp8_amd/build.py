"""Build libmsadecode.so in-tree with hipcc for gfx950.

    python sparse_attention_decode_fp8_amd/build.py [--jobs N]

Every HIP source is compiled to an object with `hipcc --offload-arch=gfx950`, then
linked into sparse_attention_decode_fp8_amd/libmsadecode.so next to this file (and the
bench's read-bandwidth reference into libmsaprobe.so).
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
SOURCES = ["kv_append.hip", "index_score.hip", "select_topk.hip", "sparse_decode.hip",
           "combine.hip", "api.cpp"]
# The bench's read-bandwidth reference, a library of its own (not part of the decode path).
PROBE_LIB = os.path.join(PKG, "libmsaprobe.so")
PROBE_SOURCES = ["stream_read.hip"]

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


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *HIP_FLAGS, *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
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
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=6)
    args = ap.parse_args()
    build(args.jobs, verbose=True)
    sys.exit(0)
