"""Build the HIP library librkv.so in-tree for gfx950 (hipcc, no JIT cache).

Usage: python -m fp8_ring_kv_amd.build  (or call build()).
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "librkv.so")
OBJ = os.path.join(ROOT, "_build")
SOURCES = ["rkv_api.cpp", "k_cache.hip", "k_attend.hip"]
# the benchmark's measurement aids: a library of their own, outside the cache ABI
PROBE_OUT = os.path.join(PKG, "librkv_probe.so")
PROBE_SOURCES = ["probe/k_probe.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    # packed fp32 ALU ops are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no value here is ever NaN: min/max need no quieting of their inputs
    # (infinities keep their meaning: -inf marks masked slots)
    "-fno-honor-nans",
    # every atomic here is issued by one lane: no wave-level aggregation, whose
    # broadcast of the returned value would wait for it on the spot
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-I", INCLUDE,
    "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(os.path.basename(src))[0] + ".o")
    extra = ["-I", os.path.join(CSRC, "probe")] if src.startswith("probe/") else []
    cmd = [hipcc(), *FLAGS, *extra, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source, link librkv.so and librkv_probe.so; returns the
    path of librkv.so."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with ThreadPoolExecutor(max_workers=len(srcs)) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[: len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], PROBE_OUT)
    if verbose:
        print(f"built {OUT} and {PROBE_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
