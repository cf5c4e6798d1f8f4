"""Builds the gfx950 HIP library ``libawq_mi355x.so`` in-tree with hipcc.

Usage:  python -m weight_only_quantization_awq_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libawq_mi355x.so")
CALIB_LIB = os.path.join(PKG, "libawq_calib.so")

SOURCES = ["awq_api.hip", "awq_noalloc.hip", "k_stats.hip", "k_search.hip", "k_pack.hip", "k_decode.hip",
           "k_prefill.hip", "k_clip.hip"]
CALIB_SOURCES = ["calib.hip"]

# Packed fp32 VALU forms are disabled (-packed-fp32-ops); no fast-math, no
# flush of denormals: the quantiser must round exactly like IEEE float32.
HIP_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-fPIC",
    "-std=c++17",
    "-Wall",
    "-Wno-unused-result",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def _compile(src: str) -> str:
    obj = os.path.join(OUT_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 and link the two shared libraries
    (the AWQ library and the roofline calibration probes)."""
    os.makedirs(OUT_DIR, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), 8)) as ex:
        objs = dict(zip(srcs, ex.map(_compile, srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CALIB_SOURCES], CALIB_LIB)
    if verbose:
        print(f"built {LIB}\nbuilt {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
