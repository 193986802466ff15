"""Build libdsa.so in-tree with hipcc for gfx950.

    python -m sparse_attention_relu_amd.build

Every source under csrc/ is compiled to an object (in parallel) and linked
into ``sparse_attention_relu_amd/libdsa.so``. Packed-fp32 instructions are
disabled for all device code.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libdsa.so")
ARCH = "gfx950"

SOURCES = ["api.cpp", "profile.cpp", "indexer.hip", "union.hip", "mla.hip",
           "cache_write.hip"]
HEADERS = ["common.h", "kernels.h", "profile.h"]

COMMON_FLAGS = ["-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-function",
                f"--offload-arch={ARCH}", "-I", os.path.join(os.path.dirname(PKG), "include")]
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# per-source extras: the query-block attention keeps 256 accumulator registers
# live, which only fits when MFMA results may be placed in the VGPR form
EXTRA_FLAGS = {"mla.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"]}


def hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found (ROCm is required to build libdsa.so)")
    return exe


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
        cmd += DEVICE_FLAGS + EXTRA_FLAGS.get(src, [])
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    try:
        build()
    except RuntimeError as e:  # pragma: no cover - build tool
        print(e, file=sys.stderr)
        sys.exit(1)
