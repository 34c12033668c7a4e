"""Build libvmoba.so in-tree: hipcc for the gfx950 kernels, g++ for host-only code.

Usage: ``python -m block_sparse_attention_layer_amd.build [-v]``.  The library lands
next to this file; objects go to ``_build/``.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libvmoba.so")

HIP_SOURCES = ["pool.hip", "select.hip", "attn_fwd.hip", "attn_bwd.hip", "noalloc.hip"]
HOST_SOURCES = ["validate.cpp", "api.cpp"]

ARCH = "gfx950"
HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # no packed-fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
]
GXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall"]


def _hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else shutil.which("hipcc")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l)  # host pass does not know the feature
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out)


def build(verbose=False, jobs=8):
    hipcc = _hipcc()
    if hipcc is None:
        raise RuntimeError("hipcc not found")
    os.makedirs(BUILD, exist_ok=True)
    steps = []
    objs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        steps.append([hipcc, *HIPCC_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src + ".o")
        objs.append(obj)
        steps.append(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), steps))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv[1:]))
