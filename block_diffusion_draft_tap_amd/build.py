"""Build libdflash.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m block_diffusion_draft_tap_amd.build

Each source compiles to an object in _build/ in parallel, then hipcc links the
shared library next to this file. Packed-fp32 instruction selection is turned
off for the device code.
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build", "dflash")
LIB = os.path.join(PKG, "libdflash.so")

SOURCES = ["gemv.hip", "gemm.hip", "skinny.hip", "attention.hip", "head.hip", "rope.hip", "i4mm.hip", "noalloc.hip",
           "dflash_api.cpp"]
ARCH = os.environ.get("DFLASH_ARCH", "gfx950")


def hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libdflash.so)")


def common_flags():
    extra = os.environ.get("DFLASH_DEFINES", "").split()  # -DNAME=VALUE tuning overrides
    return extra + ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-Wno-unused-result"]


def _compile(src):
    obj = os.path.join(BUILD, src + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=True, out=None, build_dir=None):
    global BUILD
    if build_dir:
        BUILD = build_dir
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    lib = out or LIB
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
