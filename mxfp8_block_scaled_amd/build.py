"""Build libmxfp8.so in-tree with hipcc for gfx950.

    python -m mxfp8_block_scaled_amd.build        # or __graft_entry__.build()

Every HIP source is compiled to an object (in parallel), then linked into
``mxfp8_block_scaled_amd/libmxfp8.so`` next to the binding that loads it.
Always rebuilds: the call is the "does it build" check.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmxfp8.so")
# The benchmark's calibration kernels (read stream, scaled-MFMA loop): a
# library of their own, outside the layer's C ABI.
CALIB_LIB = os.path.join(PKG, "libmxfp8_calib.so")
CALIB_SOURCES = ["calib.hip"]
ARCH = "gfx950"

SOURCES = ["api.cpp", "quant.hip", "pack.hip", "gemm_tile.hip", "gemm_skinny.hip", "gemm_mid.hip", "gemm_slab.hip", "gemm_med.hip", "moe.hip", "noalloc.hip"]

# -packed-fp32-ops: hipcc must not form v_pk_{add,mul,fma}_f32 (the host pass
# warns that it does not know the feature; that is harmless).
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmxfp8.so)")


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc()] + FLAGS + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-4000:]}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, lib)


def build(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + CALIB_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[: len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], CALIB_LIB)
    if verbose:
        print(f"built {LIB} and {CALIB_LIB}")
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
