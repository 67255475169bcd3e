"""Builds libstreamkl.so (HIP kernels + C ABI) for gfx950 in-tree with hipcc."""
from __future__ import annotations

import os
import shutil
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
SOURCES = [os.path.join(PKG_DIR, "csrc", "streamkl_kernels.hip")]
LIB_PATH = os.path.join(PKG_DIR, "libstreamkl.so")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libstreamkl.so)")


def build_library(verbose: bool = False) -> str:
    """Compile every HIP source for gfx950 into LIB_PATH (always recompiles). Returns the path."""
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
           # packed fp32 VALU forms are kept out of the generated code
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           # no NaN semantics: lets fmaxf map to v_max3_f32 without canonicalising MFMA results
           # (infinities, used for masking, are still honoured)
           "-fno-honor-nans",
           "-I", os.path.join(ROOT, "include"), "-o", tmp] + SOURCES
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + " ".join(cmd) + "\n" + res.stdout + res.stderr)
    if verbose:
        print(" ".join(cmd))
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build_library(verbose=True))
