"""Builds the HIP library (libattn_dense.so) for gfx950 in-tree with hipcc."""
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_dense.so")
SOURCES = [os.path.join(CSRC, "attn_kernels.hip"), os.path.join(CSRC, "attn_pingpong.hip"),
           os.path.join(CSRC, "attn_na3d.hip"), os.path.join(CSRC, "attn_api.hip")]

# Packed FP32 VALU forms are disabled for all device code: the compiler otherwise
# emits them from ordinary float code.
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # no NaN semantics are relied on (infinities are): lets max/min skip the
             # canonicalisation of their inputs
             "-fno-honor-nans",
             "-Wall", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the attention library)")


def build(verbose: bool = False) -> str:
    cmd = [hipcc()] + HIP_FLAGS + ["-I" + INCLUDE, "-I" + CSRC, "-o", LIB + ".tmp"] + SOURCES
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libattn_dense.so")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
