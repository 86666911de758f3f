"""Builds libmoe_mi355x.so (the C-ABI library) for gfx950 with hipcc, in-tree.

    python -m mixture_experts_routed_moe_amd.build

Cross-compiles without a GPU. Flags:
  --offload-arch=gfx950                       CDNA4 only, no other targets
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                              no packed fp32 VALU instructions
  -fno-gpu-flush-denormals-to-zero            keep fp32 subnormals (quantizer scales)
  -ffp-contract=fast-honor-pragmas            the SwiGLU sequence opts out of
                                              contraction with a pragma
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmoe_mi355x.so)")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def compile_flags():
    return ["--offload-arch=gfx950", "-O3", "-std=c++20", "-fPIC",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-fno-gpu-flush-denormals-to-zero", "-ffp-contract=fast-honor-pragmas",
            "-Wall", "-Wno-unused-function", "-I", INCLUDE, "-I", CSRC]


def build(verbose: bool = False, out: str = LIB_PATH) -> str:
    """Compiles every csrc/*.hip into one shared library; returns its path."""
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cc = hipcc()
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [cc, *compile_flags(), "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        objs.append(obj)
    tmp = out + ".tmp"
    cmd = [cc, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
