"""Compile the HIP sources of the package into libsinkattn.so (gfx950).

hipcc cross-compiles for gfx950 without a GPU present.  The library is built
in-tree, next to this file, so that it travels with the source tree.
"""
from __future__ import annotations

import glob
import os
import subprocess

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
LIB_PATH = os.path.join(PKG_DIR, "libsinkattn.so")
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    # keep the compiler from forming packed fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA builtins write VGPRs: the wide attention kernel keeps its score
    # accumulators in VGPRs for the softmax and its O accumulators in AGPRs
    # through inline asm (code of the other kernels is unchanged by this)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    # loops marked for full unrolling stay fully unrolled even when their
    # bodies are large: the backward's dK/dV loop is unrolled over its 8 ring
    # slots, and left rolled it would index its score registers at run time
    "-mllvm", "-pragma-unroll-threshold=65536",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, "-I", CSRC, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
