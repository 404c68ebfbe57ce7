"""Build the HIP shared library libwush.so in-tree for gfx950.

Usage: python -m mxfp4_activation_amd.build  (or call build()).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libwush.so")
SOURCES = ["wush_kernels.hip", "wush_gemm.hip", "wush_dequant.hip", "wush_build.hip", "wush_gptq.hip", "wush_abi.cpp"]

HIPCC_FLAGS = [
    "-O3",
    "-std=c++17",
    "--offload-arch=gfx950",
    "-fPIC",
    "-shared",
    # Products are rounded before any add: the code and the reference agree
    # on where fp32 rounding happens.
    "-ffp-contract=off",
    # No packed fp32 ops.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Matrix-core results go to ordinary VGPRs, not accumulation registers,
    # so the quantization code reads them without v_accvgpr_read copies.
    "-mllvm", "-amdgpu-mfma-vgpr-form=true",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def build(verbose: bool = False, extra_flags=None) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + HIPCC_FLAGS + list(extra_flags or []) + ["-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed (exit %d)" % r.returncode)
    if verbose and r.stderr.strip():
        sys.stderr.write(r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
