"""Build the C++ client of the C ABI (tests/c_client/wush_client).

The client links libwush.so (found next to the package through its run
path) and uses only include/wush.h and the HIP runtime, so the GPU test that
runs it shows the library working in a process with no Python binding.
"""

from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "wush_client.cpp")
EXE = os.path.join(HERE, "wush_client")


def build_client(hipcc: str, verbose: bool = False) -> str:
    tmp = EXE + ".tmp"
    cmd = [hipcc, "-O2", "-std=c++17", "--offload-arch=gfx950", "-Wall",
           "-I", os.path.join(ROOT, "include"), "-o", tmp, SRC,
           "-L", os.path.join(ROOT, "mxfp4_activation_amd"), "-lwush",
           "-Wl,-rpath,$ORIGIN/../../mxfp4_activation_amd"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed on the C client (exit %d)" % r.returncode)
    os.replace(tmp, EXE)
    return EXE
