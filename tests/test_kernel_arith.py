"""Host proofs of the quantize kernel's replacements for division.

`div7` in wush_kernels.hip forms fp32(x / 7) as the product with fp32(1/7)
plus one FMA correction of its residual.  That equals the correctly rounded
quotient for every non-negative finite fp32 x (the only inputs the kernel
gives it: a group's AbsMax).  This test proves it exhaustively on the host
(IEEE fp32, no flush to zero, the same arithmetic the device performs),
2^31 - 2^23 inputs split over the host's cores.  The formula below is the
kernel's, written in C; a change to one must be made to both.

(The kernel's other replacement, the fp16-scale reciprocal built from the
hardware reciprocal, depends on that instruction's own rounding and is
checked on the device; the INT4 parity tests cover it on every workload.)
"""

import os
import shutil
import subprocess
import tempfile

import pytest

C_SRC = r"""
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>
static float f(uint32_t u) { float x; memcpy(&x, &u, 4); return x; }
static uint32_t u(float x) { uint32_t v; memcpy(&v, &x, 4); return v; }
static float div7(float x) {
  const float r = 1.0f / 7.0f;
  const float q = x * r;
  return fmaf(fmaf(-q, 7.0f, x), r, q);
}
int main(void) {
  long long bad = 0;
  #pragma omp parallel for reduction(+:bad) schedule(static)
  for (long long b = 0; b < 0x7F800000LL; ++b) {
    const float x = f((uint32_t)b);
    if (u(div7(x)) != u(x / 7.0f)) ++bad;
  }
  printf("%lld\n", bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_div7_is_correctly_rounded_for_every_nonnegative_float():
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "div7.c"), os.path.join(d, "div7")
        with open(src, "w") as fh:
            fh.write(C_SRC)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-o", exe, src, "-lm"], check=True)
        out = subprocess.run([exe], capture_output=True, text=True, timeout=600)
        assert out.stdout.strip() == "0", out.stdout + out.stderr
        assert out.returncode == 0
