"""Reference MXFP4 GEMM (Eq. 10 forward).  TEST INFRASTRUCTURE ONLY.

Source: "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep
dive, section 3.4.6, Eq. 10.  At inference every block's transformed,
quantized activations meet that block's transformed, pre-quantized weights,
and the products of all blocks add up.  With both operands stored as MXFP4
rows over the same K axis this is one product of the decoded matrices:
    C[m][n] = sum_k a[m][k] * b[n][k].
The definition, written out: decode both operands with the codec, multiply
in float64.  Every product of two E2M1 values and two power-of-two scales is
exact in float64; the float64 sum carries at most a few float64 ulps, far
below the fp32 accumulation error the GPU is held to.
"""

from __future__ import annotations

import numpy as np

from . import quant


def gemm_mxfp4_ref(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """C [M][N] float64 from MXFP4 operands a [M][K] and b [N][K]."""
    a = quant.dequant_mxfp4(a_codes, a_scales)
    b = quant.dequant_mxfp4(b_codes, b_scales)
    return a @ b.T


def gemm_mxfp4_abs_ref(a_codes, a_scales, b_codes, b_scales) -> np.ndarray:
    """sum_k |a[m][k] b[n][k]|, the magnitude that scales an fp32 sum's error."""
    a = np.abs(quant.dequant_mxfp4(a_codes, a_scales))
    b = np.abs(quant.dequant_mxfp4(b_codes, b_scales))
    return a @ b.T


def gemm_entries_ref(a_codes, a_scales, b_codes, b_scales, rows, cols):
    """(C, sum |a b|) at the given (row, col) pairs only, for operands too large
    to multiply whole on the CPU."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    a = quant.dequant_mxfp4(a_codes[rows], a_scales[rows])
    b = quant.dequant_mxfp4(b_codes[cols], b_scales[cols])
    return np.einsum("ik,ik->i", a, b), np.einsum("ik,ik->i", np.abs(a), np.abs(b))
