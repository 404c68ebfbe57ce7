"""Pins for the reference MXFP4 GEMM (oracle.gemm), independent of its code.

* Brute force: every entry is recomputed with exact rationals from the
  E2M1 bit definition (sign bit 3; exponent bits 2:1 with bias 1; mantissa
  bit 0; exponent 0 is subnormal) and E8M0 = 2**(byte - 127), written here
  from the OCP MX definition rather than through the codec tables.
* Closed form: an all-ones left operand gives the right operand's row sums.
* Eq. 10 (deep dive, section 3.4.6): quantizing T_wush x and T_xvsh w and
  multiplying recovers x^T w up to the quantization error, and fails
  when the weight side takes the wrong transform.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

from oracle import gemm, quant
from oracle import transform as tr
from synthetic import CONFIGS, f64_to_bf16_bits, gen_calibration, gen_weight, gen_x_rows
from synthetic.gemm_operands import gen_mx_operand


def _e2m1_value(nib: int) -> Fraction:
    s, e, m = (nib >> 3) & 1, (nib >> 1) & 3, nib & 1
    mag = Fraction(m, 2) if e == 0 else Fraction(2) ** (e - 1) * (1 + Fraction(m, 2))
    return -mag if s else mag


def _row_values(codes_row, scales_row):
    out = []
    for j, byte in enumerate(codes_row.tolist()):
        for nib in (byte & 0xF, byte >> 4):
            k = len(out)
            out.append(_e2m1_value(nib) * Fraction(2) ** (int(scales_row[k // 32]) - 127))
    return out


def test_brute_force_exact_rationals():
    M, N, K = 3, 5, 64
    ac, asc = gen_mx_operand(M, K, seed=11, scale_lo=120, scale_hi=134)
    bc, bsc = gen_mx_operand(N, K, seed=12, scale_lo=120, scale_hi=134)
    C = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
    A = [_row_values(ac[m], asc[m]) for m in range(M)]
    B = [_row_values(bc[n], bsc[n]) for n in range(N)]
    for m in range(M):
        for n in range(N):
            exact = sum(a * b for a, b in zip(A[m], B[n]))
            assert C[m, n] == float(exact), (m, n)
    absC = gemm.gemm_mxfp4_abs_ref(ac, asc, bc, bsc)
    assert absC[1, 2] == float(sum(abs(a * b) for a, b in zip(A[1], B[2])))


def test_all_ones_operand_gives_row_sums():
    K = 96
    ones = np.full((2, K // 2), 0x22, dtype=np.uint8)  # E2M1 code 2 = 1.0 in both nibbles
    ones_s = np.full((2, K // 32), 127, dtype=np.uint8)
    bc, bsc = gen_mx_operand(4, K, seed=3, scale_lo=125, scale_hi=129)
    C = gemm.gemm_mxfp4_ref(ones, ones_s, bc, bsc)
    for n in range(4):
        want = float(sum(_row_values(bc[n], bsc[n])))
        assert C[0, n] == want and C[1, n] == want


def test_entries_match_full_product():
    ac, asc = gen_mx_operand(7, 256, seed=5, scale_lo=100, scale_hi=150)
    bc, bsc = gen_mx_operand(9, 256, seed=6, scale_lo=100, scale_hi=150)
    C = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
    A = gemm.gemm_mxfp4_abs_ref(ac, asc, bc, bsc)
    rows = np.array([0, 6, 3, 3])
    cols = np.array([8, 0, 4, 5])
    c, a = gemm.gemm_entries_ref(ac, asc, bc, bsc, rows, cols)
    # Scales spanning 2^-27..2^23 make the float64 sums order-dependent in
    # their last bits.
    np.testing.assert_allclose(c, C[rows, cols], rtol=1e-14, atol=0)
    np.testing.assert_allclose(a, A[rows, cols], rtol=1e-14, atol=0)


def _quantized(bits, T64):
    codes, scales = quant.run_path("mxfp4", bits, tr.transforms_to_bf16_bits(T64))
    return codes, scales


@pytest.mark.parametrize("transform", ["wush", "identity"])
def test_eq10_forward_recovers_product(transform):
    wl = CONFIGS["tiny_mxfp4"]
    x_bits = gen_x_rows(wl, 0, 64)
    x = (x_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    W = gen_weight(wl)[:48]
    w_bits = f64_to_bf16_bits(W)
    if transform == "wush":
        Tw, Tx = tr.build_transforms(gen_weight(wl), gen_calibration(wl), wl.G)
    else:
        Tw = Tx = np.broadcast_to(np.eye(wl.G), (wl.K // wl.G, wl.G, wl.G)).copy()
    xc, xs = _quantized(x_bits, Tw)
    wc, ws = _quantized(w_bits, Tx)
    C = gemm.gemm_mxfp4_ref(xc, xs, wc, ws)
    ref = x @ W.T
    rel = np.linalg.norm(C - ref) / np.linalg.norm(ref)
    assert rel < (0.1 if transform == "wush" else 0.25), rel
    if transform == "wush":
        # The weight side must take T_xvsh: T_xvsh^T T_wush = I, while
        # T_wush^T T_wush is not the identity.
        wc2, ws2 = _quantized(w_bits, Tw)
        rel_wrong = np.linalg.norm(gemm.gemm_mxfp4_ref(xc, xs, wc2, ws2) - ref) / np.linalg.norm(ref)
        assert rel_wrong > 5 * rel, (rel, rel_wrong)
