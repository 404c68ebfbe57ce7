"""Pins for GPTQ-WUSH (oracle.gptq, Algorithm 1), independent of its code.

* Algebra: with the weight quantizer off, the layer sum_b Wbar_b^T (T_X,b x_b)
  reproduces x W^T for any calibration data, in both modes.  A wrong
  transform, orientation, block order or Y update breaks it.
* Two routes to the transform (deep dive, section 3.4.6, line 8 against
  Eq. 8): when the calibration covariance is block-diagonal, the global
  Cholesky factor is block-diagonal too, and Algorithm 1's T_X for every
  block equals Eq. 8's T_wush built from the same damped moment.
* GPTQ step: the sequential Cholesky updates equal the closed-form optimal
  compensation (minimize (w - w0)^T Hb (w - w0) over the coordinates not yet
  quantized), recomputed from explicit inverses; and Hb = I gives RTN.
* Purpose: GPTQ lowers the weight quantization error on the calibration
  data relative to RTN.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import gptq
from oracle import transform as tr
from synthetic.layers import gen_linear_layer


@pytest.mark.parametrize("mode", [True, False])
def test_unquantized_layer_is_exact(mode):
    W, Xc, Xe = gen_linear_layer(128, 48, 512, 16, seed=2, n_outlier=2)
    r = gptq.gptq_wush_ref(W, Xc, 32, None, gptq=mode)
    out = gptq.layer_output(r, Xe, lambda v: v)
    ref = Xe @ W.T
    assert np.abs(out - ref).max() < 1e-9 * np.abs(ref).max()


def test_block_diagonal_covariance_gives_eq8_transform():
    rng = np.random.default_rng(4)
    d_in, d_out, G, m = 128, 64, 32, 96
    C = d_in // G
    W = rng.standard_normal((d_out, d_in)) * 0.02
    X = np.zeros((C * m, d_in))
    for b in range(C):  # each calibration token lives in one block: X^T X is block-diagonal
        X[b * m:(b + 1) * m, b * G:(b + 1) * G] = rng.standard_t(3, size=(m, G))
    r = gptq.gptq_wush_ref(W, X, G, None, gptq=False)
    Hx = X.T @ X / X.shape[0]
    Hx = Hx + gptq.DEFAULT_GPTQ_DAMP * np.mean(np.diag(Hx)) * np.eye(d_in)
    Sw, _ = tr.block_moments(W, X, G)
    for b in range(C):
        sl = slice(b * G, (b + 1) * G)
        eq8 = tr.wush_block(Sw[b], Hx[sl, sl], lam=0.0).T_wush
        assert np.abs(r.T_x[b] - eq8).max() < 1e-9 * np.abs(eq8).max()


def _obs_reference(w0, Hb, fmt):
    """Quantize coordinates in order; before each, set the remaining ones to
    the minimizer of (w - w0)^T Hb (w - w0) given the ones already fixed."""
    G = w0.shape[0]
    s, _ = gptq.group_scale(fmt, np.abs(w0).max(axis=0))
    q = np.zeros_like(w0)
    for o in range(w0.shape[1]):
        fixed = []
        for j in range(G):
            rest = np.arange(j, G)
            if fixed:
                f = np.array(fixed)
                d = w0[f, o] - q[f, o]
                # d/dw_rest of (w - w0)^T Hb (w - w0) = 0 with w_f = q_f
                w_rest = w0[rest, o] + np.linalg.solve(Hb[np.ix_(rest, rest)], Hb[np.ix_(rest, f)] @ d)
            else:
                w_rest = w0[rest, o]
            q[j, o] = gptq.quant_at_scale(fmt, np.array([w_rest[0]]), np.array([s[o]]))[0][0]
            fixed.append(j)
    return q


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_gptq_step_matches_closed_form(fmt):
    rng = np.random.default_rng(6)
    G, d_out = 8, 5
    A = rng.standard_normal((G, 3 * G))
    Hb = A @ A.T / (3 * G) + 0.1 * np.eye(G)
    w0 = rng.standard_normal((G, d_out))
    Q, _, _ = gptq.gptq_block(w0, Hb, fmt)
    np.testing.assert_allclose(Q, _obs_reference(w0, Hb, fmt), rtol=0, atol=1e-12)
    Qi, _, _ = gptq.gptq_block(w0, np.eye(G), fmt)
    Qr, _, _ = gptq.rtn_block(w0, fmt)
    np.testing.assert_array_equal(Qi, Qr)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_gptq_lowers_calibration_error(fmt):
    W, Xc, _ = gen_linear_layer(256, 64, 1024, 1, seed=8, n_outlier=3)
    ref = Xc @ W.T
    err = {}
    for mode in (True, False):
        r = gptq.gptq_wush_ref(W, Xc, 32, fmt, gptq=mode)
        err[mode] = np.mean((gptq.layer_output(r, Xc, lambda v: v) - ref) ** 2)
    assert err[True] < 0.9 * err[False], err
