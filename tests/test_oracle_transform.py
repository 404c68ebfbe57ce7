"""Pins for the oracle's offline transform construction (Eq. 7, Eq. 8).

Each check comes from an identity or a closed form that the pages state.  Each
is computed here by a route other than the oracle's formula:
  * T_xvsh^T T_wush = I, so unquantized inner products are preserved
    (papernotes "整体框架"; ai.info summary; deep dive 3.4.2).
  * H H^T = I with entries +-G^-1/2 (deep dive 3.4.4, "Why U' = H").
  * Variance equalization: T_wush Sigma_x T_wush^T = T_xvsh Sigma_w T_xvsh^T
    = H S H^T, with constant diagonal tr(S)/G (deep dive 3.4.5 and 3.4.6; the
    Eq. 56 property cited in section 2).
  * FP-model objective.  At T_wush it equals (tr S)^2 / G, the lower bound of
    Eq. 20.  It is never lower for any other invertible transform (Eq. 17,
    Eq. 20; deep dive 3.4.4).  Here tr S comes from the eigenvalues of
    Sigma_w Sigma_x, not from an SVD.
  * GPTQ-route formula: T_wush = H S^1/2 V^T X'^-1 (Algorithm 1, line 8 form).
  * Special cases: isotropic moments, diagonal moments.
"""

import numpy as np
import pytest

from oracle import transform as tr
from synthetic import CONFIGS, gen_calibration, gen_weight


def _random_moments(rng, G, n=400, d_out=300, outliers=True):
    X = rng.standard_t(3.0, (n, G))
    W = rng.standard_normal((d_out, G)) * 0.02
    if outliers:
        X[:, rng.choice(G, 2, replace=False)] *= 30.0
    return W, X


def _moments_direct(W, X):
    return W.T @ W / W.shape[0], X.T @ X / X.shape[0]


def _objective(Tx, Sw, Sx):
    """sum_k (T_W Sw T_W^T)_kk (T_X Sx T_X^T)_kk with T_W = T_X^-T: the FP-model
    one-sided loss up to E[eta^2] (deep dive 3.4.4), in x coordinates."""
    Tw = np.linalg.inv(Tx).T
    return float(np.sum(np.diag(Tw @ Sw @ Tw.T) * np.diag(Tx @ Sx @ Tx.T)))


@pytest.mark.parametrize("G", [2, 4, 8, 16, 32, 64])
def test_hadamard(G):
    H = tr.hadamard(G)
    np.testing.assert_allclose(H @ H.T, np.eye(G), atol=1e-14)
    np.testing.assert_allclose(np.abs(H), G ** -0.5, rtol=0, atol=1e-15)
    scipy_linalg = pytest.importorskip("scipy.linalg")
    np.testing.assert_allclose(H, scipy_linalg.hadamard(G) / np.sqrt(G), atol=0)


@pytest.mark.parametrize("G", [16, 32])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_block_identities(G, seed):
    rng = np.random.default_rng(seed)
    W, X = _random_moments(rng, G)
    Sw, Sx = _moments_direct(W, X)
    b = tr.wush_block(Sw, Sx, lam=0.0)
    Tw, Tx = b.T_wush, b.T_xvsh
    # inverse-transpose pair
    np.testing.assert_allclose(Tx.T @ Tw, np.eye(G), atol=1e-9)
    # inner products survive: (T_xvsh w)^T (T_wush x) = w^T x
    w = rng.standard_normal(G)
    x = rng.standard_normal(G)
    assert abs((Tx @ w) @ (Tw @ x) - w @ x) < 1e-9 * (np.abs(w) @ np.abs(x) + 1)
    # tr S from eigenvalues of Sw Sx (singular values of W'^T X' squared)
    lam = np.linalg.eigvals(Sw @ Sx).real
    trS = np.sum(np.sqrt(np.clip(lam, 0, None)))
    H = tr.hadamard(G)
    for M in (Tw @ Sx @ Tw.T, Tx @ Sw @ Tx.T):
        np.testing.assert_allclose(np.diag(M), trS / G, rtol=1e-9)
        np.testing.assert_allclose(M, H @ np.diag(b.S) @ H.T, rtol=1e-8, atol=1e-12 * trS)
    # the objective attains the Eq. 20 bound and nothing beats it
    opt = _objective(Tw, Sw, Sx)
    np.testing.assert_allclose(opt, trS ** 2 / G, rtol=1e-9)
    trS2 = float(np.sum(np.clip(lam, 0, None)))
    assert trS ** 2 / G <= trS2 * (1 + 1e-12)  # Eq. 17, left inequality
    for _ in range(20):
        R = rng.standard_normal((G, G)) + 3 * np.eye(G)
        assert _objective(R, Sw, Sx) >= opt * (1 - 1e-9)
    assert _objective(H, Sw, Sx) >= opt * (1 - 1e-9)
    assert _objective(np.eye(G), Sw, Sx) >= opt * (1 - 1e-9)


@pytest.mark.parametrize("seed", [3, 4])
def test_gptq_route_agrees(seed):
    """H S^1/2 V^T X'^-1 is the same matrix as H S^-1/2 U^T W'^T."""
    G = 32
    rng = np.random.default_rng(seed)
    W, X = _random_moments(rng, G)
    Sw, Sx = _moments_direct(W, X)
    b = tr.wush_block(Sw, Sx, lam=0.0)
    alt = tr.hadamard(G) @ np.diag(np.sqrt(b.S)) @ b.V.T @ np.linalg.inv(b.Xp)
    np.testing.assert_allclose(alt, b.T_wush, rtol=1e-7, atol=1e-9 * np.abs(b.T_wush).max())
    # Algorithm 1 forms the interaction from the weight block and the
    # activation Cholesky factor: svd(W_blk X' / sqrt(d_out)) has the same
    # singular values and right vectors (up to sign) as svd(W'^T X').
    s2 = np.linalg.svd(W @ b.Xp / np.sqrt(W.shape[0]), compute_uv=False)
    np.testing.assert_allclose(s2, b.S, rtol=1e-9)


def test_isotropic_special_case():
    """Sigma_w = aI, Sigma_x = bI  =>  T_wush^T T_wush = sqrt(a/b) I."""
    G, a, b = 32, 0.37, 5.0
    rng = np.random.default_rng(0)
    d_out, n = 4 * G, 8 * G
    Qw, _ = np.linalg.qr(rng.standard_normal((d_out, G)))
    Qx, _ = np.linalg.qr(rng.standard_normal((n, G)))
    W = np.sqrt(a * d_out) * Qw
    X = np.sqrt(b * n) * Qx
    Sw, Sx = tr.block_moments(W, X, G)
    np.testing.assert_allclose(Sw[0], a * np.eye(G), atol=1e-12)
    Tw, _ = tr.build_transforms(W, X, G, lam=0.0)
    np.testing.assert_allclose(Tw[0].T @ Tw[0], np.sqrt(a / b) * np.eye(G), atol=1e-10)


def test_diagonal_special_case():
    """Diagonal moments: column k of T_wush is +-(a_k/b_k)^(1/4) times a column
    of H, each column of H used once."""
    G = 16
    rng = np.random.default_rng(1)
    av = rng.uniform(0.1, 4.0, G)
    bv = rng.uniform(0.1, 4.0, G)
    b = tr.wush_block(np.diag(av), np.diag(bv), lam=0.0)
    H = tr.hadamard(G)
    used = set()
    for k in range(G):
        col = b.T_wush[:, k] / (av[k] / bv[k]) ** 0.25
        hits = [j for j in range(G) if np.allclose(np.abs(H.T @ col)[j], 1.0, atol=1e-10)]
        assert len(hits) == 1
        np.testing.assert_allclose(np.abs(col), G ** -0.5, atol=1e-10)
        used.add(hits[0])
    assert len(used) == G


def test_sign_canonicalization():
    G = 32
    rng = np.random.default_rng(5)
    W, X = _random_moments(rng, G)
    Sw, Sx = _moments_direct(W, X)
    b = tr.wush_block(Sw, Sx)
    lead = np.argmax(np.abs(b.V), axis=0)
    assert np.all(b.V[lead, np.arange(G)] > 0)
    np.testing.assert_allclose(b.Wp.T @ b.Xp, b.U @ np.diag(b.S) @ b.V.T, atol=1e-12)
    assert np.all(np.diff(b.S) <= 0)


def test_tiny_workload_transforms():
    """The tiny MXFP4 workload: every block satisfies the pair identity and the
    bf16 rounding of T stays within half a bf16 ulp."""
    wl = CONFIGS["tiny_mxfp4"]
    W, Xc = gen_weight(wl), gen_calibration(wl)
    Tw, Tx = tr.build_transforms(W, Xc, wl.G)
    assert Tw.shape == (wl.C, wl.G, wl.G)
    for c in range(wl.C):
        np.testing.assert_allclose(Tx[c].T @ Tw[c], np.eye(wl.G), atol=1e-8)
    bits = tr.transforms_to_bf16_bits(Tw)
    back = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.all(np.abs(back - Tw) <= np.abs(Tw) * 2.0 ** -8 + 1e-30)
