"""Offline WUSH transform construction, one G x G block at a time (float64).

Source pages ("WUSH: Near-Optimal Adaptive Transforms for LLM Quantization"):
  * Blockwise, uncentered second moments: Sigma_w = d_out^-1 W_(i) W_(i)^T and
    Sigma_x = d_batch^-1 X_(i) X_(i)^T.  Given in the papernotes.org summary,
    "关键设计" (WUSH 闭式构造), and the paper-graph deep dive, section 3.2
    ("Second-Moment Computer") and section 3.4.2.
  * W', X' are the lower-triangular Cholesky factors of those moments
    (deep dive 3.4.2).  U S V^T is the SVD of W'^T X' (Eq. 7).
  * The activation side gets T_wush = H S^-1/2 U^T W'^T and the weight side
    gets T_xvsh = H S^-1/2 V^T X'^T (Eq. 8, deep dive 3.4.4).  Together they
    satisfy T_xvsh^T T_wush = I.
  * H is the normalized Hadamard matrix, with G a power of two (deep dive 3.4.4,
    "Why U' = H").

Orientation.  The paper writes W in R^{d_in x d_out} and X in
R^{d_in x d_batch}, so channels are rows.  The inputs here use nn.Linear
order instead: a weight of shape [d_out, d_in] and calibration activations of
shape [n_cal, d_in].  Block c therefore takes columns [cG, (c+1)G) and
transposes them.

Readings where the pages are silent:
  * Damping.  The pages only say that a small damping term is added to the
    diagonal when a moment is rank-deficient.  Here both moments get
    lam * mean(diag) * I, with lam = 1e-6 by default.
  * SVD signs.  The pages do not fix them.  For each k, the pair (u_k, v_k) is
    flipped together so that v_k's largest-magnitude entry is positive; on a
    tie in magnitude, the lowest index wins.  T_wush depends on this choice,
    but every identity the pages state holds for either sign.
  * H is in Sylvester order, H_2n = [[H_n, H_n], [H_n, -H_n]], scaled by
    G^-1/2.
  * The kernel input is bf16(fp32(T_wush)): round to fp32 first, then to
    bf16, each step round-to-nearest-even.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

from .codecs import f32_to_bf16_bits

DEFAULT_DAMP = 1e-6


def hadamard(G: int) -> np.ndarray:
    """Normalized Sylvester Hadamard matrix of order G (a power of two)."""
    if G < 1 or G & (G - 1):
        raise ValueError("G must be a power of two")
    H = np.ones((1, 1))
    while H.shape[0] < G:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(G)


def block_moments(W: np.ndarray, Xcal: np.ndarray, G: int):
    """Per-block uncentered second moments.

    W: [d_out, d_in] (nn.Linear order); Xcal: [n_cal, d_in].
    Returns Sigma_w, Sigma_x of shape [C, G, G].
    """
    d_out, d_in = W.shape
    n_cal = Xcal.shape[0]
    if Xcal.shape[1] != d_in or d_in % G:
        raise ValueError("shape mismatch")
    C = d_in // G
    Wb = np.asarray(W, dtype=np.float64).reshape(d_out, C, G).transpose(1, 2, 0)  # [C, G, d_out]
    Xb = np.asarray(Xcal, dtype=np.float64).reshape(n_cal, C, G).transpose(1, 2, 0)  # [C, G, n_cal]
    Sw = np.matmul(Wb, Wb.transpose(0, 2, 1)) / d_out
    Sx = np.matmul(Xb, Xb.transpose(0, 2, 1)) / n_cal
    return Sw, Sx


def damp(S: np.ndarray, lam: float) -> np.ndarray:
    G = S.shape[-1]
    mean_diag = np.trace(S, axis1=-2, axis2=-1) / G
    return S + (lam * mean_diag)[..., None, None] * np.eye(G)


@dataclasses.dataclass
class BlockTransform:
    T_wush: np.ndarray  # activation side
    T_xvsh: np.ndarray  # weight side
    S: np.ndarray  # singular values of W'^T X', descending
    U: np.ndarray
    V: np.ndarray
    Wp: np.ndarray  # chol(Sigma_w + damping), lower
    Xp: np.ndarray  # chol(Sigma_x + damping), lower


def wush_block(Sw: np.ndarray, Sx: np.ndarray, lam: float = DEFAULT_DAMP,
               H: Optional[np.ndarray] = None) -> BlockTransform:
    """Eq. 7 and Eq. 8 for one block."""
    G = Sw.shape[0]
    if H is None:
        H = hadamard(G)
    Wp = np.linalg.cholesky(damp(Sw, lam))
    Xp = np.linalg.cholesky(damp(Sx, lam))
    U, s, Vt = np.linalg.svd(Wp.T @ Xp)
    V = Vt.T
    # Sign canonicalization: largest-|.| entry of every v_k positive.
    lead = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[lead, np.arange(G)])
    sgn[sgn == 0] = 1.0
    U = U * sgn
    V = V * sgn
    inv_sqrt_s = 1.0 / np.sqrt(s)
    T_wush = H @ (inv_sqrt_s[:, None] * U.T) @ Wp.T
    T_xvsh = H @ (inv_sqrt_s[:, None] * V.T) @ Xp.T
    return BlockTransform(T_wush, T_xvsh, s, U, V, Wp, Xp)


def build_transforms(W: np.ndarray, Xcal: np.ndarray, G: int,
                     lam: float = DEFAULT_DAMP, H: Optional[np.ndarray] = None):
    """All blocks of one layer.  Returns (T_wush, T_xvsh), each [C, G, G]."""
    Sw, Sx = block_moments(W, Xcal, G)
    C = Sw.shape[0]
    Tw = np.empty((C, G, G))
    Tx = np.empty((C, G, G))
    for c in range(C):
        b = wush_block(Sw[c], Sx[c], lam, H)
        Tw[c] = b.T_wush
        Tx[c] = b.T_xvsh
    return Tw, Tx


def transforms_to_bf16_bits(T: np.ndarray) -> np.ndarray:
    """bf16(fp32(T)), each step round-to-nearest-even, as uint16 bit patterns."""
    return f32_to_bf16_bits(np.asarray(T, dtype=np.float64).astype(np.float32))
