"""GPTQ-WUSH (Algorithm 1), weight side, float64.  TEST INFRASTRUCTURE ONLY.

Source: "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep
dive, section 3.4.6 ("GPTQ Integration (Algorithm 1)").  Several of the
algorithm's formulas are garbled on the page; the steps below are the
reading that the surrounding text supports, and each is checked by the
pins in tests/test_oracle_gptq.py.

Orientation: W is [d_out, d_in] (nn.Linear order), calibration X is
[n, d_in]; block b covers input channels [bG, (b+1)G).

  1. Hessian Hx = X^T X / n, damped by damp * mean(diag(Hx)) * I; X' its
     lower Cholesky factor (global, d_in x d_in).
  2. Target Y = W X' (the layer in the Cholesky-transformed space).
  3. For b = C-1 down to 0 (reverse block order):
       U S V^T = SVD(Y[:, b])  (thin; singular values descending; each
                                (u_k, v_k) signed so v_k's largest-magnitude
                                entry is positive, as for Eq. 8)
       S <- S / sqrt(d_out)
       T_X = Hd S^1/2 V^T X'[b, b]^-1          (activation transform)
       Wbar = sqrt(d_out) Hd S^1/2 U^T          (transformed weights, [G, d_out];
                                                 equal to T_X^-T W_b^T when Y[:, b]
                                                 is exactly W_b X'[b, b])
       Wq = GPTQ(Wbar, Hd S Hd^T)  or  RTN(Wbar)
       Y <- Y - Wsub^T T_X X'[b, :],  Wsub = Wq (GPTQ) or Wbar (RTN)
     Hd is the normalized Hadamard matrix.
  4. The layer is then sum_b Wq_b^T q(T_X,b x_b) (Eq. 10).

Readings where the page is silent or garbled:
  * Damping: GPTQ's usual relative damping, default 0.01 * mean(diag(Hx)).
  * The quantization group of Wbar is the block: one scale per (output
    channel, block), the layout the FP4 GEMM consumes.  Its scale comes
    from the block's Wbar before the GPTQ updates (fixed for the block).
  * Elements are quantized at that scale in fp32 with the same element
    rules as the activations (E2M1 round-to-nearest-even with saturation;
    INT4 round-to-nearest-even clamped to +-7).
  * The intra-block GPTQ step is the standard one: with R the upper
    Cholesky factor of Hb^-1, for j = 0..G-1: q_j = quant(w_j),
    err = (w_j - q_j) / R[j, j], w_{>j} -= R[j, >j]^T err.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from . import codecs
from .transform import hadamard

DEFAULT_GPTQ_DAMP = 0.01


@dataclasses.dataclass
class GptqWush:
    T_x: np.ndarray     # [C, G, G] activation transforms
    Wq: np.ndarray      # [d_out, d_in] dequantized transformed weights (block b in columns b)
    codes: np.ndarray   # uint8 [d_out, d_in/2], element pairs of each block's group
    scales: np.ndarray  # [d_out, C]: E8M0 uint8 (MXFP4) or fp16 bits (INT4)


def _sign_canonical(U: np.ndarray, V: np.ndarray):
    lead = np.argmax(np.abs(V), axis=0)
    sgn = np.sign(V[lead, np.arange(V.shape[1])])
    sgn[sgn == 0] = 1.0
    return U * sgn, V * sgn


def group_scale(fmt: str, amax: np.ndarray):
    """Per-group scale value and stored code for the fixed-scale quantizer."""
    a32 = np.asarray(amax, dtype=np.float32)
    if fmt == "mxfp4":
        code = codecs.e8m0_from_amax(a32)
        return codecs.e8m0_value(code), code
    if fmt == "int4":
        s16 = codecs.f32_to_f16_bits((a32 / np.float32(7.0)).astype(np.float32))
        return codecs.f16_bits_to_f32(s16).astype(np.float64), s16
    raise ValueError(fmt)


def quant_at_scale(fmt: str, w: np.ndarray, s: np.ndarray):
    """(dequantized values, nibble codes) of w at fixed per-element scales s."""
    with np.errstate(divide="ignore", invalid="ignore"):
        v = np.where(s > 0, (np.asarray(w, dtype=np.float64) / s), 0.0).astype(np.float32)
    if fmt == "mxfp4":
        code = codecs.e2m1_encode(v)
        return codecs.e2m1_decode(code) * s, code
    q = np.clip(np.round(v.astype(np.float64)), -7, 7)  # np.round: half to even
    return q * s, (q.astype(np.int64) & 0xF).astype(np.uint8)


def gptq_block(Wbar: np.ndarray, Hb: np.ndarray, fmt: str):
    """Intra-block GPTQ on Wbar [G, d_out] with Hessian Hb [G, G].
    Returns (dequantized [G, d_out], codes [G, d_out], scale codes [d_out])."""
    G = Wbar.shape[0]
    s, scode = group_scale(fmt, np.abs(Wbar).max(axis=0))
    R = np.linalg.cholesky(np.linalg.inv(Hb)).T  # upper
    W = np.array(Wbar, dtype=np.float64)
    Q = np.empty_like(W)
    codes = np.empty(W.shape, dtype=np.uint8)
    for j in range(G):
        Q[j], codes[j] = quant_at_scale(fmt, W[j], s)
        err = (W[j] - Q[j]) / R[j, j]
        W[j + 1:] -= np.outer(R[j, j + 1:], err)
    return Q, codes, scode


def rtn_block(Wbar: np.ndarray, fmt: str):
    s, scode = group_scale(fmt, np.abs(Wbar).max(axis=0))
    Q, codes = quant_at_scale(fmt, Wbar, s[None, :])
    return Q, codes, scode


def gptq_wush_ref(W: np.ndarray, Xcal: np.ndarray, G: int, fmt, gptq: bool = True,
                  damp: float = DEFAULT_GPTQ_DAMP) -> GptqWush:
    """fmt None skips the weight quantizer (Wq = Wbar), for checking the algebra."""
    W = np.asarray(W, dtype=np.float64)
    X = np.asarray(Xcal, dtype=np.float64)
    d_out, d_in = W.shape
    C = d_in // G
    Hx = X.T @ X / X.shape[0]
    Hx = Hx + damp * np.mean(np.diag(Hx)) * np.eye(d_in)
    Xp = np.linalg.cholesky(Hx)
    Y = W @ Xp
    Hd = hadamard(G)
    T_x = np.empty((C, G, G))
    Wq = np.empty((d_out, d_in))
    codes = np.empty((d_out, d_in), dtype=np.uint8)
    scales = np.zeros((d_out, C), dtype=np.uint16 if fmt == "int4" else np.uint8)
    for b in reversed(range(C)):
        sl = slice(b * G, (b + 1) * G)
        U, s, Vt = np.linalg.svd(Y[:, sl], full_matrices=False)
        U, V = _sign_canonical(U, Vt.T)
        Sn = s / np.sqrt(d_out)
        T = Hd @ (np.sqrt(Sn)[:, None] * V.T) @ np.linalg.inv(Xp[sl, sl])
        Wbar = np.sqrt(d_out) * Hd @ (np.sqrt(Sn)[:, None] * U.T)
        if fmt is None:
            Q, c, sc = Wbar, np.zeros(Wbar.shape, dtype=np.uint8), 0
            sub = Q
        elif gptq:
            Q, c, sc = gptq_block(Wbar, Hd @ np.diag(Sn) @ Hd.T, fmt)
            sub = Q
        else:
            Q, c, sc = rtn_block(Wbar, fmt)
            sub = Wbar
        Y[:, : (b + 1) * G] -= sub.T @ T @ Xp[sl, : (b + 1) * G]
        T_x[b] = T
        Wq[:, sl] = Q.T
        codes[:, sl] = c.T
        scales[:, b] = sc
    return GptqWush(T_x, Wq, codecs.pack_nibbles(codes), scales)


def layer_output(result: GptqWush, x_rows: np.ndarray, act_quant) -> np.ndarray:
    """sum_b Wq_b^T act_quant(T_X,b x_b) for float64 activations [n, d_in];
    act_quant maps transformed activations [n, G] to their quantized values
    (identity for the unquantized check)."""
    C, G, _ = result.T_x.shape
    out = np.zeros((x_rows.shape[0], result.Wq.shape[0]))
    for b in range(C):
        sl = slice(b * G, (b + 1) * G)
        out += act_quant(x_rows[:, sl] @ result.T_x[b].T) @ result.Wq[:, sl].T
    return out
