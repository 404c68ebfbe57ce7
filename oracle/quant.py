"""Reference online path: per-block transform, then RTN AbsMax quantization.

Source pages ("WUSH: Near-Optimal Adaptive Transforms for LLM Quantization"):
  * Every token's activation row is cut into contiguous blocks of G channels.
    Block c covers channels [cG, (c+1)G) (deep dive, section 3.4.1, the
    block-diagonal constraint).
  * Each block is multiplied by its own T_wush(c) and then quantized.  The
    quantization group is the transform block (deep dive, sections 3.4.6 and
    3.4.7; Eq. 10; papernotes.org, "整体框架").
  * The quantizer is round-to-nearest with an AbsMax scale (abstract; deep
    dive, section 2, "The Core Problem").

Readings where the pages are silent:
  * Pre-quantization values.  y is the exact sum of the G products
    T[c][k][j] * x[j], rounded once to fp32.  The pages give no accumulation
    precision, and this is the plain definition.  The scale and the codes are
    then derived from y in fp32.
  * Scaled element, MXFP4.  y * 2**-e, which is exact.
  * Scaled element, NVFP4 and INT4.  y * r, where r is the correctly rounded
    fp32 reciprocal of the scale.  The multiply is one fp32 rounding.
  * Layout.  Codes are [M, K/2] bytes.  Element 2j goes in bits 3:0 of byte
    j and element 2j+1 in bits 7:4.  Scales are [M, K/G], row-major.
"""

from __future__ import annotations

from fractions import Fraction
from typing import Tuple

import numpy as np

from . import codecs

# ----------------------------------------------------------------------------
# transform: y = fp32(exact sum)


def _f32_round_fraction(q: Fraction) -> np.float32:
    """Round an exact rational to the nearest fp32, ties to even mantissa."""
    if q == 0:
        return np.float32(0.0)
    f = np.float32(float(q))  # float(q) is the correctly rounded float64
    cands = [f, np.nextafter(f, np.float32(np.inf)), np.nextafter(f, np.float32(-np.inf))]
    best = None
    for c in cands:
        if not np.isfinite(c):
            continue
        d = abs(Fraction(float(c)) - q)
        even = (np.array(c, dtype=np.float32).view(np.uint32) & 1) == 0
        key = (d, 0 if even else 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def exact_dot_f32(t_row: np.ndarray, x: np.ndarray) -> np.float32:
    """fp32 rounding of sum_j t_row[j] * x[j], computed in exact rationals."""
    q = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(t_row, x)), Fraction(0))
    return _f32_round_fraction(q)


def _exponent_span(a: np.ndarray, axis: int) -> np.ndarray:
    """max - min of the binary exponents of the non-zero entries along axis
    (0 when there are fewer than two non-zero entries)."""
    _, e = np.frexp(a)
    nz = a != 0
    hi = np.where(nz, e, -100000).max(axis=axis)
    lo = np.where(nz, e, 100000).min(axis=axis)
    return np.maximum(hi - lo, 0)


def transform_ref(x_bits: np.ndarray, t_bits: np.ndarray, return_abs: bool = False):
    """y[m, cG + k] = fp32( sum_j T[c][k][j] * X[m, cG + j] ), exact sum.

    x_bits: bf16 bits [M, K]; t_bits: bf16 bits [C, G, G] (T[c][k][j]
    multiplies x_j into y_k).  Returns float32 [M, K].  With
    ``return_abs`` it also returns A = sum_j |T[c][k][j] x_j| (float64), which
    bounds the rounding error of any fp32 accumulation order.

    Method.  A bf16 value has an 8-bit significand, so each product has at
    most 16 significant bits and is exact in float64.  Suppose the products'
    exponents span s octaves.  Then every partial sum is a multiple of the
    smallest product's last bit, and stays below 32 times the largest
    product.  That needs s + 21 bits.  So the float64 sum, in any order, is
    exact when s <= 32, and one cast to fp32 rounds it correctly.  The span
    is bounded by span(x) + span(T row).  For the remaining elements the
    float64 error is below E = 2**-47 * A.  If [S - E, S + E] rounds to a
    single fp32 value, that value is the answer.  Otherwise the element is
    recomputed in exact rationals.
    """
    M, K = x_bits.shape
    C, G, G2 = t_bits.shape
    if G != G2 or C * G != K:
        raise ValueError("shape mismatch")
    X = codecs.bf16_bits_to_f32(x_bits).astype(np.float64).reshape(M, C, G).transpose(1, 0, 2)
    T = codecs.bf16_bits_to_f32(t_bits).astype(np.float64)
    S = np.matmul(X, T.transpose(0, 2, 1))  # [C, M, G]
    y = S.astype(np.float32)
    exact = (_exponent_span(X, 2)[:, :, None] + _exponent_span(T, 2)[:, None, :]) <= 32
    A = None
    if return_abs or not exact.all():
        A = np.matmul(np.abs(X), np.abs(T).transpose(0, 2, 1))
    if not exact.all():
        c_i, m_i, k_i = np.nonzero(~exact)
        s_ = S[c_i, m_i, k_i]
        e_ = A[c_i, m_i, k_i] * 2.0 ** -47 + np.abs(s_) * 2.0 ** -52
        lo = (s_ - e_).astype(np.float32)
        hi = (s_ + e_).astype(np.float32)
        for j in np.nonzero(lo != hi)[0]:
            c, m, k = c_i[j], m_i[j], k_i[j]
            y[c, m, k] = exact_dot_f32(T[c, k], X[c, m])
    y[y == 0] = 0.0  # an exactly-zero sum is +0
    y = np.ascontiguousarray(y.transpose(1, 0, 2).reshape(M, K))
    if return_abs:
        return y, np.ascontiguousarray(A.transpose(1, 0, 2).reshape(M, K))
    return y


def transform_f64(x_bits: np.ndarray, T: np.ndarray) -> np.ndarray:
    """Float64 transform with an unrounded float64 T [C, G, G] (reference for
    the pre-quantization check against the un-rounded transform)."""
    M, K = x_bits.shape
    C, G, _ = T.shape
    X = codecs.bf16_bits_to_f32(x_bits).astype(np.float64).reshape(M, C, G).transpose(1, 0, 2)
    S = np.matmul(X, np.asarray(T, dtype=np.float64).transpose(0, 2, 1))
    return np.ascontiguousarray(S.transpose(1, 0, 2).reshape(M, K))


def group_amax(y: np.ndarray, G: int) -> np.ndarray:
    M, K = y.shape
    return np.abs(y.reshape(M, K // G, G)).max(axis=2).astype(np.float32)


# ----------------------------------------------------------------------------
# MXFP4: E2M1 elements, one E8M0 scale per 32


def scaled_mxfp4(y: np.ndarray, G: int = 32):
    """Scale codes and the scaled elements v = y * 2**-e (exact)."""
    M, K = y.shape
    sc = codecs.e8m0_from_amax(group_amax(y, G))
    e = sc.astype(np.int64) - 127
    v = np.ldexp(y.reshape(M, K // G, G).astype(np.float64), -e[..., None])
    return sc, v.astype(np.float32).reshape(M, K)


def quant_mxfp4_ref(y: np.ndarray, G: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    sc, v = scaled_mxfp4(y, G)
    return codecs.pack_nibbles(codecs.e2m1_encode(v)), sc


# ----------------------------------------------------------------------------
# NVFP4: E2M1 elements, one E4M3FN scale per 16, one fp32 tensor scale g

NVFP4_TENSOR_DIV = np.float32(6.0 * 448.0)  # E2M1 max times E4M3 max


def tensor_amax_ref(y: np.ndarray) -> np.float32:
    return np.float32(np.max(np.abs(y))) if y.size else np.float32(0.0)


def nvfp4_global_scale(tensor_amax) -> np.float32:
    """g = fp32(amax / 2688): the largest block scale then encodes as 448."""
    return np.float32(np.float32(tensor_amax) / NVFP4_TENSOR_DIV)


def scaled_nvfp4(y: np.ndarray, g, G: int = 16):
    """Block scale codes and scaled elements.

    sb = fp32(amax / 6); code = E4M3(fp32(sb / g)); eff = fp32(E4M3(code) * g);
    v = fp32(y * fp32(1 / eff)).  g == 0 or eff == 0 gives zero codes.
    """
    M, K = y.shape
    g = np.float32(g)
    amax = group_amax(y, G)
    sb = (amax / np.float32(6.0)).astype(np.float32)
    if g > 0:
        ratio = (sb / g).astype(np.float32)
        code = codecs.e4m3_encode_pos(ratio)
    else:
        code = np.zeros(amax.shape, dtype=np.uint8)
    eff = (codecs.e4m3_value(code).astype(np.float32) * g).astype(np.float32)
    with np.errstate(divide="ignore"):
        r = np.where(eff > 0, np.float32(1.0) / eff, np.float32(0.0)).astype(np.float32)
    v = (y.reshape(M, K // G, G) * r[..., None]).astype(np.float32)
    return code, v.reshape(M, K)


def quant_nvfp4_ref(y: np.ndarray, g, G: int = 16) -> Tuple[np.ndarray, np.ndarray]:
    code, v = scaled_nvfp4(y, g, G)
    return codecs.pack_nibbles(codecs.e2m1_encode(v)), code


# ----------------------------------------------------------------------------
# INT4: symmetric levels -7..7, one fp16 AbsMax scale per 32

INT4_QMAX = 7


def scaled_int4(y: np.ndarray, G: int = 32):
    """fp16 scale s = fp16(fp32(amax / 7)); v = fp32(y * fp32(1 / float(s))).

    s == 0 (an all-zero group) gives r = 0 and therefore zero codes.
    """
    M, K = y.shape
    amax = group_amax(y, G)
    s16 = codecs.f32_to_f16_bits((amax / np.float32(INT4_QMAX)).astype(np.float32))
    s = codecs.f16_bits_to_f32(s16)
    with np.errstate(divide="ignore"):
        r = np.where(s > 0, np.float32(1.0) / s, np.float32(0.0)).astype(np.float32)
    v = (y.reshape(M, K // G, G) * r[..., None]).astype(np.float32)
    return s16, v.reshape(M, K)


def int4_round(v: np.ndarray) -> np.ndarray:
    """Round half to even, clamp to [-7, 7], two's-complement nibble."""
    q = np.clip(np.rint(v.astype(np.float64)), -INT4_QMAX, INT4_QMAX).astype(np.int32)
    return (q & 0xF).astype(np.uint8)


def quant_int4_ref(y: np.ndarray, G: int = 32) -> Tuple[np.ndarray, np.ndarray]:
    s16, v = scaled_int4(y, G)
    return codecs.pack_nibbles(int4_round(v)), s16


# ----------------------------------------------------------------------------
# dequantization (used by the error-bound pins and by the loss check)


def dequant_mxfp4(codes: np.ndarray, scales: np.ndarray, G: int = 32) -> np.ndarray:
    el = codecs.e2m1_decode(codecs.unpack_nibbles(codes))
    M, K = el.shape
    return (el.reshape(M, K // G, G) * codecs.e8m0_value(scales)[..., None]).reshape(M, K)


def dequant_nvfp4(codes, scales, g, G: int = 16) -> np.ndarray:
    el = codecs.e2m1_decode(codecs.unpack_nibbles(codes))
    M, K = el.shape
    eff = codecs.e4m3_value(scales) * float(np.float32(g))
    return (el.reshape(M, K // G, G) * eff[..., None]).reshape(M, K)


def dequant_int4(codes, scales16, G: int = 32) -> np.ndarray:
    q = codecs.int4_decode(codecs.unpack_nibbles(codes)).astype(np.float64)
    M, K = q.shape
    s = codecs.f16_bits_to_f32(scales16).astype(np.float64)
    return (q.reshape(M, K // G, G) * s[..., None]).reshape(M, K)


# ----------------------------------------------------------------------------
# whole path


def run_path(fmt: str, x_bits: np.ndarray, t_bits: np.ndarray, g=None):
    """Reference transform followed by the format's quantizer."""
    y = transform_ref(x_bits, t_bits)
    G = t_bits.shape[1]
    if fmt == "mxfp4":
        return quant_mxfp4_ref(y, G)
    if fmt == "nvfp4":
        if g is None:
            g = nvfp4_global_scale(tensor_amax_ref(y))
        return quant_nvfp4_ref(y, g, G)
    if fmt == "int4":
        return quant_int4_ref(y, G)
    raise ValueError(fmt)
