"""Number formats used by the online path (plain, vectorised NumPy).

The pages name MXFP4 (E2M1 elements with one shared 8-bit scale per 32),
NVFP4 (E2M1 elements, an FP8 scale per 16) and INT4 (symmetric AbsMax).
They do not give encodings.  The deep dive, section 2 ("New block-level
floating-point formats"), and the ai.info summary ("16-bit transforms ...
8-bit scales") are the closest they come.  The encodings below follow the
public OCP Microscaling v1.0 and OCP 8-bit floating point specifications,
plus IEEE 754 binary16 for the INT4 scale.

All rounding is round-to-nearest, ties-to-even.  Every encoder saturates at
the format's largest finite magnitude.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# bf16 (activations and transforms are bf16 bit patterns, uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16, round to nearest even on the bit pattern (finite x)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


# ----------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/nan.
# Magnitude code c = 0..7 has value E2M1_MAG[c]; the 4-bit code is sign<<3 | c.

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
E2M1_MAX = 6.0


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest E2M1 level; ties go to the even code.

    Magnitudes above 6 saturate to 6.  The sign of the input is kept, so a
    negative value that rounds to zero encodes as 0x8.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    code = np.zeros(a.shape, dtype=np.uint8)
    for i in range(7):
        mid = 0.5 * (E2M1_MAG[i] + E2M1_MAG[i + 1])
        # Strictly above the midpoint moves up.  Exactly on it moves up only
        # when the upper neighbour's code (i + 1) is even.
        up = (a > mid) | ((a == mid) & ((i + 1) % 2 == 0))
        code += up.astype(np.uint8)
    return code | (np.signbit(v).astype(np.uint8) << 3)


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    code = np.asarray(code, dtype=np.uint8)
    mag = E2M1_MAG[code & 7]
    return np.where(code & 8, -mag, mag)


def e2m1_level_index(code: np.ndarray) -> np.ndarray:
    """Position in the ordered level set -6..-0.5, 0, 0.5..6 (+0 and -0 equal)."""
    code = np.asarray(code, dtype=np.uint8)
    mag = (code & 7).astype(np.int32)
    return np.where(code & 8, -mag, mag)


# ----------------------------------------------------------------------------
# E8M0 shared scale (MXFP4): the scale is 2**(code - 127).


def e8m0_from_amax(amax: np.ndarray) -> np.ndarray:
    """Shared exponent e = floor(log2 amax) - 2, clamped to [-127, 127].

    2 is the exponent of E2M1's largest power of two (4).  Following the OCP
    MX rule, the group maximum therefore lands in [4, 8) after scaling, and
    values in [6, 8) saturate to 6.  amax = 0 (or any amax below 2**-125)
    clamps to e = -127.  Returns the biased code e + 127 (uint8).
    """
    amax = np.asarray(amax, dtype=np.float32)
    _, E = np.frexp(amax.astype(np.float64))  # amax = m * 2**E, m in [0.5, 1)
    floor_log2 = E.astype(np.int64) - 1
    e = np.where(amax > 0, floor_log2 - 2, -127)
    e = np.clip(e, -127, 127)
    return (e + 127).astype(np.uint8)


def e8m0_value(code: np.ndarray) -> np.ndarray:
    return np.ldexp(1.0, np.asarray(code, dtype=np.int64) - 127)


# ----------------------------------------------------------------------------
# E4M3FN (OCP FP8 E4M3): bias 7, no infinities, code 0x7F/0xFF is NaN,
# largest finite 448.  Only non-negative scales are produced here.


def _e4m3_table() -> np.ndarray:
    codes = np.arange(127)
    e = codes >> 3
    m = codes & 7
    sub = (m / 8.0) * 2.0 ** -6
    nrm = (1.0 + m / 8.0) * np.ldexp(1.0, e - 7)
    return np.where(e == 0, sub, nrm)


E4M3_VALUES = _e4m3_table()  # value of code 0..126, increasing
E4M3_MAX = 448.0


def e4m3_encode_pos(x: np.ndarray) -> np.ndarray:
    """Non-negative fp32 -> E4M3FN code, nearest with ties to even, saturating."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(x < 0) or np.any(~np.isfinite(x)):
        raise ValueError("e4m3_encode_pos expects finite non-negative input")
    hi = np.searchsorted(E4M3_VALUES, x, side="left")  # first value >= x
    hi = np.minimum(hi, 126)
    lo = np.maximum(hi - 1, 0)
    d_lo = x - E4M3_VALUES[lo]
    d_hi = E4M3_VALUES[hi] - x
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(x >= E4M3_VALUES[hi], hi, code)  # exact hit or above the top
    return code.astype(np.uint8)


def e4m3_value(code: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(code, dtype=np.int64)]


# ----------------------------------------------------------------------------
# binary16 scale (INT4): numpy's float32 -> float16 cast rounds to nearest even.


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):  # IEEE overflow to inf is the defined result
        return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def f16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


# ----------------------------------------------------------------------------
# nibble packing: element 2j -> bits 3:0 of byte j, element 2j+1 -> bits 7:4


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    if codes.shape[-1] % 2:
        raise ValueError("last dimension must be even")
    lo = codes[..., 0::2] & 0xF
    hi = codes[..., 1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0xF
    out[..., 1::2] = packed >> 4
    return out


def int4_decode(code: np.ndarray) -> np.ndarray:
    """Two's-complement nibble -> integer in [-8, 7]."""
    c = np.asarray(code, dtype=np.int32) & 0xF
    return np.where(c >= 8, c - 16, c)
