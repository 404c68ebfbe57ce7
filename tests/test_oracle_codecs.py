"""Pins for the oracle's number formats.  Checks: brute force over the
formats' value tables, exhaustive fp32 sweeps, and library casts.

The encodings are the public OCP MX (E2M1, E8M0), OCP FP8 (E4M3) and IEEE
binary16 definitions.  The pages name MXFP4 / NVFP4 / INT4 but print no
example.  Every decode table below is written out here from those definitions,
independently of ``oracle.codecs``.
"""

import numpy as np
import pytest

from oracle import codecs

# ---------------------------------------------------------------- E2M1


def _e2m1_levels_from_bits():
    """All 16 E2M1 codes decoded from sign/exponent/mantissa fields."""
    vals = []
    for code in range(16):
        s = (code >> 3) & 1
        e = (code >> 1) & 3
        m = code & 1
        mag = (m * 0.5) if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)
        vals.append(-mag if s else mag)
    return np.array(vals)


def _e2m1_brute(v):
    """Nearest level over all 16 codes; ties -> even magnitude code; the sign
    of the result follows the sign of the input."""
    lv = _e2m1_levels_from_bits()
    mags = np.abs(lv[:8])
    a = np.abs(v.astype(np.float64))
    d = np.abs(a[:, None] - mags[None, :])
    dmin = d.min(axis=1, keepdims=True)
    cand = d == dmin
    # among tied candidates prefer an even code
    even = (np.arange(8) % 2 == 0)[None, :]
    pick_even = cand & even
    has_even = pick_even.any(axis=1)
    idx = np.where(has_even, np.argmax(pick_even, axis=1), np.argmax(cand, axis=1))
    # Above 6 the nearest level is 6 itself.  Float64 distances cannot
    # resolve that for huge inputs such as 1e30, so it is set directly.
    idx = np.where(a > 6.0, 7, idx)
    return (idx | (np.signbit(v).astype(np.int64) << 3)).astype(np.uint8)


def test_e2m1_table_matches_format_definition():
    lv = _e2m1_levels_from_bits()
    np.testing.assert_array_equal(np.abs(lv[:8]), codecs.E2M1_MAG)
    np.testing.assert_array_equal(codecs.e2m1_decode(np.arange(16)), lv)


@pytest.mark.parametrize("exp", list(range(-3, 3)))
def test_e2m1_exhaustive_fp32_octave(exp):
    """Every fp32 pattern with |v| in [2**exp, 2**(exp+1)), both signs."""
    base = np.uint32((exp + 127) << 23)
    mant = np.arange(1 << 23, dtype=np.uint32)
    pos = (base | mant).view(np.float32)
    for v in (pos, -pos):
        np.testing.assert_array_equal(codecs.e2m1_encode(v), _e2m1_brute(v))


def test_e2m1_outside_octaves():
    rng = np.random.default_rng(7)
    small = rng.uniform(0, 0.125, 200000).astype(np.float32)
    big = np.exp(rng.uniform(np.log(8), np.log(3e38), 200000)).astype(np.float32)
    specials = np.array([0.0, -0.0, 8.0, 6.0, 5.0, 5.000001, 1e-45, 3.4e38], dtype=np.float32)
    for v in (small, -small, big, -big, specials, -specials):
        np.testing.assert_array_equal(codecs.e2m1_encode(v), _e2m1_brute(v))


def test_e2m1_ties_go_to_even_code():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)
    expect = np.array([0, 2, 2, 4, 4, 6, 6], dtype=np.uint8)  # even codes
    np.testing.assert_array_equal(codecs.e2m1_encode(ties), expect)
    np.testing.assert_array_equal(codecs.e2m1_encode(-ties), expect | 8)


# ---------------------------------------------------------------- E8M0


def _floor_log2_bits(a):
    """floor(log2 a) for positive normal fp32 from its exponent field."""
    return ((a.view(np.uint32) >> 23) & 0xFF).astype(np.int64) - 127


def test_e8m0_places_max_in_4_to_8():
    rng = np.random.default_rng(3)
    a = np.exp(rng.uniform(np.log(1e-30), np.log(1e30), 100000)).astype(np.float32)
    pw = np.ldexp(np.float32(1), np.arange(-120, 120)).astype(np.float32)
    a = np.concatenate([a, pw, np.nextafter(pw, np.float32(0)), np.nextafter(pw, np.float32(np.inf))])
    code = codecs.e8m0_from_amax(a)
    e = code.astype(np.int64) - 127
    scaled = np.ldexp(a.astype(np.float64), -e)
    assert np.all((scaled >= 4.0) & (scaled < 8.0))
    np.testing.assert_array_equal(e, _floor_log2_bits(a) - 2)


def test_e8m0_clamps():
    a = np.array([0.0, 1e-45, 2.0 ** -126, 2.0 ** -125, 2.0 ** -124, 3.0e38], dtype=np.float32)
    code = codecs.e8m0_from_amax(a)
    # e = floor(log2 a) - 2, clamped at -127: 0, subnormal and 2^-126, 2^-125
    # all clamp; 2^-124 gives -126; 3e38 (2^127.8) gives 125.
    np.testing.assert_array_equal(code, [0, 0, 0, 0, 1, 252])


# ---------------------------------------------------------------- E4M3FN


def _e4m3_decode_bits(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return np.nan
    mag = (m / 8) * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return -mag if s else mag


def test_e4m3_table():
    vals = np.array([_e4m3_decode_bits(c) for c in range(127)])
    np.testing.assert_array_equal(vals, codecs.E4M3_VALUES)
    assert codecs.E4M3_VALUES[-1] == 448.0
    assert codecs.E4M3_VALUES[1] == 2.0 ** -9
    assert codecs.E4M3_VALUES[8] == 2.0 ** -6
    assert np.isnan(_e4m3_decode_bits(127))


def _e4m3_brute(x):
    vals = np.array([_e4m3_decode_bits(c) for c in range(127)])
    out = np.empty(x.shape, dtype=np.uint8)
    for i, xv in enumerate(x.astype(np.float64)):
        if xv >= 448.0:
            out[i] = 126
            continue
        d = np.abs(vals - xv)
        cand = np.flatnonzero(d == d.min())
        ev = [c for c in cand if c % 2 == 0]
        out[i] = ev[0] if ev else cand[0]
    return out


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(11)
    x = np.exp(rng.uniform(np.log(1e-5), np.log(1000), 20000)).astype(np.float32)
    v = codecs.E4M3_VALUES
    mids = ((v[1:] + v[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                        v.astype(np.float32), np.array([0, 448, 449, 464, 1e30], dtype=np.float32)])
    np.testing.assert_array_equal(codecs.e4m3_encode_pos(x), _e4m3_brute(x))


# ---------------------------------------------------------------- fp16 / bf16


def _f16_all_finite():
    vals = []
    for b in range(0x7C00):  # positive finite
        e = (b >> 10) & 0x1F
        m = b & 0x3FF
        vals.append((m / 1024) * 2.0 ** -14 if e == 0 else (1 + m / 1024) * 2.0 ** (e - 15))
    return np.array(vals)


def test_f16_rounding_brute_force():
    table = _f16_all_finite()
    rng = np.random.default_rng(5)
    x = np.exp(rng.uniform(np.log(1e-9), np.log(7e4), 20000)).astype(np.float32)
    mids = ((table[1:] + table[:-1]) / 2)[::37].astype(np.float32)
    x = np.concatenate([x, mids, np.array([65504, 65519, 65520, 1e6, 0.0], dtype=np.float32)])
    got = codecs.f32_to_f16_bits(x)
    xv = x.astype(np.float64)
    hi = np.searchsorted(table, xv)
    hi_c = np.minimum(hi, len(table) - 1)
    lo_c = np.maximum(hi_c - 1, 0)
    d_lo = xv - table[lo_c]
    d_hi = table[hi_c] - xv
    pick = np.where((d_hi < d_lo) | ((d_hi == d_lo) & (hi_c % 2 == 0)), hi_c, lo_c)
    pick = np.where(xv == table[hi_c], hi_c, pick)
    # IEEE overflow: at or beyond 65504 + half an ulp (65520) rounds to inf.
    pick = np.where(xv >= 65520.0, 0x7C00, pick)
    np.testing.assert_array_equal(got, pick.astype(np.uint16))


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(9)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-30, 30, 200000))).astype(np.float32)
    u = x.view(np.uint32)
    ties = ((u & 0xFFFF0000) | 0x8000).view(np.float32)  # exact halfway patterns
    x = np.concatenate([x, ties, np.array([0.0, -0.0, 1.0, 3.0e38], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(codecs.f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------- packing


def test_pack_roundtrip_and_order():
    c = np.array([[1, 2, 3, 4]], dtype=np.uint8)
    np.testing.assert_array_equal(codecs.pack_nibbles(c), [[0x21, 0x43]])
    rng = np.random.default_rng(1)
    r = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    np.testing.assert_array_equal(codecs.unpack_nibbles(codecs.pack_nibbles(r)), r)
    np.testing.assert_array_equal(codecs.int4_decode(np.arange(16)), list(range(8)) + list(range(-8, 0)))
