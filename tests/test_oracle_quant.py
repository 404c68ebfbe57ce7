"""Pins for the oracle's reference transform and quantizers.

The checks are: hand-derived golden examples (tests/golden), brute force in
exact rationals, special transforms that reduce the path to plain quantization
of a known vector, power-of-two equivariance, and the dequantization error
bounds that follow from each grid's level spacing.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import codecs, quant
from oracle import transform as tr
from synthetic import CONFIGS, f64_to_bf16_bits, gen_calibration, gen_weight, gen_x_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(a):
    return f64_to_bf16_bits(np.asarray(a, dtype=np.float64))


def _eye_bits(C, G):
    return np.broadcast_to(_bits(np.eye(G)), (C, G, G)).copy()


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ------------------------------------------------------------ golden examples


def test_golden_mxfp4():
    fx = _load("mxfp4_hand.json")
    G, K = fx["G"], fx["K"]
    rows = fx["rows"]
    X = np.zeros((len(rows), K))
    for i, r in enumerate(rows):
        X[i, :len(r["x_block0"])] = r["x_block0"]
        for j, v in r["x_block1_sparse"].items():
            X[i, G + int(j)] = v
    T = np.zeros((2, G, G))
    T[0] = np.eye(G)
    for k in range(G):
        T[1, k, (k + 1) % G] = 1.0
    x_bits = _bits(X)
    np.testing.assert_array_equal(codecs.bf16_bits_to_f32(x_bits), X)  # exact inputs
    codes, scales = quant.run_path("mxfp4", x_bits, _bits(T))
    for i, r in enumerate(rows):
        assert list(scales[i]) == r["scales"], r["derivation"]
        assert codes[i, :16].tobytes().hex() == r["codes_hex"], r["derivation"]
        assert codes[i, 16:].tobytes().hex() == r["codes_block1_hex"], r["derivation"]


def test_golden_int4():
    fx = _load("int4_hand.json")
    G = fx["G"]
    X = np.zeros((len(fx["rows"]), G))
    for i, r in enumerate(fx["rows"]):
        X[i, :len(r["x"])] = r["x"]
    codes, s16 = quant.run_path("int4", _bits(X), _eye_bits(1, G))
    for i, r in enumerate(fx["rows"]):
        assert "%04x" % s16[i, 0] == r["scale_f16_hex"], r["derivation"]
        assert codes[i].tobytes().hex() == r["codes_hex"], r["derivation"]


def test_golden_nvfp4():
    fx = _load("nvfp4_hand.json")
    G = fx["G"]
    X = np.zeros((len(fx["rows"]), G))
    for i, r in enumerate(fx["rows"]):
        X[i, :len(r["x"])] = r["x"]
    codes, sc = quant.run_path("nvfp4", _bits(X), _eye_bits(1, G), g=np.float32(fx["g"]))
    for i, r in enumerate(fx["rows"]):
        assert sc[i, 0] == r["scale"], r["derivation"]
        assert codes[i].tobytes().hex() == r["codes_hex"], r["derivation"]


# ------------------------------------------------------------ transform step


def _fraction_dot_f32(t_row, x):
    q = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(t_row, x)), Fraction(0))
    if q == 0:
        return np.float32(0.0)
    # brute-force nearest fp32 among the bracketing candidates, ties to even
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.array(c, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def test_transform_exact_rounding_brute_force():
    """y equals the exactly rounded sum for random and cancelling inputs."""
    rng = np.random.default_rng(0)
    G, C, M = 32, 2, 6
    X = rng.standard_t(3, (M, C * G)) * np.exp(rng.uniform(-8, 8, (M, C * G)))
    T = rng.standard_normal((C, G, G)) * np.exp(rng.uniform(-6, 6, (C, G, G)))
    x_bits, t_bits = _bits(X), _bits(T)
    Xf = codecs.bf16_bits_to_f32(x_bits).astype(np.float64)
    Tf = codecs.bf16_bits_to_f32(t_bits).astype(np.float64)
    # plant near-total cancellation in row 0, block 0, output 0: x_j * t_j pairs
    Tf0 = Tf[0, 0].copy()
    Tf0[1] = -Tf0[0] * Xf[0, 0] / Xf[0, 1]
    t_bits[0, 0] = _bits(Tf0)
    Tf = codecs.bf16_bits_to_f32(t_bits).astype(np.float64)
    y = quant.transform_ref(x_bits, t_bits)
    for m in range(M):
        for c in range(C):
            for k in range(G):
                want = _fraction_dot_f32(Tf[c, k], Xf[m, c * G:(c + 1) * G])
                assert y[m, c * G + k] == want, (m, c, k)


def test_transform_double_rounding_case():
    """1 + 2^-24 + 2^-80: the exact sum lies just above the fp32 midpoint
    between 1 and 1 + 2^-23, so it rounds up.  A float64 accumulation drops
    the 2^-80 term and then lands on the tie, which would round down to 1."""
    G = 32
    x = np.zeros((1, G))
    x[0, :4] = [1.0, 2.0 ** -24, 2.0 ** -80, 2.0 ** -54]
    T = np.zeros((1, G, G))
    T[0, 0, :3] = 1.0
    T[0, 1, :3] = [1.0, 1.0, -1.0]  # just below the midpoint: rounds down
    T[0, 2, [0, 1, 3]] = 1.0  # span 54: float64 also drops the last term
    y = quant.transform_ref(_bits(x), _bits(T))
    assert y[0, 0] == np.float32(1.0 + 2.0 ** -23)
    assert y[0, 1] == np.float32(1.0)
    assert y[0, 2] == np.float32(1.0 + 2.0 ** -23)


def test_transform_cyclic_shift_not_transposed():
    """T[c][k][(k+s_c) % G] = 1 moves x_(k+s_c) into y_k (a transposed
    operand would move it the other way)."""
    rng = np.random.default_rng(1)
    G, C, M = 16, 3, 5
    X = rng.standard_normal((M, C * G))
    x_bits = _bits(X)
    T = np.zeros((C, G, G))
    shifts = [1, 5, 11]
    for c, s in enumerate(shifts):
        for k in range(G):
            T[c, k, (k + s) % G] = 1.0
    y = quant.transform_ref(x_bits, _bits(T))
    xf = codecs.bf16_bits_to_f32(x_bits)
    for c, s in enumerate(shifts):
        blk = xf[:, c * G:(c + 1) * G]
        np.testing.assert_array_equal(y[:, c * G:(c + 1) * G], np.roll(blk, -s, axis=1))


def test_transform_f64_shift_and_brute_force():
    """The float64 reference transform (unrounded T): the same cyclic shift
    as above moves x_(k+s_c) into y_k, and on a small case with a general T
    every output is within float64 summation error of the exact rational
    sum."""
    rng = np.random.default_rng(2)
    G, C, M = 16, 3, 4
    X = rng.standard_normal((M, C * G))
    x_bits = _bits(X)
    xf = codecs.bf16_bits_to_f32(x_bits).astype(np.float64)
    T = np.zeros((C, G, G))
    shifts = [2, 7, 15]
    for c, s in enumerate(shifts):
        for k in range(G):
            T[c, k, (k + s) % G] = 1.0
    y = quant.transform_f64(x_bits, T)
    for c, s in enumerate(shifts):
        np.testing.assert_array_equal(y[:, c * G:(c + 1) * G], np.roll(xf[:, c * G:(c + 1) * G], -s, axis=1))
    # General T (float64 entries, not bf16): within float64 summation error
    # of the exact rational sum, (G + 2) 2^-53 sum |T x| (G - 1 additions and
    # one product rounding per term).  A dropped term, a wrong index or a
    # transposed T is off by a whole term.
    Tg = rng.standard_normal((C, G, G))
    y = quant.transform_f64(x_bits, Tg)
    for m in range(M):
        for c in range(C):
            for k in range(G):
                terms = [Fraction(float(Tg[c, k, j])) * Fraction(float(xf[m, c * G + j])) for j in range(G)]
                exact, mag = sum(terms), sum(abs(t) for t in terms)
                assert abs(Fraction(float(y[m, c * G + k])) - exact) <= (G + 2) * mag / 2**53


def test_identity_transform_is_plain_mxfp4():
    """T = I: the path is plain OCP MXFP4 of X.  Checked element-wise against
    the round trip: every dequantized value is the grid level nearest x."""
    wl = CONFIGS["tiny_mxfp4"]
    x_bits = gen_x_bits(wl)
    codes, sc = quant.run_path("mxfp4", x_bits, _eye_bits(wl.C, 32))
    deq = quant.dequant_mxfp4(codes, sc)
    x = codecs.bf16_bits_to_f32(x_bits).astype(np.float64)
    M, K = x.shape
    scale = codecs.e8m0_value(sc)
    levels = np.concatenate([-codecs.E2M1_MAG[::-1], codecs.E2M1_MAG])
    for m in range(0, M, 7):
        for c in range(K // 32):
            xs = x[m, c * 32:(c + 1) * 32] / scale[m, c]
            dist = np.abs(xs[:, None] - levels[None, :])
            # same distance as the brute-force nearest level (at a tie both
            # neighbours qualify; the tie rule itself is pinned in the codec tests)
            np.testing.assert_array_equal(np.abs(np.abs(deq[m, c * 32:(c + 1) * 32]) / scale[m, c] - np.abs(xs)),
                                          dist.min(axis=1))


# ------------------------------------------------------------ invariances


@pytest.mark.parametrize("k", [-3, 1, 4])
def test_power_of_two_equivariance(k):
    rng = np.random.default_rng(2)
    G, C, M = 32, 4, 40
    X = rng.standard_t(3, (M, C * G))
    T = rng.standard_normal((C, G, G)) * 0.2
    xb, tb = _bits(X), _bits(T)
    xb2 = _bits(codecs.bf16_bits_to_f32(xb).astype(np.float64) * 2.0 ** k)
    c1, s1 = quant.run_path("mxfp4", xb, tb)
    c2, s2 = quant.run_path("mxfp4", xb2, tb)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s2.astype(int) - s1.astype(int), k)
    c1, s1 = quant.run_path("int4", xb, tb)
    c2, s2 = quant.run_path("int4", xb2, tb)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(codecs.f16_bits_to_f32(s2), codecs.f16_bits_to_f32(s1) * np.float32(2.0 ** k))
    T16 = rng.standard_normal((8, 16, 16)) * 0.2
    t16 = _bits(T16)
    y1 = quant.transform_ref(xb, t16)
    g1 = quant.nvfp4_global_scale(quant.tensor_amax_ref(y1))
    c1, s1 = quant.run_path("nvfp4", xb, t16)
    c2, s2 = quant.run_path("nvfp4", xb2, t16)
    g2 = quant.nvfp4_global_scale(quant.tensor_amax_ref(quant.transform_ref(xb2, t16)))
    assert g2 == g1 * np.float32(2.0 ** k)
    np.testing.assert_array_equal(c1, c2)
    np.testing.assert_array_equal(s1, s2)


# ------------------------------------------------------------ error bounds


def _wush_tiny():
    wl = CONFIGS["tiny_mxfp4"]
    Tw, _ = tr.build_transforms(gen_weight(wl), gen_calibration(wl), wl.G)
    return wl, gen_x_bits(wl), tr.transforms_to_bf16_bits(Tw)


def test_mxfp4_error_bound():
    """|deq - y| <= half the local level gap times the scale for magnitudes
    up to 6 times the scale, and <= 2 * scale in the [6, 8) saturation band."""
    wl, xb, tb = _wush_tiny()
    y = quant.transform_ref(xb, tb).astype(np.float64)
    codes, sc = quant.quant_mxfp4_ref(y.astype(np.float32))
    deq = quant.dequant_mxfp4(codes, sc)
    scale = np.repeat(codecs.e8m0_value(sc), 32, axis=1)
    v = np.abs(y) / scale
    gap = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    err = np.abs(deq - y) / scale
    inside = v <= 6
    assert np.all(err[inside] <= gap[inside] / 2 + 1e-12)
    assert np.all(err[~inside] <= 2.0)
    assert np.all(v < 8)


def test_int4_error_bound_and_range():
    wl, xb, tb = _wush_tiny()
    y = quant.transform_ref(xb, tb)
    codes, s16 = quant.quant_int4_ref(y)
    q = codecs.int4_decode(codecs.unpack_nibbles(codes))
    assert q.min() >= -7 and q.max() <= 7
    s = np.repeat(codecs.f16_bits_to_f32(s16).astype(np.float64), 32, axis=1)
    deq = quant.dequant_int4(codes, s16)
    # half a step, plus the fp16 rounding of the scale (<= 2^-11 relative per
    # step, at most 7 steps away)
    assert np.all(np.abs(deq - y) <= s * (0.5 + 7 * 2.0 ** -11) + 1e-30)
    # the group maximum maps to +-7
    amax_idx = np.abs(y.reshape(-1, 32)).argmax(axis=1)
    qa = np.abs(q.reshape(-1, 32)[np.arange(q.size // 32), amax_idx])
    assert np.all(qa[np.abs(y).reshape(-1, 32).max(axis=1) > 0] == 7)


def test_nvfp4_top_block_scale_and_bound():
    """With g from the tensor AbsMax, the block holding it encodes 448 (code
    126); every element error stays within the E2M1 half-gap times eff."""
    rng = np.random.default_rng(4)
    G, C, M = 16, 16, 64
    xb = _bits(rng.standard_t(3, (M, C * G)))
    tb = _bits(rng.standard_normal((C, G, G)) * 0.25)
    y = quant.transform_ref(xb, tb)
    amax = quant.tensor_amax_ref(y)
    g = quant.nvfp4_global_scale(amax)
    codes, sc = quant.quant_nvfp4_ref(y, g)
    top = np.unravel_index(np.argmax(np.abs(y)), y.shape)
    assert sc[top[0], top[1] // G] == 126
    assert sc.max() == 126
    deq = quant.dequant_nvfp4(codes, sc, g)
    eff = np.repeat(codecs.e4m3_value(sc) * float(g), G, axis=1)
    v = np.abs(y) / np.where(eff > 0, eff, 1)
    gap = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    ok = (v <= 6) & (eff > 0)
    err = np.abs(deq - y)
    assert np.all(err[ok] <= (gap[ok] / 2) * eff[ok] * (1 + 2.0 ** -20))
