"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Every test here runs the kernels on the current HIP device and compares them,
element by element, with ``oracle``.  The oracle gets the same seeded bf16
inputs.  The bar is in tests/parity.py.
"""

import numpy as np
import pytest

from oracle import codecs, quant
from oracle import transform as tr
from synthetic import CONFIGS, f64_to_bf16_bits, gen_calibration, gen_weight

from . import cases, parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()  # raises if libwush.so is missing: no fallback
    yield


def _dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _run(fmt, x_bits, t_bits, g=None, n_exact=False):
    from mxfp4_activation_amd import ops

    X, T = _dev_bf16(x_bits), _dev_bf16(t_bits)
    gs = None
    if fmt == "nvfp4":
        gs = torch.tensor([np.float32(g)], dtype=torch.float32, device="cuda")
    ne = torch.zeros(1, dtype=torch.int32, device="cuda") if n_exact else None
    codes, scales = ops.quant(fmt, X, T, global_scale=gs, n_exact=ne)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    if fmt == "int4":
        s = s.view(np.uint16)
    if n_exact:
        return c, s, int(ne.item())
    return c, s


def _g_for(x_bits, t_bits):
    return quant.nvfp4_global_scale(quant.tensor_amax_ref(quant.transform_ref(x_bits, t_bits)))


# ---------------------------------------------------------------- element codec


def test_e2m1_encode_matches_oracle_on_fp32_octaves():
    """Every fp32 pattern with |v| in [2^-3, 8), both signs, plus values above
    and below that range and the exact ties."""
    from mxfp4_activation_amd import ops

    mant = np.arange(1 << 23, dtype=np.uint32)
    for exp in range(-3, 3):
        pos = (np.uint32((exp + 127) << 23) | mant).view(np.float32)
        for v in (pos, -pos):
            got = ops.e2m1_encode(torch.from_numpy(v).cuda()).cpu().numpy()
            np.testing.assert_array_equal(got, codecs.e2m1_encode(v), err_msg="octave 2^%d" % exp)
    rng = np.random.default_rng(0)
    extra = np.concatenate([
        rng.uniform(0, 0.125, 100000), np.exp(rng.uniform(np.log(8), np.log(3e38), 100000)),
        [0.0, -0.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 8.0, 1e-45]]).astype(np.float32)
    for v in (extra, -extra):
        got = ops.e2m1_encode(torch.from_numpy(v).cuda()).cpu().numpy()
        np.testing.assert_array_equal(got, codecs.e2m1_encode(v))


# ---------------------------------------------------------------- tiny workload


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_tiny_workload(fmt):
    G = 16 if fmt == "nvfp4" else 32
    _, tb = cases.transforms("tiny_mxfp4", G)
    xb = cases.x_full("tiny_mxfp4")
    g = _g_for(xb, tb) if fmt == "nvfp4" else None
    c, s = _run(fmt, xb, tb, g)
    rep = parity.check(fmt, xb, tb, c, s, g)
    print(fmt, rep)


# Shapes that leave partial tiles in M, partial 256-channel columns in K, or
# both, and launches that mix complete and partial workgroups (M past a
# multiple of 64, K a multiple of 256 plus a remainder).
_RAGGED = [(1, 32), (31, 64), (33, 256), (100, 96), (257, 160), (70, 256), (100, 512), (1000, 768),
           (96, 288), (130, 4096 + 32)]
_RAGGED_G16 = [(64, 48), (40, 272), (65, 16)]


@pytest.mark.parametrize("fmt,M,K", [(f, M, K) for f in ("mxfp4", "nvfp4", "int4") for M, K in _RAGGED] +
                         [("nvfp4", M, K) for M, K in _RAGGED_G16])
def test_ragged_shapes(fmt, M, K):
    G = 16 if fmt == "nvfp4" else 32
    assert K % G == 0
    rng = np.random.default_rng(M * 1000 + K)
    X = rng.standard_t(3, (M, K))
    X[:, rng.choice(K, max(1, K // 64), replace=False)] *= 30
    W = rng.standard_normal((min(2 * K, 512), K)) * 0.02
    Xc = rng.standard_t(3, (min(4 * K, 1024), K))
    T64, _ = tr.build_transforms(W, Xc, G)
    xb, tb = f64_to_bf16_bits(X), tr.transforms_to_bf16_bits(T64)
    g = _g_for(xb, tb) if fmt == "nvfp4" else None
    c, s = _run(fmt, xb, tb, g)
    parity.check(fmt, xb, tb, c, s, g)


def test_empty_batch_is_noop():
    import mxfp4_activation_amd as wush

    lib = wush.load()
    assert lib.wush_quant_mxfp4(None, None, 0, 256, None, None, None) == 0
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    T = torch.zeros((2, 32, 32), dtype=torch.bfloat16, device="cuda")
    c, s = wush.quant_mxfp4(X, T)
    assert c.shape == (0, 32) and s.shape == (0, 2)


# ---------------------------------------------------------------- special transforms


# The pages' comparators go through the same kernel (deep dive, section 5):
# identity (plain RTN), blockwise Hadamard (RTN-H), and WUS (WUSH with the
# Hadamard factor replaced by the identity).  A cyclic shift catches a
# transposed T.
@pytest.mark.parametrize("which", ["identity", "hadamard", "wus", "cyclic"])
@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_special_transforms(which, fmt):
    wl = CONFIGS["tiny_mxfp4"]
    G = 16 if fmt == "nvfp4" else 32
    C = wl.K // G
    if which == "identity":
        T = np.broadcast_to(np.eye(G), (C, G, G))
    elif which == "hadamard":
        T = np.broadcast_to(tr.hadamard(G), (C, G, G))
    elif which == "wus":
        T, _ = tr.build_transforms(gen_weight(wl), gen_calibration(wl), G, H=np.eye(G))
    else:
        T = np.zeros((C, G, G))
        for c in range(C):
            for k in range(G):
                T[c, k, (k + 2 * c + 1) % G] = 1.0
    tb = f64_to_bf16_bits(np.ascontiguousarray(T))
    xb = cases.x_full("tiny_mxfp4")
    g = _g_for(xb, tb) if fmt == "nvfp4" else None
    c, s = _run(fmt, xb, tb, g)
    parity.check(fmt, xb, tb, c, s, g)


@pytest.mark.parametrize("kind", ["identity", "hadamard"])
@pytest.mark.parametrize("G", [16, 32])
def test_fixed_banks_match_oracle(kind, G):
    """The library's fixed banks (wush_fixed_transforms) are bit-identical to
    the oracle's identity and normalized Sylvester Hadamard matrices, in
    float64 and in the bf16 kernel layout; wush_f64_to_bf16 matches the
    oracle's bf16(fp32(.)) on random values."""
    from mxfp4_activation_amd import ops

    C = 5
    ref = np.broadcast_to(np.eye(G) if kind == "identity" else tr.hadamard(G), (C, G, G)).copy()
    got64 = ops.fixed_transforms(kind, C, G, "cuda", f64=True).cpu().numpy()
    got16 = ops.fixed_transforms(kind, C, G, "cuda").view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got64, ref)
    np.testing.assert_array_equal(got16, tr.transforms_to_bf16_bits(ref))
    rng = np.random.default_rng(G)
    v = rng.standard_normal((3, G, G)) * np.exp2(rng.integers(-60, 60, (3, G, G)))
    got = ops.f64_to_bf16(torch.from_numpy(v).cuda()).view(torch.int16).cpu().numpy().view(np.uint16)
    np.testing.assert_array_equal(got, tr.transforms_to_bf16_bits(v))


def test_scale_boundaries_take_exact_path():
    """Groups whose maximum is an exact power of two sit on an E8M0 boundary.
    The kernel must detect them and recompute them exactly, so the scale
    stays bit-exact."""
    G, M = 32, 64
    rng = np.random.default_rng(5)
    X = rng.uniform(-1, 1, (M, 4 * G))
    X[:, ::G] = 2.0 ** rng.integers(-8, 8, (M, 4))  # an exact power of two in every group
    xb = f64_to_bf16_bits(X)
    tb = f64_to_bf16_bits(np.broadcast_to(np.eye(G), (4, G, G)).copy())
    c, s, n = _run("mxfp4", xb, tb, n_exact=True)
    parity.check("mxfp4", xb, tb, c, s)
    assert n >= 1
    c, s, n = _run("int4", xb, tb, n_exact=True)
    parity.check("int4", xb, tb, c, s)


def test_tied_candidates_in_both_lane_halves():
    """Groups whose maximum is held by several outputs at once, spread over
    both halves of the 32 outputs (each half lives in a different lane of
    the pair that owns the token), with near-ties one bf16 step below: every
    group sits on an E8M0 boundary and has several candidate outputs for
    the exact step.  Through T = I and through a signed permutation (which
    moves the tied outputs to other positions and halves), scales must be
    bit-exact and every group must take the exact step."""
    G, C, M = 32, 4, 96
    rng = np.random.default_rng(29)
    e = rng.integers(-6, 6, (M, C))
    # every other channel below half the planted maximum 2^e
    X = rng.uniform(-0.45, 0.45, (M, C * G)) * np.repeat(2.0 ** e, G, axis=1)
    below = 1.0 - 2.0 ** -8  # one bf16 step below 1
    for pos, mult in [(2, 1.0), (13, 1.0), (18, 1.0), (29, 1.0), (7, below), (24, below)]:
        sign = rng.choice([-1.0, 1.0], (M, C))
        for c in range(C):
            X[:, c * G + pos] = sign[:, c] * mult * 2.0 ** e[:, c]
    xb = f64_to_bf16_bits(X)
    perm = rng.permutation(G)
    P = np.zeros((G, G))
    P[np.arange(G), perm] = rng.choice([-1.0, 1.0], G)
    for T in (np.eye(G), P):
        tb = f64_to_bf16_bits(np.ascontiguousarray(np.broadcast_to(T, (C, G, G))))
        c, s, n = _run("mxfp4", xb, tb, n_exact=True)
        rep = parity.check("mxfp4", xb, tb, c, s)
        assert n == M * C, (n, M * C)
        assert rep.n_mismatch == 0
        for fmt in ("int4", "nvfp4"):
            Gf = 16 if fmt == "nvfp4" else 32
            tf = tb if Gf == 32 else f64_to_bf16_bits(np.ascontiguousarray(np.broadcast_to(T[:16, :16], (2 * C, 16, 16))))
            g = _g_for(xb, tf) if fmt == "nvfp4" else None
            c, s = _run(fmt, xb, tf, g)
            parity.check(fmt, xb, tf, c, s, g)


@pytest.mark.parametrize("g_mult", [1.0 / 16, 64.0, 0.0])
def test_nvfp4_static_tensor_scales(g_mult):
    """NVFP4 with a calibrated (static) tensor scale instead of the data's
    own: 16x smaller drives block scales into E4M3 saturation, 64x larger
    into its subnormal codes, and the smallest allowed g (2^-100) saturates
    every block.  This walks the reciprocal table and the scale decision's
    approximate ratio across the E4M3 range."""
    G, C, M = 16, 16, 200
    rng = np.random.default_rng(37)
    X = rng.standard_normal((M, C * G)) * (2.0 ** rng.integers(-12, 12, (M, 1)))
    xb = f64_to_bf16_bits(X)
    tb = f64_to_bf16_bits(rng.standard_normal((C, G, G)) * 0.25)
    g = np.float32(_g_for(xb, tb) * g_mult) if g_mult > 0 else np.float32(2.0 ** -100)
    c, s = _run("nvfp4", xb, tb, g)
    parity.check("nvfp4", xb, tb, c, s, g)
    if g_mult > 0:
        assert np.unique(s).size > 50  # the scales span much of the E4M3 range
    else:
        assert (s == 0x7E).all()  # every block at the largest finite E4M3 code


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_extreme_magnitudes(fmt):
    """Groups of tiny values (bf16 subnormals, E8M0 code 0), huge values (fp16
    scale overflow for INT4), all-zero groups, and a mix, through T = I and
    a random T."""
    G = 16 if fmt == "nvfp4" else 32
    rng = np.random.default_rng(11)
    C, M = 8, 96
    X = rng.standard_normal((M, C * G))
    X[0:8] *= 2.0 ** -128  # subnormal region
    X[8:16] *= 2.0 ** -122
    X[16:24] *= 2.0 ** 100
    X[24:32] = 0.0
    X[32:40, ::2] *= 2.0 ** -60  # wide spread inside a group
    X[40:48] *= 2.0 ** 18  # INT4 scale beyond fp16 range
    xb = f64_to_bf16_bits(X)
    for T in (np.broadcast_to(np.eye(G), (C, G, G)), rng.standard_normal((C, G, G)) * 0.3):
        tb = f64_to_bf16_bits(np.ascontiguousarray(T))
        g = _g_for(xb, tb) if fmt == "nvfp4" else None
        c, s = _run(fmt, xb, tb, g)
        parity.check(fmt, xb, tb, c, s, g)


# ---------------------------------------------------------------- long runs


# Batches big enough that workgroups take runs of 2 or 3 tiles, with a
# ragged last run:
# - MXFP4 and NVFP4, M = 4100 at K = 4096: two-tile runs, the last run one
#   partial tile;
# - INT4, M = 4136 at K = 8192: three-tile runs, the last run one partial
#   tile; M = 4168: the last run two tiles, the second partial;
# - MXFP4, M = 8200 at K = 4096: three-tile runs, the last run two tiles,
#   the second partial;
# - M = 4600 at K = 4128 and M = 8200 at K = 4128 add a partial 256-channel
#   column (17 panel groups): 17 x 72 = 1224 two-tile workgroups, a multiple
#   of 8, so the XCD remap applies; 17 x 86 = 1462 three-tile ones, which is
#   not.
# All of these grids exceed one resident wave of workgroups, so they take
# the token-major order.  Every row is checked.
@pytest.mark.parametrize("fmt,M,K", [("mxfp4", 4100, 4096), ("int4", 4136, 8192), ("nvfp4", 4100, 4096),
                                     ("int4", 4168, 8192), ("mxfp4", 8200, 4096),
                                     ("mxfp4", 4600, 4128), ("nvfp4", 4600, 4128), ("mxfp4", 8200, 4128)])
def test_long_runs_with_ragged_tail(fmt, M, K):
    print("case", fmt, M, K, flush=True)
    G = 16 if fmt == "nvfp4" else 32
    rng = np.random.default_rng(M + K)
    X = rng.laplace(0.0, 1.0, (M, K))
    X[:, rng.choice(K, K // 100, replace=False)] *= 50
    W = rng.standard_normal((256, K)) * 0.02
    Xc = rng.laplace(0.0, 1.0, (512, K))
    T64, _ = tr.build_transforms(W, Xc, G)
    xb, tb = f64_to_bf16_bits(X), tr.transforms_to_bf16_bits(T64)
    g = _g_for(xb, tb) if fmt == "nvfp4" else None
    c, s = _run(fmt, xb, tb, g)
    for lo in range(0, M, 4096):
        rep = parity.check(fmt, xb[lo:lo + 4096], tb, c[lo:lo + 4096], s[lo:lo + 4096], g)
        print(fmt, M, K, lo, rep, flush=True)


# ---------------------------------------------------------------- support entry points


@pytest.mark.parametrize("name,G", [("tiny_mxfp4", 16), ("tiny_mxfp4", 32), ("llama8b_mxfp4", 32)])
def test_transform_f32_error_bounds(name, G):
    """The unquantized transform (wush_transform_f32) on the tiny workload and
    on the whole 4096 x 4096 headline tensor.

    * Against the oracle on the same bf16 inputs (the pages' 16-bit T): every
      value within the accumulation bound the scale guard assumes, hence
      within 2e-3 of its group's AbsMax (the benchmark spec's tolerance, asserted).
    * Against the unrounded float64 T: the extra error is the bf16 storage of
      T, at most bf16's unit roundoff 2^-8 per entry (plus 2^-23 from the
      fp32 step) times sum_j |T64_kj x_j|; asserted, and the group-relative
      deviation is printed (it runs to about 4e-3, so 2e-3 does not hold
      against the float64 T and is not claimed there)."""
    from mxfp4_activation_amd import ops

    T64, tb = cases.transforms(name, G)
    xb = cases.x_full(name)
    M, K = xb.shape
    Y = ops.transform_f32(_dev_bf16(xb), _dev_bf16(tb)).cpu().numpy()
    for lo in range(0, M, 4096):
        x, yg = xb[lo:lo + 4096], Y[lo:lo + 4096].astype(np.float64)
        m = x.shape[0]
        y_ref, A = quant.transform_ref(x, tb, return_abs=True)
        bound = (2.0 ** -17) * A + (2.0 ** -21) * np.abs(y_ref) + 2.0 ** -120
        assert np.all(np.abs(yg - y_ref) <= bound)
        err = np.abs(yg - y_ref).reshape(m, K // G, G).max(axis=2)
        amax = np.abs(y_ref).reshape(m, K // G, G).max(axis=2).astype(np.float64)
        assert np.all(err <= 2e-3 * amax)
        y64 = quant.transform_f64(x, T64)
        Xc = codecs.bf16_bits_to_f32(x).astype(np.float64).reshape(m, K // G, G).transpose(1, 0, 2)
        A64 = np.matmul(np.abs(Xc), np.abs(T64).transpose(0, 2, 1)).transpose(1, 0, 2).reshape(m, K)
        assert np.all(np.abs(yg - y64) <= (2.0 ** -8 + 2.0 ** -23) * A64 + bound)
        g64 = np.abs(y64).reshape(m, K // G, G).max(axis=2)
        rel = np.abs(yg - y64).reshape(m, K // G, G).max(axis=2) / np.where(g64 > 0, g64, 1.0)
        print("%s G=%d rows %d..: vs same-bf16-T oracle max %.2e of the group AbsMax; vs float64 T median %.2e, "
              "p99.9 %.2e, max %.2e" % (name, G, lo, (err / np.where(amax > 0, amax, 1.0)).max(), np.median(rel),
                                         np.quantile(rel, 0.999), rel.max()), flush=True)


@pytest.mark.parametrize("G,rows,blocks", [
    (16, None, None),   # the whole tiny tensor
    (32, None, None),
    (16, 77, 3),        # ragged: M not a multiple of 32, K = 48 (not a multiple of 256)
    (32, 45, 3),        # K = 96
    (32, 200, 5),       # several tiles, K = 160
])
def test_absmax_and_global_scale(G, rows, blocks):
    from mxfp4_activation_amd import ops

    _, tb = cases.transforms("tiny_mxfp4", G)
    xb = cases.x_full("tiny_mxfp4")
    if rows is not None:
        xb = np.ascontiguousarray(xb[:rows, : blocks * G])
        tb = np.ascontiguousarray(tb[:blocks])
    y = quant.transform_ref(xb, tb)
    X, T = _dev_bf16(xb), _dev_bf16(tb)
    amax = np.float32(ops.absmax_transformed(X, T).item())
    ref = quant.tensor_amax_ref(y)
    assert amax.view(np.uint32) == ref.view(np.uint32), (amax, ref)  # bit-exact
    if G == 16:
        g = np.float32(ops.nvfp4_global_scale(X, T).item())
        assert g.view(np.uint32) == quant.nvfp4_global_scale(ref).view(np.uint32)


@pytest.mark.parametrize("planted", [8199, 4111])
def test_absmax_three_tile_runs(planted):
    """G = 32 AbsMax on 8200 x 4096, which takes three-tile runs with a
    ragged last run (two tiles, the second partial).  One row is scaled by
    1000 so that it holds the tensor's maximum; the oracle computes that row
    alone.  Row 8199 sits in the last partial tile, row 4111 mid-tensor."""
    from mxfp4_activation_amd import ops

    _, tb = cases.transforms("llama8b_mxfp4")
    M, K = 8200, tb.shape[0] * 32
    rng = np.random.default_rng(planted)
    X = rng.standard_normal((M, K))  # light tails: no other row comes near the planted one
    X[planted] *= 1000.0
    xb = f64_to_bf16_bits(X)
    y = quant.transform_ref(xb[planted:planted + 1], tb)
    ref = quant.tensor_amax_ref(y)
    amax = np.float32(ops.absmax_transformed(_dev_bf16(xb), _dev_bf16(tb)).item())
    assert amax.view(np.uint32) == ref.view(np.uint32), (amax, ref)


def test_absmax_empty_is_zero():
    from mxfp4_activation_amd import ops

    _, tb = cases.transforms("tiny_mxfp4", 16)
    X = torch.empty((0, tb.shape[0] * 16), dtype=torch.bfloat16, device="cuda")
    out = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    ops.absmax_transformed(X, _dev_bf16(tb), out=out)
    assert float(out.item()) == 0.0


def test_global_scale_full_nvfp4_workload():
    """The AbsMax pre-pass over the whole 16384 x 4096 NVFP4 tensor equals the
    oracle's exact maximum bit for bit, so the device g equals the oracle's g."""
    from mxfp4_activation_amd import ops

    _, tb = cases.transforms("nvfp4")
    xb = cases.x_full("nvfp4")
    X, T = _dev_bf16(xb), _dev_bf16(tb)
    amax = np.float32(ops.absmax_transformed(X, T).item())
    g = np.float32(ops.nvfp4_global_scale(X, T).item())
    g_ref = cases.oracle_global_scale("nvfp4")
    ref = np.float32(cases.oracle_tensor_amax("nvfp4"))
    print("AbsMax %.9g, oracle %.9g, g %.9g, oracle g %.9g" % (amax, ref, g, g_ref))
    assert amax.view(np.uint32) == ref.view(np.uint32)
    assert g.view(np.uint32) == g_ref.view(np.uint32)


@pytest.mark.parametrize("G", [16, 32])
def test_absmax_near_ties(G):
    """Tokens whose transformed maxima differ by a few ulps or less, spread over
    workgroups: the pass must return the exact maximum, not a matrix-core
    value that rounds past it.  T = I + eps R keeps every output within
    about 2^-18 of its identity value, so many candidates tie within the
    accumulation bound."""
    from mxfp4_activation_amd import ops

    rng = np.random.default_rng(70 + G)
    M, C = 4100, 16
    K = C * G
    X = rng.uniform(-1, 1, (M, K))
    top = 1.75 * (1 + rng.integers(-3, 4, 40) * 2.0 ** -7)  # bf16 values within a few ulps of each other
    rows = rng.choice(M, 40, replace=False)
    X[rows, rng.integers(0, K, 40)] = top
    T = np.broadcast_to(np.eye(G), (C, G, G)) + rng.standard_normal((C, G, G)) * 2.0 ** -18
    xb, tb = f64_to_bf16_bits(X), f64_to_bf16_bits(T)
    ref = quant.tensor_amax_ref(quant.transform_ref(xb, tb))
    amax = np.float32(ops.absmax_transformed(_dev_bf16(xb), _dev_bf16(tb)).item())
    assert amax.view(np.uint32) == ref.view(np.uint32), (amax, ref)


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_zero_rows_need_no_recompute(fmt):
    """All-zero tokens (padding) take no exact recompute: an all-zero tensor
    counts none, and a tensor whose first half is zero counts exactly what
    its second half counts alone.  Outputs are zero codes and the minimum
    scale code, and the rest matches the oracle."""
    G = 16 if fmt == "nvfp4" else 32
    M, C = 512, 16
    K = C * G
    rng = np.random.default_rng(17)
    T = rng.standard_normal((C, G, G)) * 0.25
    tb = f64_to_bf16_bits(T)
    X = rng.standard_t(3, (M, K))
    X[: M // 2] = 0.0
    X[: M // 2: 7] = -0.0
    xb = f64_to_bf16_bits(X)
    g = np.float32(2.0 ** -4)
    c, s, n_zero = _run(fmt, np.zeros((M // 2, K), dtype=np.uint16), tb, g, n_exact=True)
    assert n_zero == 0
    assert not c.any() and not s.any()
    c, s, n_mixed = _run(fmt, xb, tb, g, n_exact=True)
    _, _, n_half = _run(fmt, np.ascontiguousarray(xb[M // 2:]), tb, g, n_exact=True)
    assert n_mixed == n_half, (n_mixed, n_half)
    parity.check(fmt, xb, tb, c, s, g)


def test_planted_e4m3_boundaries():
    """NVFP4 groups whose maximum sits on or right next to an E4M3 rounding
    midpoint of fp32(fp32(amax / 6) / g), across the normal and subnormal
    E4M3 range, with a static g.  T = I + eps R: with eps = 2^-19 the
    perturbation is below the accumulation bound, so the guard must send the
    group to the exact path; with eps = 2^-10 it moves the maximum off the
    midpoint by about 2^-9 relative, on either side."""
    G, C, M = 16, 16, 512
    K = C * G
    g = 2.0 ** -6
    rng = np.random.default_rng(23)
    # E4M3 values (codes 1..126) and the midpoints between neighbours
    e4 = np.array([(m / 8.0) * 2.0 ** -6 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 7)
                   for e in range(16) for m in range(8)])[1:127]
    mids = (e4[:-1] + e4[1:]) / 2
    X = rng.uniform(-0.3, 0.3, (M, K))
    targets = rng.choice(mids, (M, C)) * 6.0 * g
    X = X * (targets.repeat(G, axis=1) / 0.3)  # group values below the planted maximum
    pos = rng.integers(0, G, (M, C))
    sign = rng.choice([-1.0, 1.0], (M, C))
    for c in range(C):
        X[np.arange(M), c * G + pos[:, c]] = sign[:, c] * targets[:, c]
    xb = f64_to_bf16_bits(X)
    eps = np.where(np.arange(C) < C // 2, 2.0 ** -19, 2.0 ** -10)[:, None, None]
    T = np.broadcast_to(np.eye(G), (C, G, G)) + eps * rng.standard_normal((C, G, G))
    tb = f64_to_bf16_bits(T)
    c, s, n = _run("nvfp4", xb, tb, np.float32(g), n_exact=True)
    rep = parity.check("nvfp4", xb, tb, c, s, np.float32(g))
    print("planted E4M3 midpoints: %d exact groups of %d; %s" % (n, M * C, rep))
    assert n > 0


def test_guard_bytes_every_store_path():
    """Canary bytes before and after the code and scale buffers stay
    untouched, and two runs give identical bytes, on every store path:
    whole-tile runs of 1, 2 and 3 tiles, ragged token and channel edges, the
    G = 16 half-panel store (K/2 not a multiple of 16), and each format's
    scale width.  Stops at the first failure."""
    from mxfp4_activation_amd import ops

    shapes = [("mxfp4", 128, 256), ("mxfp4", 4096, 4096), ("mxfp4", 8200, 4096), ("mxfp4", 100, 96),
              ("mxfp4", 33, 4096 + 32), ("nvfp4", 64, 48), ("nvfp4", 40, 272), ("nvfp4", 4100, 4096),
              ("nvfp4", 256, 512), ("int4", 256, 512), ("int4", 100, 96), ("int4", 4136, 8192)]
    pad = 4096
    for fmt, M, K in shapes:
        print("case", fmt, M, K, flush=True)
        G = 16 if fmt == "nvfp4" else 32
        rng = np.random.default_rng(M + K)
        xb = f64_to_bf16_bits(rng.standard_t(3, (M, K)))
        tb = f64_to_bf16_bits(rng.standard_normal((K // G, G, G)) * 0.2)
        X, T = _dev_bf16(xb), _dev_bf16(tb)
        sbytes = 2 if fmt == "int4" else 1
        cbuf = torch.full((pad + M * K // 2 + pad,), 0xA5, dtype=torch.uint8, device="cuda")
        sbuf = torch.full((pad + M * (K // G) * sbytes + pad,), 0x5A, dtype=torch.uint8, device="cuda")
        codes = cbuf[pad:pad + M * K // 2].view(M, K // 2)
        scales = sbuf[pad:pad + M * (K // G) * sbytes]
        scales = (scales.view(torch.float16) if fmt == "int4" else scales).view(M, K // G)
        gs = torch.tensor([np.float32(2.0 ** -3)], dtype=torch.float32, device="cuda")
        ops.quant(fmt, X, T, global_scale=gs, codes=codes, scales=scales)
        first = (codes.clone(), scales.clone())
        ops.quant(fmt, X, T, global_scale=gs, codes=codes, scales=scales)
        torch.cuda.synchronize()
        assert torch.equal(first[0], codes) and torch.equal(first[1], scales), (fmt, M, K)
        cb, sb = cbuf.cpu().numpy(), sbuf.cpu().numpy()
        assert np.all(cb[:pad] == 0xA5) and np.all(cb[-pad:] == 0xA5), (fmt, M, K, "codes")
        assert np.all(sb[:pad] == 0x5A) and np.all(sb[-pad:] == 0x5A), (fmt, M, K, "scales")
        if M * K <= 1 << 20:
            s_np = scales.cpu().numpy()
            parity.check(fmt, xb, tb, codes.cpu().numpy(), s_np.view(np.uint16) if fmt == "int4" else s_np,
                         np.float32(2.0 ** -3))
