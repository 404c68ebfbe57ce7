"""GPU parity of GPTQ-WUSH (Algorithm 1) against oracle.gptq.

* The intra-block kernel (wush_gptq_block) against oracle.gptq.gptq_block
  on the same float64 inputs: both run the same float64 operations in the
  same order (no contraction), so codes, scales and dequantized values must
  match bit for bit.  R = I must give round-to-nearest.
* The whole algorithm in the library (wush_gptq_wush: blocked Cholesky,
  float64 GEMMs, the block's SVD through its Gram matrix, the intra-block
  step) against the oracle (LAPACK): the activation transforms within 1e-8
  of the block's largest entry, at most 1e-3 of the weight codes one level
  apart (a code can flip where the two SVD routes put a value within
  rounding of a midpoint), and the calibration error of the quantized layer
  within 1%.  Its Cholesky factor against LAPACK's on the same damped
  Hessian, and the upper triangle exactly zero.
* Eq. 10 end to end on the device: activations through the fused kernel
  with the GPTQ-WUSH transforms, weights from GPTQ-WUSH, the MXFP4 GEMM;
  GPTQ gives a lower output error than round-to-nearest in the same
  algorithm.
"""

import numpy as np
import pytest

from oracle import codecs, gptq
from synthetic import f64_to_bf16_bits
from synthetic.layers import gen_linear_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()
    yield


def _run_kernel(fmt, Wbar, R):
    from mxfp4_activation_amd import _lib
    from mxfp4_activation_amd.ops import _stream

    G, d_out = Wbar.shape
    Wd = torch.from_numpy(np.ascontiguousarray(Wbar)).cuda()
    Rd = torch.from_numpy(np.ascontiguousarray(R)).cuda()
    Q = torch.empty((G, d_out), dtype=torch.float64, device="cuda")
    codes = torch.empty((d_out, G // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((d_out, 1), dtype=torch.float16 if fmt == "int4" else torch.uint8, device="cuda")
    lib = _lib.load()
    _lib.check(lib.wush_gptq_block(_lib.FMT[fmt], Wd.data_ptr(), Rd.data_ptr(), G, d_out, Q.data_ptr(),
                                   codes.data_ptr(), G // 2, scales.data_ptr(), 1, _stream()), "wush_gptq_block")
    torch.cuda.synchronize()
    s = scales.cpu().numpy()[:, 0]
    return Q.cpu().numpy(), codes.cpu().numpy(), (s.view(np.uint16) if fmt == "int4" else s)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
@pytest.mark.parametrize("G,d_out", [(32, 300), (16, 77)])
def test_gptq_block_kernel_bit_exact(fmt, G, d_out):
    rng = np.random.default_rng(G + d_out)
    A = rng.standard_normal((G, 2 * G))
    Hb = A @ A.T / (2 * G) + 0.05 * np.eye(G)
    R = np.linalg.cholesky(np.linalg.inv(Hb)).T.copy()
    Wbar = rng.standard_normal((G, d_out)) * np.exp(rng.uniform(-4, 4, size=(1, d_out)))
    Wbar[:, 0] = 0.0  # an all-zero group
    Q, codes, scales = _run_kernel(fmt, Wbar, R)
    rQ, rc, rs = gptq.gptq_block(Wbar, Hb, fmt)
    np.testing.assert_array_equal(scales, rs)
    np.testing.assert_array_equal(codes, codecs.pack_nibbles(rc.T))
    np.testing.assert_array_equal(Q, rQ)
    # R = I is round-to-nearest.
    Q2, c2, _ = _run_kernel(fmt, Wbar, np.eye(G))
    rQ2, rc2, _ = gptq.rtn_block(Wbar, fmt)
    np.testing.assert_array_equal(Q2, rQ2)
    np.testing.assert_array_equal(c2, codecs.pack_nibbles(rc2.T))


@pytest.mark.parametrize("fmt,G,mode", [("mxfp4", 32, True), ("int4", 32, True), ("mxfp4", 16, False),
                                        ("int4", 16, True), ("mxfp4", 32, False)])
def test_gptq_wush_matches_oracle(fmt, G, mode):
    from mxfp4_activation_amd import gptq as pg

    print("case", fmt, G, mode, flush=True)
    W, Xc, _ = gen_linear_layer(256, 96, 1024, 1, seed=12, n_outlier=3)
    ref = gptq.gptq_wush_ref(W, Xc, G, fmt, gptq=mode)
    got = pg.gptq_wush(torch.from_numpy(W).cuda(), torch.from_numpy(Xc).cuda(), G, fmt, gptq=mode)
    torch.cuda.synchronize()
    tx = got.T_x.cpu().numpy()
    scale = np.abs(ref.T_x).max(axis=(1, 2), keepdims=True)
    assert (np.abs(tx - ref.T_x) / scale).max() < 1e-8
    lv = lambda c: (codecs.int4_decode if fmt == "int4" else codecs.e2m1_level_index)(codecs.unpack_nibbles(c))
    d = np.abs(lv(got.codes.cpu().numpy()).astype(int) - lv(ref.codes).astype(int))
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, ((d > 0).mean(), d.max())
    e_ref = np.mean((gptq.layer_output(ref, Xc, lambda v: v) - Xc @ W.T) ** 2)
    res = gptq.GptqWush(tx, got.Wq.cpu().numpy(), None, None)
    e_got = np.mean((gptq.layer_output(res, Xc, lambda v: v) - Xc @ W.T) ** 2)
    assert e_got == pytest.approx(e_ref, rel=1e-2)


@pytest.mark.parametrize("fmt,G,d_in,d_out", [("mxfp4", 32, 128, 600), ("int4", 16, 96, 600),
                                               ("int4", 32, 64, 65600)])
def test_gptq_wush_matches_oracle_many_channels(fmt, G, d_in, d_out):
    """Output channels spread over several workgroups per block (256 each,
    the last one ragged), and past 256 workgroups (65600 channels: each
    workgroup loops over several 256-channel groups).  Every workgroup
    derives the block's transforms itself; all must agree with the oracle.
    Same bar as the small case, and the scales equal."""
    from mxfp4_activation_amd import gptq as pg

    print("case", fmt, G, d_in, d_out, flush=True)
    W, Xc, _ = gen_linear_layer(d_in, d_out, 1024 if d_out < 4096 else 512, 1, seed=15 + d_out, n_outlier=2)
    ref = gptq.gptq_wush_ref(W, Xc, G, fmt, gptq=True)
    got = pg.gptq_wush(torch.from_numpy(W).cuda(), torch.from_numpy(Xc).cuda(), G, fmt, gptq=True)
    torch.cuda.synchronize()
    tx = got.T_x.cpu().numpy()
    scale = np.abs(ref.T_x).max(axis=(1, 2), keepdims=True)
    assert (np.abs(tx - ref.T_x) / scale).max() < 1e-8
    lv = lambda c: (codecs.int4_decode if fmt == "int4" else codecs.e2m1_level_index)(codecs.unpack_nibbles(c))
    d = np.abs(lv(got.codes.cpu().numpy()).astype(int) - lv(ref.codes).astype(int))
    print("weight codes one level apart: %d of %d" % ((d > 0).sum(), d.size), flush=True)
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3, ((d > 0).mean(), d.max())
    sg = got.scales.cpu().numpy()
    sr = ref.scales
    if fmt == "int4":
        sg, sr = sg.view(np.uint16), np.asarray(sr).view(np.uint16)
    mism = (sg != sr).mean()
    print("scale mismatches: %.3g" % mism, flush=True)
    assert mism <= 1e-3


def test_gptq_wush_matches_oracle_wide():
    """A 1024-wide layer: 32 blocks, a 16 x 16 grid of 64-wide tiles in the
    Hessian GEMM and the blocked Cholesky, updates of up to 992 columns.
    Same bar as the small case."""
    from mxfp4_activation_amd import gptq as pg

    W, Xc, _ = gen_linear_layer(1024, 384, 2048, 1, seed=14, n_outlier=10)
    ref = gptq.gptq_wush_ref(W, Xc, 32, "mxfp4", gptq=True)
    got = pg.gptq_wush(torch.from_numpy(W).cuda(), torch.from_numpy(Xc).cuda(), 32, "mxfp4", gptq=True)
    torch.cuda.synchronize()
    tx = got.T_x.cpu().numpy()
    scale = np.abs(ref.T_x).max(axis=(1, 2), keepdims=True)
    err = (np.abs(tx - ref.T_x) / scale).max()
    print("T_x max relative difference %.3g" % err, flush=True)
    assert err < 1e-8
    lv = lambda c: codecs.e2m1_level_index(codecs.unpack_nibbles(c))
    d = np.abs(lv(got.codes.cpu().numpy()).astype(int) - lv(ref.codes).astype(int))
    print("weight codes one level apart: %d of %d" % ((d > 0).sum(), d.size), flush=True)
    assert d.max() <= 1 and (d > 0).mean() <= 1e-3
    np.testing.assert_array_equal(got.scales.cpu().numpy(), ref.scales)


def test_gptq_wush_cholesky_factor():
    """The library's blocked Cholesky of the damped Hessian against LAPACK's
    on the same float64 Hessian (a library routine on the definition, not
    the oracle): lower factors within 1e-10 of the largest entry, zero above
    the diagonal, over 13 panels and GEMM tiles cut by the matrix edge."""
    from mxfp4_activation_amd import gptq as pg

    W, Xc, _ = gen_linear_layer(208, 40, 700, 1, seed=21, n_outlier=2)
    got = pg.gptq_wush(torch.from_numpy(W).cuda(), torch.from_numpy(Xc).cuda(), 16, "mxfp4", gptq=True)
    torch.cuda.synchronize()
    Hx = Xc.T @ Xc / Xc.shape[0]
    Hx = Hx + gptq.DEFAULT_GPTQ_DAMP * np.mean(np.diag(Hx)) * np.eye(Hx.shape[0])
    Lref = np.linalg.cholesky(Hx)
    Xp = got.Xp.cpu().numpy()
    assert np.all(np.triu(Xp, 1) == 0.0)
    assert np.abs(Xp - Lref).max() <= 1e-10 * np.abs(Lref).max()
    # The last block's target is W X' itself (no block above it).
    Y = got.Y.cpu().numpy()
    np.testing.assert_allclose(Y[:, -16:], (W @ Lref)[:, -16:], rtol=0, atol=1e-10 * np.abs(W @ Lref).max())


def test_eq10_forward_with_gptq_weights():
    from mxfp4_activation_amd import gptq as pg
    from mxfp4_activation_amd import ops, transforms

    W, Xc, Xe = gen_linear_layer(512, 256, 2048, 512, seed=13, n_outlier=5)
    Wd, Xcd = torch.from_numpy(W).cuda(), torch.from_numpy(Xc).cuda()
    Xb = torch.from_numpy(f64_to_bf16_bits(Xe).view(np.int16)).cuda().view(torch.bfloat16)
    exact = torch.from_numpy(Xe @ W.T).cuda()
    err = {}
    for mode in (True, False):
        r = pg.gptq_wush(Wd, Xcd, 32, "mxfp4", gptq=mode)
        bank = transforms.to_kernel_layout(r.T_x)
        xc, xs = ops.quant("mxfp4", Xb, bank)
        out = ops.gemm_mxfp4(xc, xs, r.codes, r.scales, out_dtype=torch.float32)
        err[mode] = float(((out.double() - exact) ** 2).mean() / (exact ** 2).mean())
    print(err)
    assert err[True] < err[False], err
