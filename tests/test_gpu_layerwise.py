"""GPU parity of the offline weight side and the layerwise loss (Eq. 5).

* wush_dequant against the oracle's decoders on seeded random codes and
  scales: bit-exact for MXFP4 (including scales that make the values
  subnormal) and INT4; for NVFP4 the device forms fp32(E4M3 * g) and then
  one more fp32 product, so each value is within 2^-22 of the exact one.
* The layerwise loss computed by the kernels (transform + quantize both
  operands, dequantize, fp32 products) against oracle.loss, for the four
  transform pairs and three formats, on the same transform bytes.  Codes
  may differ from the oracle's at accumulation ties (at most 1e-4 of
  them) and the products are fp32, so the bar is a relative 2e-3.
* The Table 1 orderings on a larger synthetic layer, computed on the GPU.
"""

import numpy as np
import pytest

from oracle import loss, quant
from oracle import transform as tr
from synthetic import f64_to_bf16_bits
from synthetic.layers import gen_linear_layer

from . import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()
    yield


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _dev_bf16(bits):
    return _dev(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


def _random_codes(rng, M, K):
    return rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)


@pytest.mark.parametrize("M,K", [(1, 32), (37, 96), (256, 4096)])
def test_dequant_mxfp4_exact(M, K):
    from mxfp4_activation_amd import ops

    rng = np.random.default_rng(M + K)
    codes = _random_codes(rng, M, K)
    # Up to 252: the quantizer's largest code (fp32 y stays below 2^128, so
    # e = floor(log2 amax) - 2 <= 125); 253 and 254 would overflow fp32.
    scales = rng.integers(0, 253, size=(M, K // 32), dtype=np.uint8)
    scales[0, 0] = 0  # 2^-127: subnormal fp32 values
    got = ops.dequant("mxfp4", _dev(codes), _dev(scales)).cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, quant.dequant_mxfp4(codes, scales, 32))


@pytest.mark.parametrize("M,K", [(3, 32), (64, 1024)])
def test_dequant_int4_exact(M, K):
    from mxfp4_activation_amd import ops

    rng = np.random.default_rng(7 * M + K)
    codes = _random_codes(rng, M, K)
    s = np.abs(rng.standard_normal((M, K // 32))).astype(np.float16)
    s[0, 0] = 0
    got = ops.dequant("int4", _dev(codes), _dev(s)).cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(got, quant.dequant_int4(codes, s.view(np.uint16), 32))


@pytest.mark.parametrize("M,K", [(5, 16), (128, 2048)])
def test_dequant_nvfp4(M, K):
    from mxfp4_activation_amd import ops

    rng = np.random.default_rng(11 * M + K)
    codes = _random_codes(rng, M, K)
    scales = rng.integers(0, 0x7F, size=(M, K // 16), dtype=np.uint8)  # non-negative finite E4M3
    g = np.float32(0.0123)
    got = ops.dequant("nvfp4", _dev(codes), _dev(scales),
                      torch.tensor([g], dtype=torch.float32, device="cuda")).cpu().numpy().astype(np.float64)
    ref = quant.dequant_nvfp4(codes, scales, g, 16)
    np.testing.assert_allclose(got, ref, rtol=2.0**-22, atol=0)


def _pairs(W, Xc, G):
    C = W.shape[1] // G
    Tw, Tx = tr.build_transforms(W, Xc, G)
    Tws, Txs = tr.build_transforms(W, Xc, G, H=np.eye(G))
    H = np.broadcast_to(tr.hadamard(G), (C, G, G)).copy()
    eye = np.broadcast_to(np.eye(G), (C, G, G)).copy()
    raw = {"I": (eye, eye), "H": (H, H), "WUS": (Tws, Txs), "WUSH": (Tw, Tx)}
    return {k: (tr.transforms_to_bf16_bits(a), tr.transforms_to_bf16_bits(b)) for k, (a, b) in raw.items()}


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_layerwise_loss_matches_oracle(fmt):
    from mxfp4_activation_amd import layerwise

    G = 16 if fmt == "nvfp4" else 32
    W, Xc, Xe = gen_linear_layer(256, 64, 512, 128, seed=21, n_outlier=3)
    xb, wb = f64_to_bf16_bits(Xe), f64_to_bf16_bits(W)
    for name, (ta, tw) in _pairs(W, Xc, G).items():
        ref = loss.layerwise_loss_ref(fmt, xb, wb, ta, tw)
        got = layerwise.layerwise_loss(fmt, _dev_bf16(xb), _dev_bf16(wb), _dev_bf16(ta), _dev_bf16(tw))
        assert got == pytest.approx(ref, rel=2e-3), (name, got, ref)


def test_weight_side_codes_match_oracle():
    """W~ = q(T_xvsh W): the fused kernel on the weight rows gives the oracle's codes and scales."""
    from mxfp4_activation_amd import layerwise

    W, Xc, _ = gen_linear_layer(512, 96, 512, 1, seed=4, n_outlier=2)
    _, tw = _pairs(W, Xc, 32)["WUSH"]
    wb = f64_to_bf16_bits(W)
    c, s, _ = layerwise.quantize("mxfp4", _dev_bf16(wb), _dev_bf16(tw))
    torch.cuda.synchronize()
    parity.check("mxfp4", wb, tw, c.cpu().numpy(), s.cpu().numpy())


def test_table1_orderings_on_gpu():
    from mxfp4_activation_amd import layerwise

    W, Xc, Xe = gen_linear_layer(2048, 512, 2048, 1024, seed=33, n_outlier=20)
    X = _dev_bf16(f64_to_bf16_bits(Xe))
    Wd = _dev_bf16(f64_to_bf16_bits(W))
    Xcd = _dev_bf16(f64_to_bf16_bits(Xc))
    res = {}
    for fmt in ("mxfp4", "nvfp4", "int4"):
        G = 16 if fmt == "nvfp4" else 32
        banks = layerwise.transform_pairs(Wd, Xcd, G)
        res[fmt] = {k: layerwise.layerwise_loss(fmt, X, Wd, a, b) for k, (a, b) in banks.items()}
    print(res)
    for fmt in ("mxfp4", "int4"):
        L = res[fmt]
        assert L["WUSH"] < L["H"] < L["I"], (fmt, L)
    L = res["nvfp4"]
    assert L["H"] > L["I"] and L["WUSH"] < 0.5 * L["I"] and L["WUS"] < 0.5 * L["I"], L
