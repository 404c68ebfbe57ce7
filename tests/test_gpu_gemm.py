"""GPU parity of the MXFP4 GEMM (deep dive, section 3.4.6, Eq. 10).

The HIP kernel is called through the C ABI and compared with ``oracle.gemm``
on the same seeded operands.

Bar:
  * Exact cases.  Operands whose every partial sum is an fp32 number (small
    scale spread, bounded K) must match bit for bit, in fp32 and, after
    round-to-nearest-even, in bf16.  This pins nibble order, operand
    orientation, scale placement and the ragged edges, for both tile
    sizes (64 x 64 for grids that would leave CUs idle, else 128 x 128)
    and K from one 256-element step to several turns of the LDS ring.
  * General cases.  Each product of two E2M1 values and two E8M0 scales is
    exact in fp32, so any fp32 summation order of the K products errs by at
    most (K - 1) * 2^-24 * sum_k |a_k b_k|.  That is the tolerance, with
    2^-8 * |C| added for a bf16 output (half an ulp, doubled for the input's
    own fp32 error).
"""

import numpy as np
import pytest

from oracle import codecs, gemm, quant
from oracle import transform as tr
from synthetic import CONFIGS, f64_to_bf16_bits, gen_calibration, gen_weight, gen_x_rows
from tests import cases
from synthetic.gemm_operands import GEMM_TOKENS, MODEL_LAYERS, QWEN3_8B_LAYERS, gen_mx_operand

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()
    yield


def _dev(a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _gemm(ac, asc, bc, bsc, out_dtype):
    from mxfp4_activation_amd import ops

    C = ops.gemm_mxfp4(_dev(ac), _dev(asc), _dev(bc), _dev(bsc), out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype == torch.bfloat16:
        return C.view(torch.int16).cpu().numpy().view(np.uint16)
    return C.cpu().numpy()


def _bf16_value(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _check_tol(got, ref, absref, K, bf16):
    tol = (K - 1) * 2.0**-24 * absref
    if bf16:
        got = _bf16_value(got)
        tol = tol + 2.0**-8 * np.abs(ref)
    err = np.abs(got.astype(np.float64) - ref)
    ratio = np.max(err / np.maximum(tol, 1e-300)) if err.size else 0.0
    assert np.all(err <= tol), f"max err/tol {ratio:.3g}"
    return ratio


_EXACT = [
    (1, 1, 256, 126, 128),
    (7, 33, 256, 126, 128),
    (128, 128, 512, 126, 128),
    (129, 257, 1024, 126, 128),
    (200, 130, 768, 126, 128),
    (300, 64, 2048, 127, 127),
    (5, 300, 256, 127, 127),
    (1000, 3000, 256, 126, 128),  # 8 x 24 tiles of 128: the 128 x 128 kernel, ragged on both edges
    (1024, 3072, 512, 127, 127),  # the 128 x 128 kernel, whole tiles
    (1000, 3000, 2304, 127, 127),  # 128 x 128, 9 steps of 256: the ring wraps mid-way
    (77, 390, 4352, 127, 127),     # 64 x 64, 17 steps
    (64, 64, 2048, 126, 128),      # 64 x 64, 8 steps: one full turn of its ring
    (1000, 5096, 512, 126, 128),   # 320 tiles of 128: 4096 columns as 128 x 128, the last 1000 as 64 x 64
]


@pytest.mark.parametrize("M,N,K,slo,shi", _EXACT)
def test_exact_small_integer_products(M, N, K, slo, shi):
    ac, asc = gen_mx_operand(M, K, seed=100 + M, scale_lo=slo, scale_hi=shi)
    bc, bsc = gen_mx_operand(N, K, seed=200 + N, scale_lo=slo, scale_hi=shi)
    ref = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
    assert np.all(ref.astype(np.float32).astype(np.float64) == ref)  # the case is exact in fp32
    got = _gemm(ac, asc, bc, bsc, torch.float32)
    np.testing.assert_array_equal(got.astype(np.float64), ref)
    got16 = _gemm(ac, asc, bc, bsc, torch.bfloat16)
    np.testing.assert_array_equal(got16, codecs.f32_to_bf16_bits(ref.astype(np.float32)))


@pytest.mark.parametrize("M,N,K", [(256, 256, 4096), (77, 390, 1280), (513, 129, 256)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_wide_scale_range_within_fp32_bound(M, N, K, out):
    ac, asc = gen_mx_operand(M, K, seed=7 + K, scale_lo=105, scale_hi=140)
    bc, bsc = gen_mx_operand(N, K, seed=8 + K, scale_lo=110, scale_hi=135)
    ref = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
    absref = gemm.gemm_mxfp4_abs_ref(ac, asc, bc, bsc)
    dt = torch.float32 if out == "f32" else torch.bfloat16
    ratio = _check_tol(_gemm(ac, asc, bc, bsc, dt), ref, absref, K, out == "bf16")
    print(f"max err / bound = {ratio:.3g}")


@pytest.mark.parametrize("layer", ["q_proj", "k_proj", "gate_proj", "down_proj"])
def test_qwen3_8b_layer_shapes_whole(layer):
    """Every entry of C at the full layer shapes at 1024 tokens (the shapes
    the GEMM is timed on), against the oracle's float64 product."""
    N, K = QWEN3_8B_LAYERS[layer]
    M = GEMM_TOKENS
    ac, asc = gen_mx_operand(M, K, seed=31, scale_lo=112, scale_hi=124)
    bc, bsc = gen_mx_operand(N, K, seed=32, scale_lo=116, scale_hi=122)
    got = _gemm(ac, asc, bc, bsc, torch.float32)
    ref = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
    absref = gemm.gemm_mxfp4_abs_ref(ac, asc, bc, bsc)
    ratio = _check_tol(got, ref, absref, K, False)
    print(f"{layer}: {M} x {N} x {K}, every entry, max err / bound = {ratio:.3g}")


@pytest.mark.parametrize("model,layer,whole", [("qwen3-14b", "q_proj", True), ("qwen3-14b", "down_proj", True),
                                               ("llama3.1-70b", "gate_proj", False),
                                               ("llama3.1-70b", "down_proj", False)])
def test_other_model_layer_shapes(model, layer, whole):
    """The Qwen3-14B and Llama-3.1-70B shapes of the per-layer comparison at
    1024 tokens: every entry where the oracle's float64 product takes
    seconds, else a grid of sampled rows and columns with every tile edge."""
    N, K = MODEL_LAYERS[model][layer]
    M = GEMM_TOKENS
    ac, asc = gen_mx_operand(M, K, seed=41, scale_lo=112, scale_hi=124)
    bc, bsc = gen_mx_operand(N, K, seed=42, scale_lo=116, scale_hi=122)
    got = _gemm(ac, asc, bc, bsc, torch.float32)
    if whole:
        rows, cols = np.arange(M), np.arange(N)
    else:
        rng = np.random.default_rng(1)
        rows = np.unique(np.r_[0, 127, 128, M - 1, rng.choice(M, 24, replace=False)])
        cols = np.unique(np.r_[0, 127, 128, N - 1, rng.choice(N, 24, replace=False)])
    ref = gemm.gemm_mxfp4_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
    absref = gemm.gemm_mxfp4_abs_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
    ratio = _check_tol(got[np.ix_(rows, cols)], ref, absref, K, False)
    print(f"{model} {layer}: {M} x {N} x {K}, {ref.size} entries, max err / bound = {ratio:.3g}")


@pytest.mark.parametrize("layer", ["q_proj", "k_proj"])
def test_qwen3_8b_layer_shapes_8192_tokens_sampled(layer):
    """8192 tokens, whose grids run several waves of 128 x 128 workgroups; a
    grid of sampled rows and columns, including the first and last ones of
    every edge tile, is checked."""
    N, K = QWEN3_8B_LAYERS[layer]
    M = 8192
    ac, asc = gen_mx_operand(M, K, seed=31, scale_lo=112, scale_hi=124)
    bc, bsc = gen_mx_operand(N, K, seed=32, scale_lo=116, scale_hi=122)
    got = _gemm(ac, asc, bc, bsc, torch.float32)
    rng = np.random.default_rng(0)
    rows = np.unique(np.r_[0, 127, 128, M - 1, rng.choice(M, 20, replace=False)])
    cols = np.unique(np.r_[0, 127, 128, N - 1, rng.choice(N, 20, replace=False)])
    ref = gemm.gemm_mxfp4_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
    absref = gemm.gemm_mxfp4_abs_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
    _check_tol(got[np.ix_(rows, cols)], ref, absref, K, False)


def _packed_layout_ref(bc, bs):
    """The wush_gemm_pack_b layout as include/wush.h states it, in NumPy."""
    N, K = bc.shape[0], bc.shape[1] * 2
    Np, nk = (N + 127) // 128 * 128, K // 256
    rows = np.minimum(np.arange(Np), N - 1)
    c = bc[rows].reshape(Np // 128, 128, nk, 8, 16)       # tile, r, step, chunk, byte
    r = np.arange(128)
    pc = np.empty((Np // 128, nk, 128, 8, 16), np.uint8)  # tile, step, r, slot, byte
    for slot in range(8):
        chunk = slot ^ ((r // 2) % 8)
        # c[:, r, :, chunk, :] puts the (r, chunk) index first: [r][tile][step][byte]
        pc[:, :, :, slot, :] = c[:, r, :, chunk, :].transpose(1, 2, 0, 3)
    s = bs[rows].reshape(Np // 128, 128, nk, 8).transpose(0, 2, 1, 3)
    return pc.reshape(-1), np.ascontiguousarray(s).reshape(-1)


@pytest.mark.parametrize("N,K", [(128, 256), (200, 512), (1, 768)])
def test_pack_b_layout(N, K):
    """The packing kernel writes the layout the header documents (rows past
    N repeat row N - 1)."""
    from mxfp4_activation_amd import ops

    bc, bs = gen_mx_operand(N, K, seed=60 + N, scale_lo=110, scale_hi=140)
    pb = ops.gemm_pack_b(_dev(bc), _dev(bs))
    torch.cuda.synchronize()
    ec, es = _packed_layout_ref(bc, bs)
    np.testing.assert_array_equal(pb.codes.cpu().numpy(), ec)
    np.testing.assert_array_equal(pb.scales.cpu().numpy(), es)


@pytest.mark.parametrize("M,N,K", [(7, 33, 256), (64, 200, 512), (77, 390, 4352), (1000, 3000, 2304),
                                   (1000, 5096, 512), (1024, 1024, 4096), (1024, 4096, 4096)])
def test_packed_b_matches_unpacked(M, N, K):
    """The GEMM with packed weights, and with both operands packed, gives the
    unpacked GEMM's result bit for bit in fp32 and bf16: 64 x 64 tiles that
    are second halves of packed 128-row tiles, ragged edges, the split last
    wave, and whole layer shapes."""
    from mxfp4_activation_amd import ops

    print("packed", M, N, K, flush=True)
    ac, asc = gen_mx_operand(M, K, seed=70 + M, scale_lo=105, scale_hi=140)
    bc, bsc = gen_mx_operand(N, K, seed=71 + N, scale_lo=110, scale_hi=135)
    a, a_s, b, b_s = _dev(ac), _dev(asc), _dev(bc), _dev(bsc)
    c1 = ops.gemm_mxfp4(a, a_s, b, b_s, out_dtype=torch.float32)
    pb = ops.gemm_pack_b(b, b_s)
    c2 = ops.gemm_mxfp4_packed((a, a_s), pb, out_dtype=torch.float32)
    c3 = ops.gemm_mxfp4_packed((a, a_s), pb, out_dtype=torch.bfloat16)
    # Both operands packed (A re-laid here by the weight packer, which writes
    # the same layout the packed quantizer does).
    pa = ops.gemm_pack_b(a, a_s)
    c5 = ops.gemm_mxfp4_packed(pa, pb, out_dtype=torch.float32)
    c6 = ops.gemm_mxfp4_packed(pa, pb, out_dtype=torch.bfloat16)
    c4 = ops.gemm_mxfp4(a, a_s, b, b_s, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int32), c2.view(torch.int32))
    assert torch.equal(c3.view(torch.int16), c4.view(torch.int16))
    assert torch.equal(c1.view(torch.int32), c5.view(torch.int32))
    assert torch.equal(c4.view(torch.int16), c6.view(torch.int16))
    if M * N * K <= 1 << 31:
        ref = gemm.gemm_mxfp4_ref(ac, asc, bc, bsc)
        absref = gemm.gemm_mxfp4_abs_ref(ac, asc, bc, bsc)
        _check_tol(c2.cpu().numpy(), ref, absref, K, False)


@pytest.mark.parametrize("M,K", [(128, 256), (77, 512), (1000, 2304), (1024, 4096), (4096, 4096)])
def test_quant_mxfp4_packed_layout(M, K):
    """wush_quant_mxfp4_packed writes the row-major quantizer's codes and
    scales, bit for bit, in the packed layout (rows past M, which it does
    not write, are left out of the comparison), and the GEMM on two packed
    operands gives the row-major GEMM's result."""
    from mxfp4_activation_amd import ops

    print("packed quant", M, K, flush=True)
    _, tb = cases.transforms("tiny_mxfp4")
    reps = K // 256
    T = _dev(np.tile(tb, (reps, 1, 1)).view(np.int16)).view(torch.bfloat16)
    rng = np.random.default_rng(M + K)
    X = _dev(f64_to_bf16_bits(rng.standard_t(3, size=(M, K))).view(np.int16)).view(torch.bfloat16)
    codes, scales = ops.quant_mxfp4(X, T)
    pq = ops.quant_mxfp4_packed(X, T)
    torch.cuda.synchronize()
    c, sc = codes.cpu().numpy(), scales.cpu().numpy()
    Mp = (M + 127) // 128 * 128
    pad_c = np.zeros((Mp, K // 2), np.uint8)
    pad_s = np.zeros((Mp, K // 32), np.uint8)
    pad_c[:M], pad_s[:M] = c, sc
    ec, es = _packed_layout_ref(pad_c, pad_s)
    gc = pq.codes.cpu().numpy().reshape(Mp // 128, K // 256, 128, 128).copy()
    gs = pq.scales.cpu().numpy().reshape(Mp // 128, K // 256, 128, 8).copy()
    ec = ec.reshape(gc.shape).copy()
    es = es.reshape(gs.shape).copy()
    # Byte block [t][step][r] is row r's 128 code bytes (chunks permuted
    # within the row), and [t][step][r] of the scales its 8 scale bytes.
    # Rows past M: zero on both sides before comparing.
    for t in range(Mp // 128):
        dead = t * 128 + np.arange(128) >= M
        gc[t][:, dead] = 0
        ec[t][:, dead] = 0
        gs[t][:, dead] = 0
        es[t][:, dead] = 0
    np.testing.assert_array_equal(gc, ec)
    np.testing.assert_array_equal(gs, es)
    if K >= 256 and M >= 64:
        N = 384
        bc, bsc = gen_mx_operand(N, K, seed=5, scale_lo=110, scale_hi=130)
        pb = ops.gemm_pack_b(_dev(bc), _dev(bsc))
        c_row = ops.gemm_mxfp4_packed((codes, scales), pb, out_dtype=torch.float32)
        c_pk = ops.gemm_mxfp4_packed(pq, pb, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(c_row.view(torch.int32), c_pk.view(torch.int32))


@pytest.mark.parametrize("M,N,K", [(64, 64, 2048), (64, 64, 4096), (2048, 2048, 2048), (1024, 4096, 4096)])
def test_fresh_operands_every_call(M, N, K):
    """Several calls in a row, each with new A operands.  A load that has not
    landed when its stage is read would leave the previous call's data in
    LDS; with identical inputs on every call that stale data would be right
    and hide the error, so every call here gets different codes and
    scales."""
    bc, bsc = gen_mx_operand(N, K, seed=12, scale_lo=124, scale_hi=130)
    rows = np.unique(np.r_[np.arange(0, M, max(1, M // 48)), M - 1])
    cols = np.unique(np.r_[np.arange(0, N, max(1, N // 48)), N - 1])
    for call in range(5):
        ac, asc = gen_mx_operand(M, K, seed=300 + call, scale_lo=124, scale_hi=130)
        got = _gemm(ac, asc, bc, bsc, torch.float32)
        ref = gemm.gemm_mxfp4_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
        absref = gemm.gemm_mxfp4_abs_ref(ac[rows], asc[rows], bc[cols], bsc[cols])
        _check_tol(got[np.ix_(rows, cols)], ref, absref, K, False)


def test_zero_rows_is_a_no_op():
    from mxfp4_activation_amd import ops

    ac, asc = gen_mx_operand(0, 256, seed=1)
    bc, bsc = gen_mx_operand(8, 256, seed=2)
    C = ops.gemm_mxfp4(_dev(ac), _dev(asc), _dev(bc), _dev(bsc), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert C.shape == (0, 8)


def test_quantized_layer_forward():
    """Quantize activations with T_wush and weights with T_xvsh on the GPU,
    multiply on the GPU, and compare with the oracle's quantize + multiply.

    Where the GPU codes equal the oracle's (all but tie cases), the GEMM
    output is held to the fp32 bound; the forward itself must recover
    x^T w as closely as the oracle's does."""
    from mxfp4_activation_amd import ops

    wl = CONFIGS["tiny_mxfp4"]
    x_bits = gen_x_rows(wl, 0, wl.M)
    W = gen_weight(wl)
    w_bits = f64_to_bf16_bits(W)
    Tw, Tx = tr.build_transforms(W, gen_calibration(wl), wl.G)
    tw_bits, tx_bits = tr.transforms_to_bf16_bits(Tw), tr.transforms_to_bf16_bits(Tx)

    def dev_bf16(b):
        return _dev(b.view(np.int16)).view(torch.bfloat16)

    xc_g, xs_g = ops.quant("mxfp4", dev_bf16(x_bits), dev_bf16(tw_bits))
    wc_g, ws_g = ops.quant("mxfp4", dev_bf16(w_bits), dev_bf16(tx_bits))
    C_g = ops.gemm_mxfp4(xc_g, xs_g, wc_g, ws_g, out_dtype=torch.float32)
    torch.cuda.synchronize()
    C_g = C_g.cpu().numpy().astype(np.float64)

    xc, xs = quant.run_path("mxfp4", x_bits, tw_bits)
    wc, ws = quant.run_path("mxfp4", w_bits, tx_bits)
    same_rows = np.all(xc_g.cpu().numpy() == xc, axis=1) & np.all(xs_g.cpu().numpy() == xs, axis=1)
    same_cols = np.all(wc_g.cpu().numpy() == wc, axis=1) & np.all(ws_g.cpu().numpy() == ws, axis=1)
    assert same_rows.mean() > 0.9 and same_cols.mean() > 0.9
    ref = gemm.gemm_mxfp4_ref(xc, xs, wc, ws)
    absref = gemm.gemm_mxfp4_abs_ref(xc, xs, wc, ws)
    sel = np.ix_(same_rows, same_cols)
    _check_tol(C_g[sel], ref[sel], absref[sel], wl.K, False)

    x = _bf16_value(x_bits)
    exact = x @ _bf16_value(w_bits).T
    rel_gpu = np.linalg.norm(C_g - exact) / np.linalg.norm(exact)
    rel_ref = np.linalg.norm(ref - exact) / np.linalg.norm(exact)
    assert rel_gpu <= rel_ref * 1.01 + 1e-6, (rel_gpu, rel_ref)
