"""C-ABI checks that need no GPU.  The library loads, it exports every
symbol include/wush.h declares, and argument validation rejects bad calls
before any HIP call."""

import ctypes
import os
import re

import pytest

import mxfp4_activation_amd as wush
from mxfp4_activation_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    src = open(os.path.join(ROOT, "include", "wush.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wush_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    lib = wush.load()
    decl = _declared_symbols()
    assert len(decl) >= 10
    for name in decl:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, "binding lacks " + name
    assert set(_lib.SIGNATURES) == set(decl)
    assert lib.wush_abi_version() == _lib.ABI_VERSION == 2


def test_status_strings():
    lib = wush.load()
    for s in range(5):
        assert lib.wush_status_string(s)


A = 1 << 20  # a 16-byte-aligned fake device address; validation never dereferences it


@pytest.mark.parametrize("fmt", [0, 1, 2])
def test_validation_rejects_bad_arguments(fmt):
    lib = wush.load()
    G = 16 if fmt == 1 else 32
    gs = 3 << 20
    q = lambda X, T, M, K, c, s, g=gs: lib.wush_quant(fmt, X, T, M, K, g, c, s, None, None)
    assert q(A, A * 2, 0, 4 * G, None, None) == _lib.WUSH_OK  # empty batch: no-op
    assert q(A, A * 2, -1, 4 * G, A * 3, A * 4) == _lib.WUSH_EINVAL
    assert q(A, A * 2, 8, G + 1, A * 3, A * 4) == _lib.WUSH_EINVAL
    assert q(A, A * 2, 8, 0, A * 3, A * 4) == _lib.WUSH_EINVAL
    assert q(None, A * 2, 8, G, A * 3, A * 4) == _lib.WUSH_EINVAL
    assert q(A, A * 2, 8, G, None, A * 4) == _lib.WUSH_EINVAL
    assert q(A + 2, A * 2, 8, G, A * 3, A * 4) == _lib.WUSH_EALIGN
    assert q(A, A * 2 + 8, 8, G, A * 3, A * 4) == _lib.WUSH_EALIGN
    assert q(A, A * 2, 8, G, A * 3 + 4, A * 4) == _lib.WUSH_EALIGN
    assert q(A, A * 2, 8, G, A * 3 + 8, A * 4) == _lib.WUSH_EALIGN  # codes need 16 bytes
    assert q(A, A * 2, 8, G, A * 3, A * 4 + 4) == _lib.WUSH_EALIGN  # scales need at least 8
    if fmt != 0:
        assert q(A, A * 2, 8, G, A * 3, A * 4 + 8) == _lib.WUSH_EALIGN  # NVFP4 and INT4 scales need 16
    # codes overlapping X
    assert q(A, A * 8, 8, 4 * G, A + 64, A * 16) == _lib.WUSH_EINVAL
    if fmt == 1:
        assert q(A, A * 2, 8, G, A * 3, A * 4, None) == _lib.WUSH_EINVAL
    if fmt == 2:
        assert q(A, A * 2, 8, G, A * 3, A * 4 + 1) == _lib.WUSH_EALIGN
    assert lib.wush_last_error()


def test_unknown_format_and_G():
    lib = wush.load()
    assert lib.wush_quant(7, A, A, 8, 32, None, A, A, None, None) == _lib.WUSH_EUNSUPPORTED
    assert lib.wush_transform_f32(A, A * 2, 8, 64, 8, A * 4, None) == _lib.WUSH_EUNSUPPORTED
    assert lib.wush_e2m1_encode(A, -1, A * 2, None) == _lib.WUSH_EINVAL
    assert lib.wush_e2m1_encode(A, 0, None, None) == _lib.WUSH_OK


def test_binding_raises_with_detail():
    lib = wush.load()
    st = lib.wush_quant_mxfp4(A, A, 8, 33, A * 2, A * 3, None)
    with pytest.raises(_lib.WushError, match="multiple of 32"):
        _lib.check(st, "wush_quant_mxfp4")


def test_gemm_validation_rejects_bad_arguments():
    lib = wush.load()
    B = A * 64  # far apart: no overlaps unless a test places one
    g = lambda ac, as_, bc, bs, M, N, K, C, t=0: lib.wush_gemm_mxfp4(ac, as_, bc, bs, M, N, K, C, t, None)
    args = (A, A * 2, A * 3, A * 4)
    assert g(*args, 0, 16, 256, B) == _lib.WUSH_OK  # M = 0: no-op
    assert g(*args, 16, 0, 256, B) == _lib.WUSH_OK
    assert g(*args, -1, 16, 256, B) == _lib.WUSH_EINVAL
    assert g(*args, 16, 16, 128, B) == _lib.WUSH_EINVAL  # K not a multiple of 256
    assert g(*args, 16, 16, 0, B) == _lib.WUSH_EINVAL
    assert g(*args, 16, 16, 256, B, 2) == _lib.WUSH_EINVAL  # unknown output type
    assert g(None, A * 2, A * 3, A * 4, 16, 16, 256, B) == _lib.WUSH_EINVAL
    assert g(*args, 16, 16, 256, None) == _lib.WUSH_EINVAL
    assert g(A + 8, A * 2, A * 3, A * 4, 16, 16, 256, B) == _lib.WUSH_EALIGN
    assert g(A, A * 2 + 4, A * 3, A * 4, 16, 16, 256, B) == _lib.WUSH_EALIGN
    assert g(*args, 16, 16, 256, B + 2) == _lib.WUSH_EALIGN
    assert g(*args, 16, 16, 256, A * 3 + 64) == _lib.WUSH_EINVAL  # C overlaps b_codes
    assert g(*args, 16, 16, 384, B) == _lib.WUSH_EINVAL
    assert b"multiple of 256" in lib.wush_last_error()


def test_gemm_packed_validation_rejects_bad_arguments():
    lib = wush.load()
    B = A * 64
    g = lambda ac, as_, bc, bs, M, N, K, C, t=0, ap=0: lib.wush_gemm_mxfp4_packed(ac, as_, ap, bc, bs, M, N, K, C, t,
                                                                               None)
    args = (A, A * 2, A * 3, A * 4)
    assert g(*args, 0, 16, 256, B) == _lib.WUSH_OK  # M = 0: no-op
    assert g(*args, -1, 16, 256, B) == _lib.WUSH_EINVAL
    assert g(*args, 16, 16, 128, B) == _lib.WUSH_EINVAL  # K not a multiple of 256
    assert g(*args, 16, 16, 256, B, 2) == _lib.WUSH_EINVAL
    assert g(A, A * 2, None, A * 4, 16, 16, 256, B) == _lib.WUSH_EINVAL
    assert g(A, A * 2, A * 3 + 8, A * 4, 16, 16, 256, B) == _lib.WUSH_EALIGN
    assert g(A, A * 2, A * 3, A * 4 + 4, 16, 16, 256, B) == _lib.WUSH_EALIGN
    # Packed B covers N rounded up to 128 rows (16 KB of codes at K = 256):
    # a C placed past N's 2 KB but inside the padding overlaps it.
    assert g(*args, 16, 16, 256, A * 3 + 4096) == _lib.WUSH_EINVAL
    assert b"overlaps" in lib.wush_last_error()
    assert g(*args, 16, 16, 256, B, 0, 2) == _lib.WUSH_EINVAL  # a_packed is 0 or 1
    # Packed A covers M rounded up to 128 rows as well.
    assert g(*args, 16, 16, 256, A + 4096, 0, 1) == _lib.WUSH_EINVAL


def test_quant_mxfp4_packed_validation_rejects_bad_arguments():
    lib = wush.load()
    q = lambda X, T, M, K, c, s: lib.wush_quant_mxfp4_packed(X, T, M, K, c, s, None)
    B = A * 64
    assert q(A, A * 2, 0, 256, B, B * 2) == _lib.WUSH_OK  # M = 0: no-op
    assert q(A, A * 2, 4, 320, B, B * 2) == _lib.WUSH_EINVAL  # K not a multiple of 256
    assert b"multiple of 256" in lib.wush_last_error()
    assert q(A, A * 2, 4, 256, None, B * 2) == _lib.WUSH_EINVAL
    assert q(A, A * 2, 4, 256, B + 8, B * 2) == _lib.WUSH_EALIGN
    assert q(A, A * 2, 4, 256, B, B * 2 + 4) == _lib.WUSH_EALIGN
    # M = 4 rows pad to 128: the packed codes span 16 KB, so scales 8 KB in overlap.
    assert q(A, A * 2, 4, 256, B, B + 8192) == _lib.WUSH_EINVAL
    assert q(A, A * 2, 4, 256, A + 1024, B * 2) == _lib.WUSH_EINVAL  # codes overlap X


def test_gemm_pack_b_validation_rejects_bad_arguments():
    lib = wush.load()
    p = lambda bc, bs, N, K, pc, ps: lib.wush_gemm_pack_b(bc, bs, N, K, pc, ps, None)
    B = A * 64
    assert p(A, A * 2, 0, 256, B, B * 2) == _lib.WUSH_OK  # N = 0: no-op
    assert p(A, A * 2, -1, 256, B, B * 2) == _lib.WUSH_EINVAL
    assert p(A, A * 2, 16, 320, B, B * 2) == _lib.WUSH_EINVAL  # K not a multiple of 256
    assert p(None, A * 2, 16, 256, B, B * 2) == _lib.WUSH_EINVAL
    assert p(A, A * 2, 16, 256, B, None) == _lib.WUSH_EINVAL
    assert p(A + 8, A * 2, 16, 256, B, B * 2) == _lib.WUSH_EALIGN
    assert p(A, A * 2, 16, 256, B + 8, B * 2) == _lib.WUSH_EALIGN
    assert p(A, A * 2, 16, 256, B, B * 2 + 4) == _lib.WUSH_EALIGN
    assert p(A, A * 2, 16, 256, A + 1024, B * 2) == _lib.WUSH_EINVAL  # packed codes overlap the codes
    assert p(A, A * 2, 16, 256, B, B + 8192) == _lib.WUSH_EINVAL  # packed scales inside packed codes
    assert b"overlap" in lib.wush_last_error()


def test_dequant_validation_rejects_bad_arguments():
    lib = wush.load()
    B = A * 64
    d = lambda fmt, c, s, g, M, K, o: lib.wush_dequant(fmt, c, s, g, M, K, o, None)
    assert d(0, A, A * 2, None, 0, 64, B) == _lib.WUSH_OK  # M = 0: no-op
    assert d(3, A, A * 2, None, 4, 64, B) == _lib.WUSH_EUNSUPPORTED
    assert d(0, A, A * 2, None, -1, 64, B) == _lib.WUSH_EINVAL
    assert d(0, A, A * 2, None, 4, 48, B) == _lib.WUSH_EINVAL  # MXFP4 needs K % 32
    assert d(1, A, A * 2, None, 4, 48, B) == _lib.WUSH_EINVAL  # NVFP4 needs its global scale
    assert d(1, A, A * 2, A * 3, 4, 40, B) == _lib.WUSH_EINVAL  # K % 16
    assert d(0, A + 4, A * 2, None, 4, 64, B) == _lib.WUSH_EALIGN
    assert d(2, A, A * 2 + 1, None, 4, 64, B) == _lib.WUSH_EALIGN
    assert d(0, A, A * 2, None, 4, 64, B + 4) == _lib.WUSH_EALIGN
    assert d(0, A, A * 2, None, 4, 64, A) == _lib.WUSH_EINVAL  # out overlaps codes
    assert d(0, None, A * 2, None, 4, 64, B) == _lib.WUSH_EINVAL


def test_build_transforms_validation():
    lib = wush.load()
    B = A * 64
    b = lambda W, do, X, nc, di, G, damp=1e-6, tw=B, tx=B * 2: lib.wush_build_transforms(
        W, do, X, nc, di, G, damp, 1, tw, tx, None, None, None)
    assert b(A, 8, A * 2, 8, 64, 24) == _lib.WUSH_EUNSUPPORTED
    assert b(A, 0, A * 2, 8, 64, 32) == _lib.WUSH_EINVAL
    assert b(A, 8, A * 2, 0, 64, 32) == _lib.WUSH_EINVAL
    assert b(A, 8, A * 2, 8, 48, 32) == _lib.WUSH_EINVAL
    assert b(A, 8, A * 2, 8, 64, 32, damp=-1.0) == _lib.WUSH_EINVAL
    assert b(A + 8, 8, A * 2, 8, 64, 32) == _lib.WUSH_EALIGN
    assert b(A, 8, A * 2, 8, 64, 32, tw=B + 4) == _lib.WUSH_EALIGN
    assert b(A, 8, A * 2, 8, 64, 32, tx=B) == _lib.WUSH_EINVAL  # outputs overlap
    assert b(None, 8, A * 2, 8, 64, 32) == _lib.WUSH_EINVAL


def test_gptq_block_validation():
    lib = wush.load()
    B = A * 64
    g = lambda fmt, G, d, cs=16, c=B * 3: lib.wush_gptq_block(fmt, A, A * 2, G, d, B, c, cs, B * 5, 1, None)
    assert g(0, 32, 0) == _lib.WUSH_OK
    assert g(1, 32, 8) == _lib.WUSH_EUNSUPPORTED  # NVFP4 not offered
    assert g(0, 24, 8) == _lib.WUSH_EUNSUPPORTED
    assert g(0, 32, -1) == _lib.WUSH_EINVAL
    assert g(0, 32, 8, cs=8) == _lib.WUSH_EINVAL  # row stride shorter than a group's bytes
    assert g(0, 32, 8, cs=18) == _lib.WUSH_EALIGN
    assert g(0, 32, 8, c=B * 3 + 2) == _lib.WUSH_EALIGN
    assert g(0, 32, 8, c=B) == _lib.WUSH_EINVAL  # codes overlap Q


def test_gptq_wush_validation():
    """GPTQ-WUSH rejects bad formats, shapes, damping, alignment and
    overlapping buffers before any HIP call (fake device addresses)."""
    lib = wush.load()
    B = A * 64

    def g(fmt=0, G=32, d_out=40, n=16, d_in=64, damp=0.01, xp=B, codes=B * 5, scales=B * 6):
        return lib.wush_gptq_wush(fmt, A, A * 2, d_out, n, d_in, G, damp, 1, xp, B * 2, B * 3, B * 4, codes,
                                  scales, None)

    assert g(fmt=1) == _lib.WUSH_EUNSUPPORTED  # NVFP4 not offered
    assert g(G=24, d_in=48) == _lib.WUSH_EUNSUPPORTED
    assert g(d_in=48) == _lib.WUSH_EINVAL  # G does not divide d_in
    assert g(d_out=31) == _lib.WUSH_EINVAL  # a block's thin SVD needs G rows
    assert g(n=0) == _lib.WUSH_EINVAL
    assert g(damp=-1.0) == _lib.WUSH_EINVAL
    assert g(damp=float("nan")) == _lib.WUSH_EINVAL
    assert g(xp=B + 4) == _lib.WUSH_EALIGN
    assert g(codes=B * 5 + 2) == _lib.WUSH_EALIGN
    assert g(fmt=2, scales=B * 6 + 1) == _lib.WUSH_EALIGN
    assert g(codes=B * 2) == _lib.WUSH_EINVAL  # codes overlap Y
    assert g(xp=A) == _lib.WUSH_EINVAL  # X' overlaps W


def test_support_entry_validation():
    lib = wush.load()
    B = A * 64
    assert lib.wush_absmax_transformed(A, A * 2, 8, 64, 24, B, None) == _lib.WUSH_EUNSUPPORTED
    assert lib.wush_absmax_transformed(A, A * 2, 8, 64, 32, None, None) == _lib.WUSH_EINVAL
    assert lib.wush_absmax_transformed(A, A * 2, 8, 64, 32, B + 2, None) == _lib.WUSH_EALIGN
    assert lib.wush_nvfp4_global_scale(A, A * 2, 8, 40, B, None) == _lib.WUSH_EINVAL
    assert lib.wush_transform_f32(A, A * 2, 8, 64, 32, B + 4, None) == _lib.WUSH_EALIGN
    assert lib.wush_fixed_transforms(2, 4, 32, B, None, None) == _lib.WUSH_EINVAL
    assert lib.wush_fixed_transforms(1, 4, 8, B, None, None) == _lib.WUSH_EUNSUPPORTED
    assert lib.wush_fixed_transforms(1, 4, 32, None, None, None) == _lib.WUSH_EINVAL
    assert lib.wush_fixed_transforms(1, 4, 32, None, B + 8, None) == _lib.WUSH_EALIGN
    assert lib.wush_fixed_transforms(0, 0, 32, B, None, None) == _lib.WUSH_OK
    assert lib.wush_f64_to_bf16(A, -1, B, None) == _lib.WUSH_EINVAL
    assert lib.wush_f64_to_bf16(A + 4, 8, B, None) == _lib.WUSH_EALIGN
    assert lib.wush_f64_to_bf16(A, 8, A + 8, None) == _lib.WUSH_EINVAL
    assert lib.wush_f64_to_bf16(A, 0, None, None) == _lib.WUSH_OK


def test_binding_checks_caller_buffers():
    """The binding's buffer check (used for every caller-supplied output and
    for global_scale / n_exact) rejects wrong dtype, shape, layout and device
    before the library is called."""
    torch = pytest.importorskip("torch")
    from mxfp4_activation_amd.ops import _check_buf

    dev = torch.device("cpu")
    ok = torch.empty((4, 8), dtype=torch.uint8)
    _check_buf(ok, "codes", torch.uint8, (4, 8), dev)
    with pytest.raises(TypeError, match="codes must be torch.uint8"):
        _check_buf(ok.view(torch.int8), "codes", torch.uint8, (4, 8), dev)
    with pytest.raises(TypeError, match="scales must be torch.float16"):
        _check_buf(torch.empty((4, 2), dtype=torch.uint8), "scales", torch.float16, (4, 1), dev)
    with pytest.raises(ValueError, match="shape"):
        _check_buf(ok, "codes", torch.uint8, (4, 9), dev)
    with pytest.raises(ValueError, match="contiguous"):
        _check_buf(torch.empty((8, 4), dtype=torch.uint8).t(), "codes", torch.uint8, (4, 8), dev)
    with pytest.raises(ValueError, match="must be on"):
        _check_buf(ok, "codes", torch.uint8, (4, 8), torch.device("cuda", 0))
    with pytest.raises(TypeError):
        _check_buf(None, "out", torch.float32, (1,), dev)
