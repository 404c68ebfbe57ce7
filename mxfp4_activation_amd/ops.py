"""PyTorch-facing wrappers over the C ABI (argument marshalling only).

Every function takes device tensors on the current HIP device.  It allocates
the outputs with torch unless the caller passes them, and enqueues the
library call on torch's current stream.  No arithmetic of the path runs here.
"""

from __future__ import annotations

from typing import NamedTuple, Optional, Tuple

import torch

from . import _lib

_G = {"mxfp4": 32, "nvfp4": 16, "int4": 32}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check_x_t(X: torch.Tensor, T: torch.Tensor, G: int) -> Tuple[int, int]:
    if X.dtype != torch.bfloat16 or T.dtype != torch.bfloat16:
        raise TypeError("X and T must be bfloat16")
    if not (X.is_cuda and T.is_cuda):
        raise ValueError("X and T must be device tensors")
    if T.device != X.device or X.device.index != torch.cuda.current_device():
        raise ValueError("X and T must be on the current device (X on %s, T on %s, current cuda:%d)"
                         % (X.device, T.device, torch.cuda.current_device()))
    if X.dim() != 2:
        raise ValueError("X must be [M, K]")
    M, K = X.shape
    if T.dim() != 3 or tuple(T.shape[1:]) != (G, G) or T.shape[0] * G != K:
        raise ValueError("T must be [K/%d, %d, %d] for K=%d, got %s" % (G, G, G, K, tuple(T.shape)))
    if not (X.is_contiguous() and T.is_contiguous()):
        raise ValueError("X and T must be contiguous")
    return M, K


def _check_buf(t: torch.Tensor, name: str, dtype: torch.dtype, shape, device) -> None:
    """A caller-supplied buffer must be a contiguous device tensor of exactly
    this dtype and shape on the inputs' device."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s (got %s)" % (name, dtype, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s (got %s)" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.device != device:
        raise ValueError("%s must be on %s (got %s)" % (name, device, t.device))


def quant(fmt: str, X: torch.Tensor, T: torch.Tensor, global_scale: Optional[torch.Tensor] = None,
          codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
          n_exact: Optional[torch.Tensor] = None):
    """Fused transform + quantization.  Returns (codes, scales)."""
    G = _G[fmt]
    M, K = _check_x_t(X, T, G)
    dev = X.device
    sdt = torch.float16 if fmt == "int4" else torch.uint8
    if codes is None:
        codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty((M, K // G), dtype=sdt, device=dev)
    _check_buf(codes, "codes", torch.uint8, (M, K // 2), dev)
    _check_buf(scales, "scales", sdt, (M, K // G), dev)
    gs = 0
    if fmt == "nvfp4":
        if global_scale is None:
            raise ValueError("nvfp4 needs a 1-element float32 global_scale tensor")
        _check_buf(global_scale.view(-1) if global_scale.dim() else global_scale.view(1), "global_scale",
                   torch.float32, (1,), dev)
        gs = global_scale.data_ptr()
    ne = 0
    if n_exact is not None:
        _check_buf(n_exact.view(-1) if n_exact.dim() else n_exact.view(1), "n_exact", torch.int32, (1,), dev)
        ne = n_exact.data_ptr()
    lib = _lib.load()
    st = lib.wush_quant(_lib.FMT[fmt], X.data_ptr(), T.data_ptr(), M, K, gs or None, codes.data_ptr(),
                        scales.data_ptr(), ne or None, _stream())
    _lib.check(st, "wush_quant(%s)" % fmt)
    return codes, scales


def quant_mxfp4(X, T, codes=None, scales=None):
    return quant("mxfp4", X, T, codes=codes, scales=scales)


def quant_nvfp4(X, T, global_scale, codes=None, scales=None):
    return quant("nvfp4", X, T, global_scale=global_scale, codes=codes, scales=scales)


def quant_int4(X, T, codes=None, scales=None):
    return quant("int4", X, T, codes=codes, scales=scales)


def build_transforms(W: torch.Tensor, Xcal: torch.Tensor, G: int, damp: float = 1e-6, use_hadamard: bool = True,
                     bf16: bool = True):
    """WUSH (or WUS) transforms built on the GPU from a bf16 weight [d_out, d_in]
    and bf16 calibration activations [n_cal, d_in].  Returns (T_wush, T_xvsh)
    float64 [d_in/G, G, G] and, if bf16, their bf16(fp32(T)) kernel-layout
    copies (else None)."""
    for t in (W, Xcal):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError("W and Xcal must be contiguous 2-D bf16 device tensors")
    d_out, d_in = W.shape
    n_cal = Xcal.shape[0]
    if Xcal.shape[1] != d_in:
        raise ValueError("W and Xcal disagree on d_in")
    C = d_in // G if G else 0
    dev = W.device
    tw = torch.empty((C, G, G), dtype=torch.float64, device=dev)
    tx = torch.empty((C, G, G), dtype=torch.float64, device=dev)
    bw = torch.empty((C, G, G), dtype=torch.bfloat16, device=dev) if bf16 else None
    bx = torch.empty((C, G, G), dtype=torch.bfloat16, device=dev) if bf16 else None
    lib = _lib.load()
    _lib.check(lib.wush_build_transforms(W.data_ptr(), d_out, Xcal.data_ptr(), n_cal, d_in, G, float(damp),
                                         1 if use_hadamard else 0, tw.data_ptr(), tx.data_ptr(),
                                         bw.data_ptr() if bf16 else None, bx.data_ptr() if bf16 else None, _stream()),
               "wush_build_transforms")
    return tw, tx, bw, bx


def dequant(fmt: str, codes: torch.Tensor, scales: torch.Tensor, global_scale: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp32 values of quantized rows (codes [M][K/2], scales [M][K/G])."""
    G = _G[fmt]
    if codes.dtype != torch.uint8 or not codes.is_cuda or not codes.is_contiguous() or codes.dim() != 2:
        raise ValueError("codes must be a contiguous 2-D uint8 device tensor")
    M, K = codes.shape[0], codes.shape[1] * 2
    sdt = torch.float16 if fmt == "int4" else torch.uint8
    if scales.dtype != sdt or tuple(scales.shape) != (M, K // G) or not scales.is_contiguous():
        raise ValueError("scales must be a contiguous %s tensor of shape (M, K/%d)" % (sdt, G))
    if fmt == "nvfp4" and (global_scale is None or global_scale.dtype != torch.float32 or global_scale.numel() != 1):
        raise ValueError("NVFP4 needs a one-element fp32 device global_scale")
    if out is None:
        out = torch.empty((M, K), dtype=torch.float32, device=codes.device)
    elif out.dtype != torch.float32 or tuple(out.shape) != (M, K) or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    lib = _lib.load()
    gs = global_scale.data_ptr() if fmt == "nvfp4" else None
    _lib.check(lib.wush_dequant(_lib.FMT[fmt], codes.data_ptr(), scales.data_ptr(), gs, M, K, out.data_ptr(), _stream()),
               "wush_dequant")
    return out


def gemm_mxfp4(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
               out_dtype: torch.dtype = torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C[m][n] = sum_k a[m][k] b[n][k] for MXFP4 operands (codes [rows][K/2],
    E8M0 scales [rows][K/32]), fp32 accumulation, output fp32 or bf16."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    for t in (a_codes, a_scales, b_codes, b_scales):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError("codes and scales must be contiguous 2-D uint8 device tensors")
    M, N, K = a_codes.shape[0], b_codes.shape[0], a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K or tuple(a_scales.shape) != (M, K // 32) or tuple(b_scales.shape) != (N, K // 32):
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    lib = _lib.load()
    _lib.check(lib.wush_gemm_mxfp4(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(),
                                   M, N, K, out.data_ptr(), 1 if out_dtype == torch.bfloat16 else 0, _stream()),
               "wush_gemm_mxfp4")
    return out


class Packed(NamedTuple):
    """An MXFP4 GEMM operand in the packed layout (wush_gemm_pack_b,
    wush_quant_mxfp4_packed): rows rounded up to a multiple of 128; per
    128-row tile and 256-element K step, the codes and scales in the order
    the GEMM kernel stages them."""
    codes: torch.Tensor   # uint8 [rows_p * K / 2]
    scales: torch.Tensor  # uint8 [rows_p * K / 32]
    rows: int             # unpadded row count
    K: int


def _rows_p(rows: int) -> int:
    return (rows + 127) // 128 * 128


def gemm_pack_b(b_codes: torch.Tensor, b_scales: torch.Tensor) -> Packed:
    """Re-lay MXFP4 weights (codes [N][K/2], E8M0 scales [N][K/32]) for
    gemm_mxfp4_packed; done once, offline."""
    for t in (b_codes, b_scales):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous() or t.dim() != 2:
            raise ValueError("codes and scales must be contiguous 2-D uint8 device tensors")
    N, K = b_codes.shape[0], b_codes.shape[1] * 2
    if tuple(b_scales.shape) != (N, K // 32):
        raise ValueError("operand shapes do not match")
    pc = torch.empty(_rows_p(N) * K // 2, dtype=torch.uint8, device=b_codes.device)
    ps = torch.empty(_rows_p(N) * K // 32, dtype=torch.uint8, device=b_codes.device)
    lib = _lib.load()
    _lib.check(lib.wush_gemm_pack_b(b_codes.data_ptr(), b_scales.data_ptr(), N, K, pc.data_ptr(), ps.data_ptr(),
                                    _stream()), "wush_gemm_pack_b")
    return Packed(pc, ps, N, K)


def quant_mxfp4_packed(X: torch.Tensor, T: torch.Tensor, out: Optional[Packed] = None) -> Packed:
    """quant_mxfp4 with the codes and scales written in the GEMM's packed
    operand layout (the same values, placed for gemm_mxfp4_packed)."""
    M, K = _check_x_t(X, T, 32)
    if K % 256:
        raise ValueError("the packed layout needs K to be a multiple of 256")
    if out is None:
        out = Packed(torch.empty(_rows_p(M) * K // 2, dtype=torch.uint8, device=X.device),
                     torch.empty(_rows_p(M) * K // 32, dtype=torch.uint8, device=X.device), M, K)
    elif (out.rows != M or out.K != K or out.codes.numel() != _rows_p(M) * K // 2
          or out.scales.numel() != _rows_p(M) * K // 32):
        raise ValueError("out has the wrong size")
    for t in (out.codes, out.scales):
        if t.dtype != torch.uint8 or t.device != X.device or not t.is_contiguous():
            raise ValueError("out must be contiguous uint8 tensors on X's device")
    lib = _lib.load()
    _lib.check(lib.wush_quant_mxfp4_packed(X.data_ptr(), T.data_ptr(), M, K, out.codes.data_ptr(),
                                           out.scales.data_ptr(), _stream()), "wush_quant_mxfp4_packed")
    return out


def gemm_mxfp4_packed(a, b: Packed, out_dtype: torch.dtype = torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """gemm_mxfp4 with the weights from gemm_pack_b: the same result.  a is
    either (codes [M][K/2], scales [M][K/32]) as quant_mxfp4 writes them, or
    a Packed operand from quant_mxfp4_packed."""
    if out_dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("out_dtype must be float32 or bfloat16")
    a_packed = isinstance(a, Packed)
    if a_packed:
        a_codes, a_scales, M, K = a.codes, a.scales, a.rows, a.K
        if a_codes.numel() != _rows_p(M) * K // 2 or a_scales.numel() != _rows_p(M) * K // 32:
            raise ValueError("operand shapes do not match")
    else:
        a_codes, a_scales = a
        if a_codes.dim() != 2:
            raise ValueError("a_codes must be 2-D")
        M, K = a_codes.shape[0], a_codes.shape[1] * 2
        if tuple(a_scales.shape) != (M, K // 32):
            raise ValueError("operand shapes do not match")
    for t in (a_codes, a_scales, b.codes, b.scales):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("codes and scales must be contiguous uint8 device tensors")
    N = b.rows
    if b.K != K or b.codes.numel() != _rows_p(N) * K // 2 or b.scales.numel() != _rows_p(N) * K // 32:
        raise ValueError("operand shapes do not match")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=a_codes.device)
    elif out.dtype != out_dtype or tuple(out.shape) != (M, N) or not out.is_contiguous():
        raise ValueError("out has the wrong shape, dtype or layout")
    lib = _lib.load()
    _lib.check(lib.wush_gemm_mxfp4_packed(a_codes.data_ptr(), a_scales.data_ptr(), 1 if a_packed else 0,
                                          b.codes.data_ptr(), b.scales.data_ptr(), M, N, K, out.data_ptr(),
                                          1 if out_dtype == torch.bfloat16 else 0, _stream()),
               "wush_gemm_mxfp4_packed")
    return out


def transform_f32(X: torch.Tensor, T: torch.Tensor, Y: Optional[torch.Tensor] = None) -> torch.Tensor:
    G = T.shape[-1]
    M, K = _check_x_t(X, T, G)
    if Y is None:
        Y = torch.empty((M, K), dtype=torch.float32, device=X.device)
    _check_buf(Y, "Y", torch.float32, (M, K), X.device)
    lib = _lib.load()
    _lib.check(lib.wush_transform_f32(X.data_ptr(), T.data_ptr(), M, K, G, Y.data_ptr(), _stream()),
               "wush_transform_f32")
    return Y


def absmax_transformed(X: torch.Tensor, T: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Largest |y| of the exactly rounded transform over the whole tensor, as
    a one-element fp32 device tensor."""
    G = T.shape[-1]
    M, K = _check_x_t(X, T, G)
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=X.device)
    _check_buf(out, "out", torch.float32, (1,), X.device)
    lib = _lib.load()
    _lib.check(lib.wush_absmax_transformed(X.data_ptr(), T.data_ptr(), M, K, G, out.data_ptr(), _stream()),
               "wush_absmax_transformed")
    return out


def nvfp4_global_scale(X: torch.Tensor, T: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    M, K = _check_x_t(X, T, 16)
    if out is None:
        out = torch.empty((1,), dtype=torch.float32, device=X.device)
    _check_buf(out, "out", torch.float32, (1,), X.device)
    lib = _lib.load()
    _lib.check(lib.wush_nvfp4_global_scale(X.data_ptr(), T.data_ptr(), M, K, out.data_ptr(), _stream()),
               "wush_nvfp4_global_scale")
    return out


def e2m1_encode(v: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if v.dtype != torch.float32 or not v.is_cuda or not v.is_contiguous():
        raise ValueError("v must be a contiguous float32 device tensor")
    if out is None:
        out = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check_buf(out, "out", torch.uint8, v.shape, v.device)
    lib = _lib.load()
    _lib.check(lib.wush_e2m1_encode(v.data_ptr(), v.numel(), out.data_ptr(), _stream()), "wush_e2m1_encode")
    return out


def fixed_transforms(kind: str, C: int, G: int, device, f64: bool = False):
    """Identity ("identity") or normalized Sylvester Hadamard ("hadamard")
    bank [C, G, G], built by the library on the device: the bf16 kernel
    layout, or float64 with f64=True."""
    kinds = {"identity": 0, "hadamard": 1}
    if kind not in kinds:
        raise ValueError("kind must be 'identity' or 'hadamard'")
    dt = torch.float64 if f64 else torch.bfloat16
    out = torch.empty((C, G, G), dtype=dt, device=device)
    lib = _lib.load()
    _lib.check(lib.wush_fixed_transforms(kinds[kind], C, G, out.data_ptr() if f64 else None,
                                         None if f64 else out.data_ptr(), _stream()), "wush_fixed_transforms")
    return out


def f64_to_bf16(T: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """bf16(fp32(T)) of a float64 device tensor (the kernel layout of a bank)."""
    if T.dtype != torch.float64 or not T.is_cuda or not T.is_contiguous():
        raise ValueError("T must be a contiguous float64 device tensor")
    if out is None:
        out = torch.empty(T.shape, dtype=torch.bfloat16, device=T.device)
    _check_buf(out, "out", torch.bfloat16, T.shape, T.device)
    lib = _lib.load()
    _lib.check(lib.wush_f64_to_bf16(T.data_ptr(), T.numel(), out.data_ptr(), _stream()), "wush_f64_to_bf16")
    return out
