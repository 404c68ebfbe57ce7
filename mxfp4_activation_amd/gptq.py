"""GPTQ-WUSH (Algorithm 1) on the GPU, float64.

"WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep dive,
section 3.4.6: the weight side is calibrated block by block in reverse
order, interleaving the transform construction with GPTQ.

  1. Hx = X^T X / n damped by damp * mean(diag(Hx)) * I; X' = chol(Hx) (global).
  2. Y = W X'.
  3. For b = C-1 .. 0: thin SVD Y[:, b] = U S V^T (v_k's largest entry
     positive); S <- S / sqrt(d_out); T_X = Hd S^1/2 V^T X'[b, b]^-1 (the
     activation transform used online); Wbar = sqrt(d_out) Hd S^1/2 U^T; GPTQ
     of Wbar with the block Hessian Hd S Hd^T (or round-to-nearest); then
     Y <- Y - Wsub^T T_X X'[b, :] with Wsub the quantized block (GPTQ) or
     Wbar (RTN).

The dense linear algebra (global Cholesky, thin SVDs, triangular inverses,
the Y updates) runs as torch float64 operations on the device; the
quantization of every block runs in the library's intra-block GPTQ kernel
(wush_gptq_block), which writes the codes and scales in the row layout the
MXFP4 GEMM and the dequantizer read.  MXFP4 and INT4 are supported; NVFP4
would need a per-tensor scale for weights that do not exist until the last
block is done.
"""

from __future__ import annotations

import dataclasses
import math

import torch

from . import _lib
from .ops import _stream
from .transforms import hadamard_f64

DEFAULT_GPTQ_DAMP = 0.01


@dataclasses.dataclass
class GptqWushResult:
    T_x: torch.Tensor     # float64 [C, G, G] activation transforms
    Wq: torch.Tensor      # float64 [d_out, d_in] dequantized transformed weights
    codes: torch.Tensor   # uint8 [d_out, d_in/2]
    scales: torch.Tensor  # [d_out, C]: uint8 E8M0 (MXFP4) or float16 (INT4)


def gptq_wush(W: torch.Tensor, Xcal: torch.Tensor, G: int, fmt: str, gptq: bool = True,
              damp: float = DEFAULT_GPTQ_DAMP) -> GptqWushResult:
    """W [d_out, d_in] and calibration activations Xcal [n, d_in] on the device
    (any float dtype; computed in float64)."""
    if fmt not in ("mxfp4", "int4"):
        raise ValueError("GPTQ-WUSH supports mxfp4 and int4")
    dev = W.device
    W = W.to(torch.float64)
    X = Xcal.to(device=dev, dtype=torch.float64)
    d_out, d_in = W.shape
    if d_in % G or X.shape[1] != d_in:
        raise ValueError("shape mismatch")
    C = d_in // G
    Hx = X.t() @ X / X.shape[0]
    Hx += damp * torch.diagonal(Hx).mean() * torch.eye(d_in, dtype=torch.float64, device=dev)
    Xp = torch.linalg.cholesky(Hx)
    Y = W @ Xp
    Hd = hadamard_f64(G, dev)
    eye = torch.eye(G, dtype=torch.float64, device=dev)
    T_x = torch.empty((C, G, G), dtype=torch.float64, device=dev)
    Wq = torch.empty((d_out, d_in), dtype=torch.float64, device=dev)
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, C), dtype=torch.float16 if fmt == "int4" else torch.uint8, device=dev)
    Q = torch.empty((G, d_out), dtype=torch.float64, device=dev)
    lib = _lib.load()
    fmt_id = _lib.FMT[fmt]
    for b in reversed(range(C)):
        lo, hi = b * G, (b + 1) * G
        U, s, Vh = torch.linalg.svd(Y[:, lo:hi], full_matrices=False)
        V = Vh.t()
        lead = V.abs().argmax(dim=0)
        sgn = torch.sign(V[lead, torch.arange(G, device=dev)])
        sgn[sgn == 0] = 1.0
        U = U * sgn
        V = V * sgn
        Sn = s / math.sqrt(d_out)
        rs = Sn.sqrt()
        Xbb_inv = torch.linalg.solve_triangular(Xp[lo:hi, lo:hi], eye, upper=False)
        T = Hd @ (rs[:, None] * V.t()) @ Xbb_inv
        Wbar = (math.sqrt(d_out) * (Hd @ (rs[:, None] * U.t()))).contiguous()
        if gptq:
            Hb = Hd @ torch.diag(Sn) @ Hd.t()
            R = torch.linalg.cholesky(torch.linalg.inv(Hb)).t().contiguous()
        else:
            R = eye
        _lib.check(lib.wush_gptq_block(fmt_id, Wbar.data_ptr(), R.data_ptr(), G, d_out, Q.data_ptr(),
                                       codes.data_ptr() + lo // 2, codes.stride(0), scales.data_ptr() + b * scales.element_size(),
                                       scales.stride(0), _stream()), "wush_gptq_block")
        sub = Q if gptq else Wbar
        Y[:, :hi] -= sub.t() @ T @ Xp[lo:hi, :hi]
        T_x[b] = T
        Wq[:, lo:hi] = Q.t()
    return GptqWushResult(T_x, Wq, codes, scales)
