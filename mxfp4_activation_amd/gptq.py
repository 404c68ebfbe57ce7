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

Every step runs in the library (wush_gptq_wush): the Hessian, its blocked
Cholesky factorization and the float64 GEMMs, per block the SVD (through
the block's Gram matrix), the transforms and the intra-block GPTQ, and the
dequantized weights.  This module only allocates
the outputs and passes pointers.  MXFP4 and INT4 are supported; NVFP4
would need a per-tensor scale for weights that do not exist until the last
block is done.
"""

from __future__ import annotations

import dataclasses

import torch

from . import _lib
from .ops import _stream

DEFAULT_GPTQ_DAMP = 0.01


@dataclasses.dataclass
class GptqWushResult:
    T_x: torch.Tensor     # float64 [C, G, G] activation transforms
    Wq: torch.Tensor      # float64 [d_out, d_in] dequantized transformed weights
    codes: torch.Tensor   # uint8 [d_out, d_in/2]
    scales: torch.Tensor  # [d_out, C]: uint8 E8M0 (MXFP4) or float16 (INT4)
    Xp: torch.Tensor      # float64 [d_in, d_in] lower Cholesky factor of the damped Hessian
    Y: torch.Tensor       # float64 [d_out, d_in]: block b's columns = the target block b was fitted to


def gptq_wush(W: torch.Tensor, Xcal: torch.Tensor, G: int, fmt: str, gptq: bool = True,
              damp: float = DEFAULT_GPTQ_DAMP) -> GptqWushResult:
    """W [d_out, d_in] and calibration activations Xcal [n, d_in] on the device
    (any float dtype; passed to the library as float64)."""
    if fmt not in ("mxfp4", "int4"):
        raise ValueError("GPTQ-WUSH supports mxfp4 and int4")
    if W.dim() != 2 or Xcal.dim() != 2 or not W.is_cuda or Xcal.device != W.device:
        raise ValueError("W and Xcal must be 2-D tensors on the same device")
    dev = W.device
    W = W.to(torch.float64).contiguous()
    X = Xcal.to(torch.float64).contiguous()
    d_out, d_in = W.shape
    if d_in % G or X.shape[1] != d_in:
        raise ValueError("shape mismatch")
    C = d_in // G
    f64 = dict(dtype=torch.float64, device=dev)
    Xp = torch.empty((d_in, d_in), **f64)
    Y = torch.empty((d_out, d_in), **f64)
    T_x = torch.empty((C, G, G), **f64)
    Wq = torch.empty((d_out, d_in), **f64)
    codes = torch.empty((d_out, d_in // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((d_out, C), dtype=torch.float16 if fmt == "int4" else torch.uint8, device=dev)
    lib = _lib.load()
    _lib.check(lib.wush_gptq_wush(_lib.FMT[fmt], W.data_ptr(), X.data_ptr(), d_out, X.shape[0], d_in, G, float(damp),
                                  1 if gptq else 0, Xp.data_ptr(), Y.data_ptr(), T_x.data_ptr(), Wq.data_ptr(),
                                  codes.data_ptr(), scales.data_ptr(), _stream()), "wush_gptq_wush")
    return GptqWushResult(T_x, Wq, codes, scales, Xp, Y)
