"""Offline weight side and layerwise loss on the GPU.

"WUSH: Near-Optimal Adaptive Transforms for LLM Quantization":
  * Weights are transformed and quantized offline, W~ = q(T_xvsh W) per
    block (deep dive, sections 3.4.6 and 3.4.8): the same fused kernel as
    the activations, fed the weight rows and the weight-side bank.
  * The layerwise loss of Eq. 5 (deep dive, section 3.4.1) is the mean
    squared error per output element between the unquantized product and
    the product of the two quantized operands.

Transform pairs (activation bank, weight bank) compared in Table 1 (deep
dive, section 5): I (plain RTN), H (blockwise Hadamard on both sides), WUS
(WUSH without the Hadamard factor) and WUSH.  The kernels do the transform,
quantization and dequantization; the two products are torch fp32 GEMMs.
"""

from __future__ import annotations

from typing import Dict, Tuple

import torch

from . import ops, transforms

TRANSFORM_PAIRS = ("I", "H", "WUS", "WUSH")


def transform_pairs(W: torch.Tensor, Xcal: torch.Tensor, G: int) -> Dict[str, Tuple[torch.Tensor, torch.Tensor]]:
    """bf16 kernel-layout banks (activation side, weight side) for each pair,
    built by the library from a bf16 device weight W [d_out, d_in] and bf16
    device calibration activations Xcal [n_cal, d_in]."""
    C = W.shape[1] // G
    wush_a, wush_w, _, _ = transforms.wush_bank(W, Xcal, G)
    wus_a, wus_w, _, _ = transforms.wush_bank(W, Xcal, G, use_hadamard=False)
    eye = transforms.identity_bank(C, G, W.device)
    had = transforms.hadamard_bank(C, G, W.device)
    return {"I": (eye, eye), "H": (had, had), "WUS": (wus_a, wus_w), "WUSH": (wush_a, wush_w)}


def quantize(fmt: str, X: torch.Tensor, bank: torch.Tensor):
    """(codes, scales, global_scale or None) of q(T x) for every row of a bf16 operand.
    NVFP4 takes the operand's own dynamic tensor scale."""
    g = ops.nvfp4_global_scale(X, bank) if fmt == "nvfp4" else None
    codes, scales = ops.quant(fmt, X, bank, global_scale=g)
    return codes, scales, g


def layerwise_loss(fmt: str, X: torch.Tensor, W: torch.Tensor, act_bank: torch.Tensor,
                   weight_bank: torch.Tensor) -> float:
    """Eq. 5 for bf16 activations X [n, d_in] and weight W [d_out, d_in] (nn.Linear order)."""
    xc, xs, xg = quantize(fmt, X, act_bank)
    wc, ws, wg = quantize(fmt, W, weight_bank)
    xq = ops.dequant(fmt, xc, xs, xg)
    wq = ops.dequant(fmt, wc, ws, wg)
    prev = torch.backends.cuda.matmul.allow_tf32
    torch.backends.cuda.matmul.allow_tf32 = False
    try:
        diff = xq @ wq.t() - X.float() @ W.float().t()
    finally:
        torch.backends.cuda.matmul.allow_tf32 = prev
    return float(diff.double().pow(2).mean().item())
