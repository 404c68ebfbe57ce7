"""Transform banks T[C][G][G] for the fused kernel, built by the library.

The calibration side of "WUSH: Near-Optimal Adaptive Transforms for LLM
Quantization" (Eq. 7 and Eq. 8; deep dive, sections 3.2 and 3.4.2-3.4.4):
blockwise uncentered second moments of the weight and of calibration
activations, their lower Cholesky factors W', X', the SVD W'^T X' = U S V^T,
then T_wush = H S^-1/2 U^T W'^T for the activations and
T_xvsh = H S^-1/2 V^T X'^T for the weights.  All of it runs in the HIP
library (``wush_build_transforms``, float64 on the device); this module only
allocates and forwards.

The data-agnostic comparators of the pages' evaluation (deep dive, section
5) go through the same kernel: the identity (plain RTN), the blockwise
normalized Hadamard matrix (RTN-H), and WUS (WUSH with H replaced by I).
They come from ``wush_fixed_transforms`` and ``wush_build_transforms``.
"""

from __future__ import annotations

from typing import Tuple

import torch

from . import ops

DEFAULT_DAMP = 1e-6


def _bf16_device(t: torch.Tensor, name: str) -> None:
    if t.dtype != torch.bfloat16 or not t.is_cuda or t.dim() != 2 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 2-D bf16 device tensor" % name)


def wush_bank(W: torch.Tensor, Xcal: torch.Tensor, G: int, use_hadamard: bool = True,
              damp: float = DEFAULT_DAMP) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """(activation bank, weight bank) in the bf16 kernel layout, then the same
    two in float64, for a bf16 weight W [d_out, d_in] (nn.Linear order) and
    bf16 calibration activations Xcal [n_cal, d_in], both on the device.
    use_hadamard=False gives the WUS variant."""
    _bf16_device(W, "W")
    _bf16_device(Xcal, "Xcal")
    tw, tx, bw, bx = ops.build_transforms(W, Xcal, G, damp=damp, use_hadamard=use_hadamard, bf16=True)
    return bw, bx, tw, tx


def identity_bank(C: int, G: int, device) -> torch.Tensor:
    """Plain RTN: T[c] = I, bf16 kernel layout."""
    return ops.fixed_transforms("identity", C, G, device)


def hadamard_bank(C: int, G: int, device) -> torch.Tensor:
    """RTN-H: T[c] = H / sqrt(G) (Sylvester order), bf16 kernel layout."""
    return ops.fixed_transforms("hadamard", C, G, device)


def hadamard_f64(G: int, device) -> torch.Tensor:
    """The normalized Sylvester Hadamard matrix [G, G] in float64."""
    return ops.fixed_transforms("hadamard", 1, G, device, f64=True)[0]


def to_kernel_layout(T: torch.Tensor) -> torch.Tensor:
    """A float64 device bank -> bf16(fp32(T)), contiguous, on the device."""
    return ops.f64_to_bf16(T.contiguous())
