"""Offline construction of the per-block transform bank T[C][G][G].

This is the calibration side of "WUSH: Near-Optimal Adaptive Transforms for
LLM Quantization".  The steps:
  * Blockwise uncentered second moments of the weight and the calibration
    activations (papernotes.org, "整体框架"; deep dive, section 3.2).
  * Their lower Cholesky factors W', X' and the SVD W'^T X' = U S V^T (Eq. 7).
  * T_wush = H S^-1/2 U^T W'^T for the activations and
    T_xvsh = H S^-1/2 V^T X'^T for the weights (Eq. 8, deep dive 3.4.4).
    These satisfy T_xvsh^T T_wush = I.

Every block is solved in one batched float64 torch.linalg call.  The same
readings as the online path's documentation apply:
  * damping lam * mean(diag) * I on both moments;
  * each pair (u_k, v_k) is signed so that v_k's largest-magnitude entry is
    positive;
  * H is Sylvester-ordered and scaled by G^-1/2.

The comparison transforms the pages evaluate go through the same kernel.  The
pages call them RTN-I (identity), RTN-H (blockwise Hadamard) and WUS (WUSH
without H); see deep dive, section 5.
"""

from __future__ import annotations

from typing import Tuple

import torch

DEFAULT_DAMP = 1e-6


def hadamard(G: int, dtype=torch.float64, device=None) -> torch.Tensor:
    if G < 1 or G & (G - 1):
        raise ValueError("G must be a power of two")
    H = torch.ones((1, 1), dtype=dtype, device=device)
    while H.shape[0] < G:
        H = torch.cat([torch.cat([H, H], 1), torch.cat([H, -H], 1)], 0)
    return H / (G ** 0.5)


def _block_moments(W: torch.Tensor, Xcal: torch.Tensor, G: int) -> Tuple[torch.Tensor, torch.Tensor]:
    d_out, d_in = W.shape
    n_cal = Xcal.shape[0]
    C = d_in // G
    Wb = W.reshape(d_out, C, G).permute(1, 0, 2)  # [C, d_out, G]
    Xb = Xcal.reshape(n_cal, C, G).permute(1, 0, 2)  # [C, n_cal, G]
    Sw = torch.bmm(Wb.transpose(1, 2), Wb) / d_out
    Sx = torch.bmm(Xb.transpose(1, 2), Xb) / n_cal
    return Sw, Sx


def _damp(S: torch.Tensor, lam: float) -> torch.Tensor:
    G = S.shape[-1]
    md = torch.diagonal(S, dim1=-2, dim2=-1).mean(-1)
    return S + (lam * md)[:, None, None] * torch.eye(G, dtype=S.dtype, device=S.device)


def wush_transforms(W: torch.Tensor, Xcal: torch.Tensor, G: int, damp: float = DEFAULT_DAMP,
                    use_hadamard: bool = True) -> Tuple[torch.Tensor, torch.Tensor]:
    """T_wush (activation side) and T_xvsh (weight side), float64 [C, G, G].

    W: [d_out, d_in] weight in nn.Linear order; Xcal: [n_cal, d_in]
    calibration activations.  use_hadamard=False gives the WUS variant.
    """
    W = torch.as_tensor(W, dtype=torch.float64)
    Xcal = torch.as_tensor(Xcal, dtype=torch.float64)
    if W.shape[1] != Xcal.shape[1] or W.shape[1] % G:
        raise ValueError("shape mismatch")
    Sw, Sx = _block_moments(W, Xcal, G)
    Wp = torch.linalg.cholesky(_damp(Sw, damp))
    Xp = torch.linalg.cholesky(_damp(Sx, damp))
    U, s, Vh = torch.linalg.svd(Wp.transpose(1, 2) @ Xp)
    V = Vh.transpose(1, 2)
    idx = V.abs().argmax(dim=1, keepdim=True)  # [C, 1, G]: row of each column's largest entry
    sgn = torch.sign(torch.gather(V, 1, idx))
    sgn[sgn == 0] = 1.0
    U = U * sgn
    V = V * sgn
    H = hadamard(G, device=W.device) if use_hadamard else torch.eye(G, dtype=torch.float64, device=W.device)
    scale = s.rsqrt()[:, :, None]  # S^-1/2 applied to rows
    T_wush = H @ (scale * U.transpose(1, 2)) @ Wp.transpose(1, 2)
    T_xvsh = H @ (scale * V.transpose(1, 2)) @ Xp.transpose(1, 2)
    return T_wush, T_xvsh


def identity_transforms(C: int, G: int) -> torch.Tensor:
    return torch.eye(G, dtype=torch.float64).expand(C, G, G).clone()


def hadamard_transforms(C: int, G: int) -> torch.Tensor:
    return hadamard(G).expand(C, G, G).clone()


def to_kernel_layout(T: torch.Tensor) -> torch.Tensor:
    """float64 [C, G, G] -> contiguous bf16, rounded through fp32 (RNE both)."""
    return T.to(torch.float32).to(torch.bfloat16).contiguous()
