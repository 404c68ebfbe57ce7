"""Layerwise loss of joint weight-activation quantization.  TEST INFRASTRUCTURE ONLY.

Source: "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization", deep
dive, section 3.4.1, Eq. 5: the mean squared error per output element
between W^T X and q(T_W W)^T q(T_X X), i.e. the squared Frobenius norm of
the difference divided by d_out * d_batch.  In nn.Linear orientation
(W [d_out, d_in], X [n, d_in]) the same number is
    mean over tokens t and outputs o of (q(T_X x_t) . q(T_W w_o) - x_t . w_o)^2.
Both transforms act blockwise on the input-channel axis (Eq. 10: T_X =
T_wush on the activations, T_W = T_xvsh on the weights).  q is this
package's quantizer (quant.run_path) followed by its dequantization; the
NVFP4 tensor scale of each operand comes from that operand's own
transformed AbsMax.  Everything is float64.
"""

from __future__ import annotations

import numpy as np

from . import quant


def _bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def quantized_values(fmt: str, bits: np.ndarray, t_bits: np.ndarray) -> np.ndarray:
    """Dequantized q(T x) for every row of a bf16 operand, float64 [rows, K]."""
    G = t_bits.shape[1]
    y = quant.transform_ref(bits, t_bits)
    if fmt == "mxfp4":
        codes, scales = quant.quant_mxfp4_ref(y, G)
        return quant.dequant_mxfp4(codes, scales, G)
    if fmt == "nvfp4":
        g = quant.nvfp4_global_scale(quant.tensor_amax_ref(y))
        codes, scales = quant.quant_nvfp4_ref(y, g, G)
        return quant.dequant_nvfp4(codes, scales, g, G)
    if fmt == "int4":
        codes, scales = quant.quant_int4_ref(y, G)
        return quant.dequant_int4(codes, scales, G)
    raise ValueError(fmt)


def layerwise_loss_ref(fmt: str, x_bits: np.ndarray, w_bits: np.ndarray, tx_bits: np.ndarray,
                       tw_bits: np.ndarray) -> float:
    """Eq. 5 for activations x_bits [n, K] and weight w_bits [d_out, K] (bf16 bits)."""
    xq = quantized_values(fmt, x_bits, tx_bits)
    wq = quantized_values(fmt, w_bits, tw_bits)
    exact = _bf16_to_f64(x_bits) @ _bf16_to_f64(w_bits).T
    return float(np.mean((xq @ wq.T - exact) ** 2))
