"""Seeded random MXFP4 operands and the linear-layer shapes of the GEMM workload.

Random bytes only: E2M1 code nibbles and E8M0 scale bytes drawn uniformly
from the requested ranges.  Nothing here decodes or multiplies them.
"""

from __future__ import annotations

from typing import Dict, Tuple

import numpy as np

# Linear layers of one Qwen3-8B decoder block as (N = output features,
# K = input features): hidden size 4096, 32 query heads and 8 key/value heads
# of width 128, MLP width 12288.
QWEN3_8B_LAYERS: Dict[str, Tuple[int, int]] = {
    "q_proj": (4096, 4096),
    "k_proj": (1024, 4096),
    "v_proj": (1024, 4096),
    "o_proj": (4096, 4096),
    "gate_proj": (12288, 4096),
    "up_proj": (12288, 4096),
    "down_proj": (4096, 12288),
}

# The other two models of the pages' per-layer speedup comparison (deep
# dive, section 5), from their published architecture sizes.
# Qwen3-14B: hidden size 5120, 40 query and 8 key/value heads of width 128,
# MLP width 17408.
QWEN3_14B_LAYERS: Dict[str, Tuple[int, int]] = {
    "q_proj": (5120, 5120),
    "k_proj": (1024, 5120),
    "v_proj": (1024, 5120),
    "o_proj": (5120, 5120),
    "gate_proj": (17408, 5120),
    "up_proj": (17408, 5120),
    "down_proj": (5120, 17408),
}
# Llama-3.1-70B: hidden size 8192, 64 query and 8 key/value heads of width
# 128, MLP width 28672.
LLAMA31_70B_LAYERS: Dict[str, Tuple[int, int]] = {
    "q_proj": (8192, 8192),
    "k_proj": (1024, 8192),
    "v_proj": (1024, 8192),
    "o_proj": (8192, 8192),
    "gate_proj": (28672, 8192),
    "up_proj": (28672, 8192),
    "down_proj": (8192, 28672),
}
MODEL_LAYERS: Dict[str, Dict[str, Tuple[int, int]]] = {
    "qwen3-8b": QWEN3_8B_LAYERS,
    "qwen3-14b": QWEN3_14B_LAYERS,
    "llama3.1-70b": LLAMA31_70B_LAYERS,
}

# Projections that share their input, run as one linear layer with the
# concatenated weight (one transform bank built from that weight): q|k|v and
# gate|up.
QWEN3_8B_FUSED: Dict[str, Tuple[int, int]] = {
    "qkv_proj": (4096 + 1024 + 1024, 4096),
    "gate_up_proj": (2 * 12288, 4096),
}

# Token batch of the per-layer GEMM measurement.
GEMM_TOKENS = 1024


def gen_mx_operand(rows: int, K: int, seed: int, scale_lo: int = 127, scale_hi: int = 127,
                   mag_max: int = 7) -> Tuple[np.ndarray, np.ndarray]:
    """(codes u8 [rows][K/2], scales u8 [rows][K/32]).

    Each nibble has a uniform sign bit and a uniform magnitude code in
    [0, mag_max]; each scale byte is uniform in [scale_lo, scale_hi]."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    rng = np.random.default_rng(seed)
    mag = rng.integers(0, mag_max + 1, size=(rows, K), dtype=np.uint8)
    sign = rng.integers(0, 2, size=(rows, K), dtype=np.uint8) << 3
    nib = mag | sign
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(scale_lo, scale_hi + 1, size=(rows, K // 32), dtype=np.uint8)
    return codes, scales
