"""Pins for the layerwise loss (oracle.loss, Eq. 5), independent of its code.

* Zero: operands whose blocks are already on the MXFP4 / INT4 grid
  (every block holds its scale's largest level) quantize exactly under
  T = I, so the loss is exactly 0.  A transposed operand, a missing
  dequantization step or a wrong reference product would not give 0.
* Power of two: scaling X (or W) by 2 leaves every code unchanged and
  doubles every scale, in all three formats, so the loss grows by exactly 4.
* Aggregation: the mean over tokens and outputs, recomputed with plain
  loops from the dequantized operands.
* Table 1's qualitative orderings (deep dive, section 5, "Per-Layer
  Quantization Loss"), checked on a synthetic heavy-tailed layer with
  outlier channels.  Only the orderings that do not hinge on trained
  weights are asserted: WUSH < H < I for MXFP4 and INT4; for NVFP4 the
  blockwise Hadamard alone is worse than I, while WUS and WUSH are both
  well below I.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import loss, quant
from oracle import transform as tr
from synthetic import f64_to_bf16_bits
from synthetic.layers import gen_linear_layer

E2M1_LEVELS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _eye_bits(K, G):
    return tr.transforms_to_bf16_bits(np.broadcast_to(np.eye(G), (K // G, G, G)).copy())


def _grid_rows(rng, rows, K, fmt):
    """Rows whose 32-blocks sit exactly on the format's grid."""
    x = np.empty((rows, K))
    for r in range(rows):
        for c in range(K // 32):
            k = int(rng.integers(-6, 6))
            if fmt == "mxfp4":
                v = rng.choice(E2M1_LEVELS, 32) * rng.choice([-1.0, 1.0], 32)
                v[rng.integers(32)] = 4.0 * rng.choice([-1.0, 1.0])  # block amax 4 * 2^k -> scale 2^k
            else:
                v = rng.integers(-7, 8, 32).astype(np.float64)
                v[rng.integers(32)] = 7.0 * rng.choice([-1.0, 1.0])  # amax 7 * 2^k -> fp16 scale 2^k
            x[r, 32 * c:32 * c + 32] = np.ldexp(v, k)
    return f64_to_bf16_bits(x)


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_grid_operands_give_zero_loss(fmt):
    rng = np.random.default_rng(3)
    K = 128
    x = _grid_rows(rng, 6, K, fmt)
    w = _grid_rows(rng, 5, K, fmt)
    eye = _eye_bits(K, 32)
    assert loss.layerwise_loss_ref(fmt, x, w, eye, eye) == 0.0
    # A Hadamard moves the values off the grid: the loss becomes positive.
    H = tr.transforms_to_bf16_bits(np.broadcast_to(tr.hadamard(32), (K // 32, 32, 32)).copy())
    assert loss.layerwise_loss_ref(fmt, x, w, H, H) > 0.0


@pytest.mark.parametrize("fmt", ["mxfp4", "nvfp4", "int4"])
def test_power_of_two_scaling(fmt):
    G = 16 if fmt == "nvfp4" else 32
    W, Xc, Xe = gen_linear_layer(64, 24, 256, 20, seed=5, n_outlier=2)
    Tw, Tx = tr.build_transforms(W, Xc, G)
    tx, tw = tr.transforms_to_bf16_bits(Tw), tr.transforms_to_bf16_bits(Tx)
    xb, wb = f64_to_bf16_bits(Xe), f64_to_bf16_bits(W)
    base = loss.layerwise_loss_ref(fmt, xb, wb, tx, tw)
    assert base > 0
    assert loss.layerwise_loss_ref(fmt, f64_to_bf16_bits(2 * Xe), wb, tx, tw) == 4 * base
    assert loss.layerwise_loss_ref(fmt, xb, f64_to_bf16_bits(0.5 * W), tx, tw) == base / 4


def test_aggregation_by_loops():
    W, Xc, Xe = gen_linear_layer(64, 3, 256, 4, seed=9, n_outlier=1)
    Tw, Tx = tr.build_transforms(W, Xc, 32)
    tx, tw = tr.transforms_to_bf16_bits(Tw), tr.transforms_to_bf16_bits(Tx)
    xb, wb = f64_to_bf16_bits(Xe), f64_to_bf16_bits(W)
    xq = loss.quantized_values("mxfp4", xb, tx)
    wq = loss.quantized_values("mxfp4", wb, tw)
    total = 0.0
    for t in range(4):
        for o in range(3):
            q = sum(xq[t, k] * wq[o, k] for k in range(64))
            e = sum(Xe[t, k] * W[o, k] for k in range(64))
            total += (q - e) ** 2
    assert loss.layerwise_loss_ref("mxfp4", xb, wb, tx, tw) == pytest.approx(total / 12, rel=1e-12)


def _losses(fmt, d_in=512, d_out=256, n=256, seed=0):
    G = 16 if fmt == "nvfp4" else 32
    C = d_in // G
    W, Xc, Xe = gen_linear_layer(d_in, d_out, 1024, n, seed=seed, n_outlier=5, outlier_mult=30.0)
    xb, wb = f64_to_bf16_bits(Xe), f64_to_bf16_bits(W)
    Tw, Tx = tr.build_transforms(W, Xc, G)
    Tws, Txs = tr.build_transforms(W, Xc, G, H=np.eye(G))
    H = np.broadcast_to(tr.hadamard(G), (C, G, G)).copy()
    eye = np.broadcast_to(np.eye(G), (C, G, G)).copy()
    banks = {"I": (eye, eye), "H": (H, H), "WUS": (Tws, Txs), "WUSH": (Tw, Tx)}
    return {k: loss.layerwise_loss_ref(fmt, xb, wb, tr.transforms_to_bf16_bits(a), tr.transforms_to_bf16_bits(b))
            for k, (a, b) in banks.items()}


@pytest.mark.parametrize("fmt", ["mxfp4", "int4"])
def test_table1_orderings_fp4_int4(fmt):
    L = _losses(fmt)
    assert L["WUSH"] < L["H"] < L["I"], L


def test_table1_orderings_nvfp4():
    L = _losses("nvfp4")
    assert L["H"] > L["I"], L                       # the Hadamard alone hurts NVFP4
    assert L["WUSH"] < 0.5 * L["I"] and L["WUS"] < 0.5 * L["I"], L
    assert abs(L["WUSH"] - L["WUS"]) < 0.35 * L["WUS"], L  # essentially tied
