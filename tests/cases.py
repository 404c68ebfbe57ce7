"""Seeded test cases shared by the GPU tests: inputs and oracle transforms.

Inputs come from ``synthetic``.  Transforms are built by the oracle
(float64, then bf16), so no input of a parity test comes from the GPU path.
"""

from __future__ import annotations

import functools

import numpy as np

from oracle import transform as tr
from synthetic import CONFIGS, Workload, gen_calibration, gen_weight, gen_x_bits, gen_x_rows


@functools.lru_cache(maxsize=None)
def transforms(name: str, G: int = 0):
    """(T_wush float64, T_bf16 bits) for a workload, built offline by the oracle.

    G overrides the workload's block size (for example, G=16 transforms on
    the tiny workload's statistics)."""
    wl = CONFIGS[name]
    G = G or wl.G
    T64, _ = tr.build_transforms(gen_weight(wl), gen_calibration(wl), G)
    return T64, tr.transforms_to_bf16_bits(T64)


@functools.lru_cache(maxsize=4)
def x_full(name: str) -> np.ndarray:
    return gen_x_bits(CONFIGS[name])


def x_rows(name: str, lo: int, hi: int, M: int = 0) -> np.ndarray:
    wl: Workload = CONFIGS[name]
    return gen_x_rows(wl, lo, hi, M or wl.M)


@functools.lru_cache(maxsize=None)
def oracle_tensor_amax(name: str) -> np.float32:
    """The oracle's AbsMax of the whole transformed tensor, in row chunks."""
    from oracle import quant

    _, tb = transforms(name)
    xb = x_full(name)
    amax = np.float32(0.0)
    for lo in range(0, xb.shape[0], 4096):
        amax = max(amax, quant.tensor_amax_ref(quant.transform_ref(xb[lo:lo + 4096], tb)))
    return np.float32(amax)


def oracle_global_scale(name: str) -> np.float32:
    """NVFP4 tensor scale from the oracle's AbsMax of the whole tensor."""
    from oracle import quant

    return quant.nvfp4_global_scale(oracle_tensor_amax(name))


def sample_rows(M: int, n_edge: int = 48, n_rand: int = 160, seed: int = 0) -> np.ndarray:
    """First and last rows of the tensor plus a seeded random sample."""
    rng = np.random.default_rng(seed)
    rows = set(range(min(n_edge, M))) | set(range(max(0, M - n_edge), M))
    rows |= set(rng.choice(M, min(n_rand, M), replace=False).tolist())
    return np.array(sorted(rows))
