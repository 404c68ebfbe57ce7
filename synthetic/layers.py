"""Seeded synthetic linear layers for the layerwise loss: a weight, a
calibration batch and an evaluation batch.

Random numbers only, rounded to bf16 (round-to-nearest-even); nothing here
transforms or quantizes.  The activation law follows the workloads: heavy
tails (Student-t with 3 degrees of freedom, or Laplace) and a few persistent
outlier channels shared by the calibration and evaluation batches.  The
weight is N(0, w_std) in nn.Linear order [d_out, d_in].
"""

from __future__ import annotations

from typing import Tuple

import numpy as np

from .workloads import f64_to_bf16_bits


def _bf16_values(a: np.ndarray) -> np.ndarray:
    return (f64_to_bf16_bits(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gen_linear_layer(d_in: int, d_out: int, n_cal: int, n_eval: int, seed: int, dist: str = "student_t3",
                     n_outlier: int = 0, outlier_mult: float = 30.0, w_std: float = 0.02
                     ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(W [d_out, d_in], X_cal [n_cal, d_in], X_eval [n_eval, d_in]), float64 values of bf16 numbers."""
    rng = np.random.default_rng(seed)
    outliers = rng.choice(d_in, n_outlier, replace=False) if n_outlier else np.zeros(0, dtype=np.int64)

    def acts(n):
        x = rng.standard_t(3, size=(n, d_in)) if dist == "student_t3" else rng.laplace(size=(n, d_in))
        x[:, outliers] *= outlier_mult
        return _bf16_values(x)

    W = _bf16_values(rng.standard_normal((d_out, d_in)) * w_std)
    return W, acts(n_cal), acts(n_eval)
