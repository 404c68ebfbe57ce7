"""Seeded synthetic activations, weights and calibration sets.

Source pages: "WUSH: Near-Optimal Adaptive Transforms for LLM Quantization"
(arXiv 2512.00956).  The pages measure on trained Llama/Qwen layers, with
calibration tokens from a public web-text corpus.  Neither the weights nor the
corpus is available, so these generators stand in for them.  They keep the
activation widths (4096, 14336, 8192).  They also keep the structure that
motivates the method: heavy tails, plus a few persistent outlier channels
(paper-graph deep dive, section 2, "The Core Problem").  These are inputs only.
The transform and the codecs live elsewhere.

Rules, kept the same for every workload:
  * Outlier channels come from ``rng.choice(K, n, replace=False)`` with the
    workload's outlier seed.  The calibration set and the run-time
    activations share them, because outliers belong to the layer.
  * Values are drawn in float64.  They are rounded to float32 (numpy's
    round-to-nearest-even), then to bf16 (round-to-nearest-even on the bit
    pattern, below).  The result is returned as uint16 bit patterns.
  * Activations are produced in chunks of ``CHUNK`` rows.  Chunk i is seeded by
    ``SeedSequence(seed).spawn(n_chunks)[i]``, so any row range can be
    regenerated without drawing the rows before it.
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Dict, Iterable, Optional, Tuple

import numpy as np

CHUNK = 4096


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    fmt: str  # "mxfp4" | "nvfp4" | "int4"
    M: int  # tokens
    K: int  # channels (d_in)
    G: int  # transform block = quantization group
    dist: str  # "normal" | "student_t3" | "laplace"
    n_outlier: int
    outlier_mult: float
    d_out: int  # rows of the nn.Linear-ordered weight [d_out x d_in]
    n_cal: int  # calibration tokens
    seed_w: int
    seed_cal: int
    seed_x: int
    seed_outlier: int
    w_std: float = 0.02

    @property
    def C(self) -> int:
        return self.K // self.G


def _wl(idx, name, fmt, M, K, G, dist, n_out, mult, d_out, n_cal):
    b = idx * 1000
    return Workload(name, fmt, M, K, G, dist, n_out, mult, d_out, n_cal,
                    b + 1, b + 2, b + 3, b + 4)


# Index 1..5 follow the workload list: a tiny MXFP4 case, then three
# model-shaped layers and one large INT4 batch.  n_outlier rounds
# fraction * K to the nearest integer (1% of 4096 = 41, 0.5% of
# 14336 = 72, 1% of 8192 = 82).
CONFIGS: Dict[str, Workload] = {
    "tiny_mxfp4": _wl(1, "tiny_mxfp4", "mxfp4", 128, 256, 32, "normal", 2, 50.0, 256, 512),
    "llama8b_mxfp4": _wl(2, "llama8b_mxfp4", "mxfp4", 4096, 4096, 32, "student_t3", 41, 30.0, 4096, 2048),
    "downproj_mxfp4": _wl(3, "downproj_mxfp4", "mxfp4", 8192, 14336, 32, "laplace", 72, 100.0, 4096, 2048),
    "nvfp4": _wl(4, "nvfp4", "nvfp4", 16384, 4096, 16, "student_t3", 41, 30.0, 4096, 2048),
    "int4": _wl(5, "int4", "int4", 65536, 8192, 32, "laplace", 82, 50.0, 8192, 4096),
}


def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 (RNE) -> bf16 (RNE) bit patterns as uint16.

    Finite inputs only.  The bf16 step adds 0x7FFF plus the lowest kept bit,
    then truncates, which rounds to nearest with ties to even.
    """
    f = np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def outlier_channels(wl: Workload) -> np.ndarray:
    rng = np.random.default_rng(wl.seed_outlier)
    return np.sort(rng.choice(wl.K, wl.n_outlier, replace=False))


def _draw(rng: np.random.Generator, dist: str, shape) -> np.ndarray:
    if dist == "normal":
        return rng.standard_normal(shape)
    if dist == "student_t3":
        return rng.standard_t(3.0, shape)
    if dist == "laplace":
        return rng.laplace(0.0, 1.0, shape)
    raise ValueError(dist)


def _chunk_f64(wl: Workload, seq: np.random.SeedSequence, n: int,
               outl: np.ndarray) -> np.ndarray:
    block = _draw(np.random.default_rng(seq), wl.dist, (n, wl.K))
    block[:, outl] *= wl.outlier_mult
    return block


def _rows_bits(wl: Workload, seed: int, n_rows: int, lo: int, hi: int,
               workers: Optional[int] = None) -> np.ndarray:
    """bf16 bits of rows [lo, hi) of an n_rows x K activation-like matrix.

    Chunks are drawn in a thread pool (numpy's generators and casts release
    the GIL); each chunk has its own generator, so the result does not depend
    on the number of workers.
    """
    n_chunks = max(1, -(-n_rows // CHUNK))
    seqs = np.random.SeedSequence(seed).spawn(n_chunks)
    outl = outlier_channels(wl)
    out = np.empty((hi - lo, wl.K), dtype=np.uint16)
    if hi <= lo:
        return out

    def job(ci: int) -> None:
        r0 = ci * CHUNK
        r1 = min(n_rows, r0 + CHUNK)
        a, b = max(lo, r0), min(hi, r1)
        block = _chunk_f64(wl, seqs[ci], r1 - r0, outl)
        out[a - lo:b - lo] = f64_to_bf16_bits(block[a - r0:b - r0])

    chunks = range(lo // CHUNK, (hi - 1) // CHUNK + 1)
    if workers is None:
        workers = min(8, len(os.sched_getaffinity(0)))
    if workers <= 1 or len(chunks) == 1:
        for ci in chunks:
            job(ci)
    else:
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(job, chunks))
    return out


def gen_x_rows(wl: Workload, lo: int, hi: int, M: Optional[int] = None) -> np.ndarray:
    """bf16 bits of run-time activation rows [lo, hi) (uint16, [hi-lo, K])."""
    M = wl.M if M is None else M
    if not (0 <= lo <= hi <= M):
        raise ValueError("row range out of bounds")
    return _rows_bits(wl, wl.seed_x, M, lo, hi)


def gen_x_bits(wl: Workload, M: Optional[int] = None) -> np.ndarray:
    """bf16 bits of the whole run-time activation X (uint16, [M, K])."""
    M = wl.M if M is None else M
    return gen_x_rows(wl, 0, M, M)


def gen_calibration(wl: Workload) -> np.ndarray:
    """Calibration activations [n_cal, K], float64 values of bf16 numbers.

    Same law and outlier channels as the run-time rows, separate seed.
    """
    bits = _rows_bits(wl, wl.seed_cal, wl.n_cal, 0, wl.n_cal)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gen_weight(wl: Workload) -> np.ndarray:
    """Weight [d_out, K] (nn.Linear order), N(0, w_std) rounded through bf16."""
    rng = np.random.default_rng(wl.seed_w)
    w = rng.standard_normal((wl.d_out, wl.K)) * wl.w_std
    bits = f64_to_bf16_bits(w)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def iter_chunks(M: int, chunk: int = CHUNK) -> Iterable[Tuple[int, int]]:
    for lo in range(0, M, chunk):
        yield lo, min(M, lo + chunk)
