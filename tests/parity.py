"""Parity checker: GPU (codes, scales) against the oracle, element by element.

Bar, per format:
  * Scales must match bit for bit, every byte or every fp16 pattern.
  * Codes are compared as positions in the ordered level set, so +0 and -0
    count as the same level.  A code may differ only by one level.  It may
    differ only where the oracle's scaled value lies within the kernel's
    accumulation error bound of a rounding midpoint.  No more than 1e-4 of
    all codes may differ.
The error bound comes from the arithmetic.  The kernel's fp32 matrix-core sum
is within 2^-17 * sum_j |T_kj x_j| + 2^-21 * |y_k| of the exact sum.  The
scaled value carries that bound times the scale multiplier, plus two fp32
ulps for the multiply.
"""

from __future__ import annotations

import dataclasses

import numpy as np

from oracle import codecs, quant

E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
INT4_MIDS = np.arange(7) + 0.5  # 0.5 .. 6.5


@dataclasses.dataclass
class ParityReport:
    n_codes: int
    n_mismatch: int
    max_level_diff: int
    worst_margin: float  # max over mismatches of (distance to midpoint / window); <= 1 passes
    n_groups: int

    @property
    def frac(self) -> float:
        return self.n_mismatch / max(1, self.n_codes)


def _level(fmt, nib):
    if fmt == "int4":
        return codecs.int4_decode(nib)
    return codecs.e2m1_level_index(nib)


def _scaled(fmt, y, g, G):
    """Oracle scale codes, scaled values v and the per-element multiplier."""
    M, K = y.shape
    if fmt == "mxfp4":
        sc, v = quant.scaled_mxfp4(y, G)
        mul = np.ldexp(1.0, 127 - sc.astype(np.int64))
    elif fmt == "nvfp4":
        sc, v = quant.scaled_nvfp4(y, g, G)
        eff = (codecs.e4m3_value(sc).astype(np.float32) * np.float32(g)).astype(np.float32)
        with np.errstate(divide="ignore"):
            mul = np.where(eff > 0, np.float32(1.0) / eff, np.float32(0.0)).astype(np.float64)
    else:
        sc, v = quant.scaled_int4(y, G)
        s = codecs.f16_bits_to_f32(sc)
        with np.errstate(divide="ignore"):
            mul = np.where(s > 0, np.float32(1.0) / s, np.float32(0.0)).astype(np.float64)
    return sc, v, np.repeat(mul, G, axis=1)


def check(fmt: str, x_bits: np.ndarray, t_bits: np.ndarray, codes_gpu: np.ndarray, scales_gpu: np.ndarray,
          g=None, max_frac: float = 1e-4) -> ParityReport:
    """Compare GPU outputs for the rows in x_bits against the oracle."""
    G = t_bits.shape[1]
    y, A = quant.transform_ref(x_bits, t_bits, return_abs=True)
    if fmt == "nvfp4" and g is None:
        g = quant.nvfp4_global_scale(quant.tensor_amax_ref(y))
    sc_ref, v, mul = _scaled(fmt, y, g, G)
    if fmt == "mxfp4":
        codes_ref = codecs.pack_nibbles(codecs.e2m1_encode(v))
    elif fmt == "nvfp4":
        codes_ref = codecs.pack_nibbles(codecs.e2m1_encode(v))
    else:
        codes_ref = codecs.pack_nibbles(quant.int4_round(v))
        sc_ref = sc_ref.view(np.uint16)
        scales_gpu = np.asarray(scales_gpu).view(np.uint16)

    bad_sc = np.argwhere(np.asarray(scales_gpu) != sc_ref)
    if bad_sc.size:
        m, c = bad_sc[0]
        grp = y[m, c * G:(c + 1) * G]
        raise AssertionError(
            "%s: %d scale mismatches of %d; first at token %d block %d: gpu %r ref %r (group amax %r)"
            % (fmt, len(bad_sc), sc_ref.size, m, c, scales_gpu[m, c], sc_ref[m, c], np.abs(grp).max()))

    lg = _level(fmt, codecs.unpack_nibbles(codes_gpu))
    lr = _level(fmt, codecs.unpack_nibbles(codes_ref))
    diff = lg - lr
    idx = np.argwhere(diff != 0)
    rep = ParityReport(int(lg.size), int(len(idx)), int(np.abs(diff).max()) if len(idx) else 0, 0.0,
                       int(sc_ref.size))
    if len(idx) == 0:
        return rep
    if rep.max_level_diff > 1:
        m, k = idx[np.argmax(np.abs(diff[tuple(idx.T)]))]
        raise AssertionError("%s: code off by %d levels at token %d channel %d (y=%r)"
                             % (fmt, rep.max_level_diff, m, k, y[m, k]))
    mids = INT4_MIDS if fmt == "int4" else E2M1_MIDS
    vv = np.abs(v[tuple(idx.T)].astype(np.float64))
    dist = np.min(np.abs(vv[:, None] - mids[None, :]), axis=1)
    w = ((2.0 ** -17) * A[tuple(idx.T)] + (2.0 ** -21) * np.abs(y[tuple(idx.T)])) * mul[tuple(idx.T)]
    w = w + 2.0 * np.spacing(np.float32(np.maximum(vv, 1e-30))).astype(np.float64)
    ratio = dist / w
    rep.worst_margin = float(ratio.max())
    if rep.worst_margin > 1.0:
        j = int(np.argmax(ratio))
        m, k = idx[j]
        raise AssertionError("%s: code mismatch away from a rounding midpoint at token %d channel %d: "
                             "v=%r, distance %g > window %g" % (fmt, m, k, v[m, k], dist[j], w[j]))
    if rep.frac > max_frac:
        raise AssertionError("%s: %d code mismatches (%.2e) exceed %g" % (fmt, rep.n_mismatch, rep.frac, max_frac))
    return rep
