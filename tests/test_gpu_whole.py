"""Whole-tensor parity at the full workload sizes, in the launch
configuration the benchmark times.

Every row of the Llama-3.1-8B-shaped, down-projection, NVFP4 and INT4
workloads (4096 x 4096, 8192 x 14336, 16384 x 4096, 65536 x 8192) is compared
with the oracle, 4096 rows at a time, to the bar in tests/parity.py: scales
bit for bit, codes at most one level apart and only within the accumulation
bound of a rounding midpoint, at most 1e-4 of them.  The kernel runs once
per workload on the whole tensor; its outputs are kept for the row ranges
that follow.  The NVFP4 tensor scale is checked twice: the oracle's g fed to
the quantizer, and the device's own g (the AbsMax pre-pass) end to end.
"""

import functools

import numpy as np
import pytest

from oracle import quant
from synthetic import CONFIGS

from . import cases, parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CHUNK = 4096


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()  # raises if libwush.so is missing: no fallback
    yield


def _dev_bf16(bits: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@functools.lru_cache(maxsize=2)
def _gpu_outputs(name: str, dynamic_g: bool = False):
    """(codes, scales, exact groups, g) of one kernel pass over the whole
    tensor.  NVFP4 takes the oracle's g, or with dynamic_g the device's own
    (wush_nvfp4_global_scale on the same tensor, in the same stream)."""
    from mxfp4_activation_amd import ops

    wl = CONFIGS[name]
    _, tb = cases.transforms(name)
    xb = cases.x_full(name)
    X, T = _dev_bf16(xb), _dev_bf16(tb)
    gs, g = None, None
    if wl.fmt == "nvfp4":
        if dynamic_g:
            gs = ops.nvfp4_global_scale(X, T)
        else:
            gs = torch.tensor([cases.oracle_global_scale(name)], dtype=torch.float32, device="cuda")
    ne = torch.zeros(1, dtype=torch.int32, device="cuda")
    codes, scales = ops.quant(wl.fmt, X, T, global_scale=gs, n_exact=ne)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    s = scales.cpu().numpy()
    if wl.fmt == "int4":
        s = s.view(np.uint16)
    if gs is not None:
        g = np.float32(gs.item())
    del X, T, codes, scales
    torch.cuda.empty_cache()
    return c, s, int(ne.item()), g


def _check_rows(name, lo, hi, g, c, s):
    wl = CONFIGS[name]
    _, tb = cases.transforms(name)
    xb = cases.x_full(name)
    tot = parity.ParityReport(0, 0, 0, 0.0, 0)
    for a in range(lo, hi, CHUNK):
        b = min(hi, a + CHUNK)
        rep = parity.check(wl.fmt, xb[a:b], tb, c[a:b], s[a:b], g)
        tot.n_codes += rep.n_codes
        tot.n_mismatch += rep.n_mismatch
        tot.n_groups += rep.n_groups
        tot.max_level_diff = max(tot.max_level_diff, rep.max_level_diff)
        tot.worst_margin = max(tot.worst_margin, rep.worst_margin)
        print("  rows %d..%d: %d code mismatches" % (a, b, rep.n_mismatch), flush=True)
    assert tot.frac <= 1e-4
    return tot


# (workload, first row, last row): INT4's 65536 rows are checked in four
# parts so that each part stays well inside a test's time limit.
_PARTS = [("llama8b_mxfp4", 0, None), ("downproj_mxfp4", 0, None), ("nvfp4", 0, None)] + \
    [("int4", p * 16384, (p + 1) * 16384) for p in range(4)]


@pytest.mark.parametrize("name,lo,hi", _PARTS)
def test_whole_tensor(name, lo, hi):
    wl = CONFIGS[name]
    hi = wl.M if hi is None else hi
    print("case", name, wl.M, wl.K, "rows", lo, hi, flush=True)
    g = cases.oracle_global_scale(name) if wl.fmt == "nvfp4" else None
    c, s, n_exact, _ = _gpu_outputs(name)
    rep = _check_rows(name, lo, hi, g, c, s)
    print("PARITY %s rows %d..%d: groups %d, codes %d, mismatches %d (%.2e), max level diff %d, worst margin %.3f; "
          "exact groups in the whole launch %d of %d" % (name, lo, hi, rep.n_groups, rep.n_codes, rep.n_mismatch,
                                                        rep.frac, rep.max_level_diff, rep.worst_margin, n_exact,
                                                        wl.M * (wl.K // wl.G)), flush=True)


def test_nvfp4_dynamic_scale_end_to_end():
    """The NVFP4 step with its own tensor scale: the device's AbsMax pre-pass
    gives g, the quantizer uses it, and the whole 16384 x 4096 output matches
    the oracle's path (the oracle's exact tensor AbsMax, its g, its
    quantizer).  g must match bit for bit for the scales to."""
    name = "nvfp4"
    g_ref = cases.oracle_global_scale(name)
    c, s, _, g = _gpu_outputs(name, dynamic_g=True)
    print("device g %r (bits %08x), oracle g %r (bits %08x)"
          % (g, g.view(np.uint32), g_ref, g_ref.view(np.uint32)), flush=True)
    assert g.view(np.uint32) == g_ref.view(np.uint32)
    rep = _check_rows(name, 0, CONFIGS[name].M, g_ref, c, s)
    print("PARITY nvfp4 dynamic g: codes %d, mismatches %d" % (rep.n_codes, rep.n_mismatch), flush=True)
    assert quant.nvfp4_global_scale(cases.oracle_tensor_amax(name)).view(np.uint32) == g_ref.view(np.uint32)
