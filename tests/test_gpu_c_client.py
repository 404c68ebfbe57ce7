"""The C ABI used from a C++ program with no Python binding in the process.

tests/c_client/wush_client (built by __graft_entry__.build()) links
libwush.so, allocates device memory and a stream with plain HIP calls and
calls the per-format entry points of include/wush.h.  Its codes and scales
are held to the same bar as the binding's (tests/parity.py), against the
oracle on the same seeded inputs: scales bit-exact, codes within one level
at rounding ties.
"""

from __future__ import annotations

import os
import struct
import subprocess

import numpy as np
import pytest

from oracle import quant
from tests import cases, parity

pytestmark = pytest.mark.gpu

EXE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_client", "wush_client")
FMT_ID = {"mxfp4": 0, "nvfp4": 1, "int4": 2}


def _run(tmp_path, fmt, xb, tb, g_static=0.0):
    assert os.path.exists(EXE), "C client not built: run __graft_entry__.build()"
    M, K = xb.shape
    G = tb.shape[1]
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(b"WUSHCLI1" + struct.pack("<iiqqf", FMT_ID[fmt], G, M, K, g_static))
        f.write(np.ascontiguousarray(xb, dtype=np.uint16).tobytes())
        f.write(np.ascontiguousarray(tb, dtype=np.uint16).tobytes())
    print("client: %s M=%d K=%d G=%d g=%r" % (fmt, M, K, G, g_static), flush=True)
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, "client exit %d: %s" % (r.returncode, r.stderr)
    raw = out.read_bytes()
    assert raw[:8] == b"WUSHOUT1"
    (g_used,) = struct.unpack("<f", raw[8:12])
    n_codes = M * K // 2
    codes = np.frombuffer(raw, np.uint8, n_codes, 12).reshape(M, K // 2)
    sdt = np.uint16 if fmt == "int4" else np.uint8
    scales = np.frombuffer(raw, sdt, M * (K // G), 12 + n_codes).reshape(M, K // G)
    assert len(raw) == 12 + n_codes + scales.nbytes
    return codes, scales, np.float32(g_used)


@pytest.mark.parametrize("fmt,M,K", [("mxfp4", 128, 256), ("mxfp4", 77, 160), ("int4", 128, 256), ("int4", 45, 96),
                                     ("nvfp4", 128, 256), ("nvfp4", 33, 48)])
def test_client_matches_oracle(tmp_path, fmt, M, K):
    G = 16 if fmt == "nvfp4" else 32
    _, tb = cases.transforms("tiny_mxfp4", G)
    xb = cases.x_rows("tiny_mxfp4", 0, M)[:, :K]
    tb = tb[:K // G]
    codes, scales, g = _run(tmp_path, fmt, xb, tb)
    if fmt == "nvfp4":
        # The device computed the tensor scale (wush_nvfp4_global_scale): it
        # must be the oracle's, bit for bit.
        y = quant.transform_ref(xb, tb)
        g_ref = quant.nvfp4_global_scale(quant.tensor_amax_ref(y))
        assert g.view(np.uint32) == np.float32(g_ref).view(np.uint32), (g, g_ref)
    rep = parity.check(fmt, xb, tb, codes, scales, g=g if fmt == "nvfp4" else None)
    print(rep)


def test_client_nvfp4_static_scale(tmp_path):
    _, tb = cases.transforms("tiny_mxfp4", 16)
    xb = cases.x_rows("tiny_mxfp4", 0, 64)
    g = np.float32(0.0123)
    codes, scales, g_used = _run(tmp_path, "nvfp4", xb, tb, float(g))
    assert g_used == g
    parity.check("nvfp4", xb, tb, codes, scales, g=g)


def test_client_empty_batch(tmp_path):
    _, tb = cases.transforms("tiny_mxfp4")
    xb = np.zeros((0, 256), np.uint16)
    codes, scales, _ = _run(tmp_path, "mxfp4", xb, tb)
    assert codes.shape == (0, 128) and scales.shape == (0, 8)


def test_client_eq10_forward(tmp_path):
    """The whole forward from C: wush_quant_mxfp4_packed on the activations,
    wush_gemm_pack_b on MXFP4 weights, wush_gemm_mxfp4_packed.  C is
    compared with the oracle's quantize-then-multiply on the same inputs.
    At least 99% of the entries must lie within the fp32 accumulation bound,
    and every entry within it plus one E2M1 step of one activation element
    (a code that differs at a rounding tie moves a whole row of C)."""
    from oracle import gemm
    from synthetic.gemm_operands import gen_mx_operand

    assert os.path.exists(EXE), "C client not built: run __graft_entry__.build()"
    M, N, K = 200, 300, 512
    _, tb = cases.transforms("tiny_mxfp4", 32)
    tb = np.concatenate([tb, tb])  # 16 blocks for K = 512
    xb = np.concatenate([cases.x_rows("tiny_mxfp4", 0, 128), cases.x_rows("tiny_mxfp4", 0, 72)])
    xb = np.ascontiguousarray(np.concatenate([xb, xb], axis=1))
    wc, ws = gen_mx_operand(N, K, seed=77, scale_lo=118, scale_hi=126)
    inp, out = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(b"WUSHGEM1" + struct.pack("<qqq", M, N, K))
        for arr in (xb.astype(np.uint16), tb.astype(np.uint16), wc, ws):
            f.write(np.ascontiguousarray(arr).tobytes())
    print("client: gemm M=%d N=%d K=%d" % (M, N, K), flush=True)
    r = subprocess.run([EXE, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, "client exit %d: %s" % (r.returncode, r.stderr)
    raw = out.read_bytes()
    assert raw[:8] == b"WUSHOUTG" and len(raw) == 8 + 4 * M * N
    C = np.frombuffer(raw, np.float32, M * N, 8).reshape(M, N).astype(np.float64)
    ac, asc = quant.run_path("mxfp4", xb, tb)
    ref = gemm.gemm_mxfp4_ref(ac, asc, wc, ws)
    absref = gemm.gemm_mxfp4_abs_ref(ac, asc, wc, ws)
    err = np.abs(C - ref)
    tol = (K - 1) * 2.0**-24 * absref
    # One E2M1 step is at most 2 (between 4 and 6) times the block's scale.
    step_a = 2.0 * np.exp2(np.repeat(asc.astype(np.float64) - 127.0, 32, axis=1))  # [M][K]
    w = np.abs(quant.dequant_mxfp4(wc, ws))
    one_step = (step_a[:, None, :] * w[None, :, :]).max(axis=2)  # [M][N]
    inside = np.mean(err <= tol)
    print("entries within the fp32 bound: %.4f" % inside, flush=True)
    assert inside >= 0.99
    assert np.all(err <= tol + one_step)


def test_client_reports_bad_shape(tmp_path):
    # K not a multiple of G never reaches the library: the client rejects
    # the header.  A K the library rejects (MXFP4 needs K % 32 == 0 and the
    # client forwards it) is covered by tests/test_abi.py.
    assert os.path.exists(EXE), "C client not built: run __graft_entry__.build()"
    inp = tmp_path / "in.bin"
    inp.write_bytes(b"WUSHCLI1" + struct.pack("<iiqqf", 0, 32, 4, 40, 0.0))
    r = subprocess.run([EXE, str(inp), str(tmp_path / "out.bin")], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "bad input header" in r.stderr
