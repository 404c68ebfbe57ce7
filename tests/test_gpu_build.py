"""GPU parity of the offline transform construction (wush_build_transforms).

The kernel builds T_wush and T_xvsh in float64 (moments, damping, Cholesky,
one-sided Jacobi SVD, sign rule, products).  It is compared with
oracle.transform, which uses LAPACK's SVD, on the same bf16 inputs:
  * float64 T per block within 1e-9 of the oracle's, relative to the block's
    largest entry (both are float64 computations of the same closed form;
    the singular vectors differ only in rounding);
  * T_xvsh^T T_wush = I on the GPU output;
  * the bf16(fp32(T)) copies equal the oracle's bits except where the
    float64 value sits at a rounding boundary (at most one bf16 ulp, and
    rarely);
  * determinism, ragged row counts, G = 16 and the WUS variant;
  * rank-deficient moments (fewer rows than G), where T is not unique, by
    the invariants the pages fix.
"""

import numpy as np
import pytest

from oracle import transform as tr
from synthetic import CONFIGS, f64_to_bf16_bits, gen_calibration, gen_weight
from synthetic.layers import gen_linear_layer

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    import mxfp4_activation_amd as wush

    wush.load()
    yield


def _dev_bf16(a):
    return torch.from_numpy(np.ascontiguousarray(f64_to_bf16_bits(a)).view(np.int16)).cuda().view(torch.bfloat16)


def _check(W, Xc, G, use_h=True, tol=1e-9):
    from mxfp4_activation_amd import ops

    H = None if use_h else np.eye(G)
    ref_w, ref_x = tr.build_transforms(W, Xc, G, H=H)
    tw, tx, bw, bx = ops.build_transforms(_dev_bf16(W), _dev_bf16(Xc), G, use_hadamard=use_h)
    torch.cuda.synchronize()
    tw, tx = tw.cpu().numpy(), tx.cpu().numpy()
    for got, ref in ((tw, ref_w), (tx, ref_x)):
        scale = np.abs(ref).max(axis=(1, 2), keepdims=True)
        err = np.abs(got - ref) / scale
        assert err.max() < tol, err.max()
    ident = np.matmul(tx.transpose(0, 2, 1), tw)
    assert np.abs(ident - np.eye(G)).max() < 1e-9
    for got_b, ref in ((bw, ref_w), (bx, ref_x)):
        gb = got_b.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.int64)
        rb = tr.transforms_to_bf16_bits(ref).astype(np.int64)
        d = np.abs(gb - rb)
        assert d.max() <= 1 and (d > 0).mean() <= 1e-3, (d.max(), (d > 0).mean())
    return tw, tx


def test_tiny_workload_g32():
    wl = CONFIGS["tiny_mxfp4"]
    _check(gen_weight(wl), gen_calibration(wl), 32)


def test_tiny_workload_g16_and_wus():
    wl = CONFIGS["tiny_mxfp4"]
    _check(gen_weight(wl), gen_calibration(wl), 16)
    _check(gen_weight(wl), gen_calibration(wl), 32, use_h=False)


def test_headline_layer():
    wl = CONFIGS["llama8b_mxfp4"]
    _check(gen_weight(wl), gen_calibration(wl), 32)


def test_ragged_row_counts():
    W, Xc, _ = gen_linear_layer(128, 100, 77, 1, seed=5, n_outlier=1)
    _check(W, Xc, 32)


@pytest.mark.parametrize("d_out,n_cal", [(1, 1), (3, 65)])
def test_rank_deficient_moments_keep_the_invariants(d_out, n_cal):
    """Fewer rows than G: the damped moments have repeated eigenvalues, so the
    singular vectors (and T) are not unique.  What the pages fix still holds:
    T_xvsh^T T_wush = I, and both sides equalize to the same H S H^T with a
    constant diagonal (deep dive, section 3.4.4)."""
    from mxfp4_activation_amd import ops

    W, Xc, _ = gen_linear_layer(128, d_out, n_cal, 1, seed=d_out + n_cal, n_outlier=1)
    tw, tx, _, _ = ops.build_transforms(_dev_bf16(W), _dev_bf16(Xc), 32)
    torch.cuda.synchronize()
    tw, tx = tw.cpu().numpy(), tx.cpu().numpy()
    assert np.isfinite(tw).all() and np.isfinite(tx).all()
    Sw, Sx = tr.block_moments(W, Xc, 32)
    Sw, Sx = tr.damp(Sw, tr.DEFAULT_DAMP), tr.damp(Sx, tr.DEFAULT_DAMP)
    for c in range(tw.shape[0]):
        assert np.abs(tx[c].T @ tw[c] - np.eye(32)).max() < 1e-6
        A = tw[c] @ Sx[c] @ tw[c].T
        B = tx[c] @ Sw[c] @ tx[c].T
        assert np.abs(A - B).max() < 1e-6 * np.abs(A).max()
        d = np.diag(A)
        assert np.abs(d - d.mean()).max() < 1e-6 * d.mean()


def test_deterministic():
    from mxfp4_activation_amd import ops

    wl = CONFIGS["tiny_mxfp4"]
    W, Xc = _dev_bf16(gen_weight(wl)), _dev_bf16(gen_calibration(wl))
    a = ops.build_transforms(W, Xc, 32)
    b = ops.build_transforms(W, Xc, 32)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
