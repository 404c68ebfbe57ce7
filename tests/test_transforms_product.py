"""The product's batched torch transform builder against the oracle's
per-block NumPy construction (CPU)."""

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from mxfp4_activation_amd import transforms as pt  # noqa: E402
from oracle import transform as tr  # noqa: E402
from synthetic import CONFIGS, gen_calibration, gen_weight  # noqa: E402


@pytest.mark.parametrize("G", [16, 32])
def test_matches_oracle(G):
    wl = CONFIGS["tiny_mxfp4"]
    W, Xc = gen_weight(wl), gen_calibration(wl)
    Tw_ref, Tx_ref = tr.build_transforms(W, Xc, G)
    Tw, Tx = pt.wush_transforms(torch.from_numpy(W), torch.from_numpy(Xc), G)
    np.testing.assert_allclose(Tw.numpy(), Tw_ref, rtol=1e-8, atol=1e-10)
    np.testing.assert_allclose(Tx.numpy(), Tx_ref, rtol=1e-8, atol=1e-10)
    bf = pt.to_kernel_layout(Tw).view(torch.int16).numpy().view(np.uint16)
    ref = tr.transforms_to_bf16_bits(Tw_ref)
    assert np.mean(bf == ref) > 0.999  # float64 noise can flip a rare rounding tie


def test_wus_variant_and_banks():
    wl = CONFIGS["tiny_mxfp4"]
    W, Xc = gen_weight(wl), gen_calibration(wl)
    Tw, Tx = pt.wush_transforms(torch.from_numpy(W), torch.from_numpy(Xc), 32, use_hadamard=False)
    eye = torch.eye(32, dtype=torch.float64)
    assert torch.allclose(Tx.transpose(1, 2) @ Tw, eye.expand_as(Tw), atol=1e-8)
    H = pt.hadamard_transforms(8, 32)
    assert torch.allclose(H[3] @ H[3].T, eye, atol=1e-14)
    assert torch.equal(pt.identity_transforms(2, 16)[1], torch.eye(16, dtype=torch.float64))
