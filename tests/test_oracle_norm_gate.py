"""Pins for the read epilogue oracle (RMS-Norm and output gate): closed forms,
invariances, and agreement with PyTorch's own rms_norm / silu / sigmoid in
float64 on the CPU, a library computation independent of the C code."""
import numpy as np
import pytest

import oracle

torch = pytest.importorskip("torch")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("act", ["none", "silu", "sigmoid"])
def test_matches_library_rms_norm_and_activations(act):
    y, g, gamma = _rand((3, 5, 40), 1), _rand((3, 5, 40), 2), _rand((40,), 3)
    eps = 1e-5
    ref = torch.nn.functional.rms_norm(torch.from_numpy(y).double(), (40,),
                                       torch.from_numpy(gamma).double(), eps)
    gt = torch.from_numpy(g).double()
    if act == "silu":
        ref = ref * torch.nn.functional.silu(gt)
    elif act == "sigmoid":
        ref = ref * torch.sigmoid(gt)
    got = oracle.norm_gate(y, None if act == "none" else g, gamma, eps, act)
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-13, atol=1e-15)


def test_constant_row_closed_form():
    # y = c 1: mean(y^2) = c^2, so o = c / sqrt(c^2 + eps) * gamma (mean, not sum, over d)
    gamma = np.array([0.5, -2.0, 3.0, 1.0], np.float32)
    for c, eps in ((1.0, 0.0), (-2.0, 0.0), (0.5, 0.25)):
        y = np.full((1, 4), c, np.float32)
        got = oracle.norm_gate(y, None, gamma, eps, "none")
        np.testing.assert_allclose(got[0], c / np.sqrt(c * c + eps) * gamma.astype(np.float64),
                                   rtol=1e-15)


def test_scale_invariance_without_eps_and_gate_values():
    y, g, gamma = _rand((6, 16), 4), _rand((6, 16), 5), _rand((16,), 6)
    a = oracle.norm_gate(y, g, gamma, 0.0, "silu")
    b = oracle.norm_gate(y * np.float32(8.0), g, gamma, 0.0, "silu")
    np.testing.assert_allclose(a, b, rtol=1e-14)
    # SiLU(0) = 0 and sigmoid(0) = 1/2; SiLU(1) = 1 / (1 + e^-1)
    zero = np.zeros_like(g)
    assert np.all(oracle.norm_gate(y, zero, gamma, 1e-6, "silu") == 0.0)
    np.testing.assert_allclose(oracle.norm_gate(y, zero, gamma, 1e-6, "sigmoid"),
                               0.5 * oracle.norm_gate(y, None, gamma, 1e-6, "none"), rtol=1e-15)
    one = np.ones_like(g)
    np.testing.assert_allclose(oracle.norm_gate(y, one, gamma, 1e-6, "silu"),
                               oracle.norm_gate(y, None, gamma, 1e-6, "none") / (1 + np.exp(-1.0)),
                               rtol=1e-14)
