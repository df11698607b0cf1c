"""Pins of the oracle's residual add + RMSNorm (oracle/norm.py) against what
the definition and the mathematics fix: torch's own rms_norm (an independent
library routine) in fp64, closed forms and invariants.  Each pin fails under
a plausible mistake in the oracle: a sum instead of the mean, eps outside
the root, a dropped weight, a dropped residual, the root left out."""
import math

import numpy as np
import pytest
import torch

from oracle import mx, norm


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


@pytest.mark.parametrize("T,H,eps", [(3, 64, 1e-6), (5, 4096, 1e-5), (1, 32, 0.5)])
def test_matches_torch_rms_norm(T, H, eps):
    x, r, w = _rand((T, H), 1), _rand((T, H), 2), 1.0 + _rand((H,), 3, 0.1)
    z, y = norm.add_rmsnorm(x, r, w, eps)
    zt = torch.from_numpy(x) + torch.from_numpy(r)
    yt = torch.nn.functional.rms_norm(zt, (H,), weight=torch.from_numpy(w), eps=eps)
    np.testing.assert_array_equal(z, zt.numpy())
    np.testing.assert_allclose(y, yt.numpy(), rtol=1e-12, atol=1e-14)


def test_constant_row_closed_form():
    """A row of equal values c normalises to sign(c) * w (eps 0)."""
    H = 48
    x = np.array([[3.0] * H, [-0.25] * H])
    w = 1.0 + _rand((H,), 4, 0.1)
    _, y = norm.add_rmsnorm(x, None, w, 0.0)
    np.testing.assert_allclose(y[0], w, rtol=1e-15)
    np.testing.assert_allclose(y[1], -w, rtol=1e-15)


def test_one_hot_row_closed_form():
    """One nonzero element a in a row of d: mean(z^2) = a^2 / d, so the
    element becomes sqrt(d) * sign(a) (eps 0) and the rest stay 0."""
    H = 64
    x = np.zeros((1, H))
    x[0, 5] = -7.5
    _, y = norm.add_rmsnorm(x, None, np.ones(H), 0.0)
    assert y[0, 5] == pytest.approx(-math.sqrt(H), rel=1e-15)
    assert np.all(np.delete(y[0], 5) == 0.0)


def test_unit_mean_square_and_eps():
    """w = 1: mean(y^2) = ms / (ms + eps) per row, ms = mean(z^2)."""
    x, r = _rand((4, 256), 5), _rand((4, 256), 6)
    for eps in (0.0, 1e-6, 0.3):
        z, y = norm.add_rmsnorm(x, r, np.ones(256), eps)
        ms = np.mean(z * z, axis=1)
        np.testing.assert_allclose(np.mean(y * y, axis=1), ms / (ms + eps), rtol=1e-13)


def test_scale_invariance():
    """eps 0: scaling a row by c > 0 leaves y unchanged."""
    x = _rand((2, 128), 7)
    w = 1.0 + _rand((128,), 8, 0.1)
    _, y1 = norm.add_rmsnorm(x, None, w, 0.0)
    _, y2 = norm.add_rmsnorm(x * 37.0, None, w, 0.0)
    np.testing.assert_allclose(y1, y2, rtol=1e-14)


def test_residual_is_added():
    """A residual of zeros is the first-layer form; a residual equal to x
    doubles z (and, eps 0, leaves y unchanged)."""
    x = _rand((3, 96), 9)
    w = 1.0 + _rand((96,), 10, 0.1)
    z0, y0 = norm.add_rmsnorm(x, None, w, 1e-6)
    z1, y1 = norm.add_rmsnorm(x, np.zeros_like(x), w, 1e-6)
    np.testing.assert_array_equal(z0, z1)
    np.testing.assert_array_equal(y0, y1)
    z2, y2 = norm.add_rmsnorm(x, x, w, 0.0)
    np.testing.assert_array_equal(z2, 2 * x)
    _, y3 = norm.add_rmsnorm(x, None, w, 0.0)
    np.testing.assert_allclose(y2, y3, rtol=1e-14)


def test_bf16_sum_is_exact_in_fp64():
    """bf16 inputs: z = x + r is exact in fp64, so rounding it to bf16 once
    gives the correctly rounded residual (the value the GPU must match)."""
    g = torch.Generator().manual_seed(11)
    x = torch.randn((8, 512), generator=g).to(torch.bfloat16)
    r = (torch.randn((8, 512), generator=g) * 300).to(torch.bfloat16)
    z, _ = norm.add_rmsnorm(x.double().numpy(), r.double().numpy(), np.ones(512), 1e-6)
    want = (x.float() + r.float()).to(torch.bfloat16).double().numpy()  # fp32 add, then RNE
    np.testing.assert_array_equal(mx.bf16_round(z), want)
