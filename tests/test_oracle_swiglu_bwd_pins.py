"""Pins of the oracle's SwiGLU backward (CPU only), none of which restates its formula: central finite
differences of the forward oracle's silu composition, torch.autograd through torch's silu, and closed forms
(a zero gate halves the up-gradient path: silu'(0) = 1/2, silu(0) = 0)."""
import numpy as np
import torch

import oracle


def _inputs(M, F, D, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((M, D)), rng.standard_normal((F, D)) / np.sqrt(D), rng.standard_normal((M, 2 * F)) * 2


def _loss(dout, Wd, z):
    F = Wd.shape[0]
    g, u = z[:, :F], z[:, F:]
    y = np.vectorize(oracle.silu)(g) * u
    return float(np.sum((y @ Wd) * dout))


def test_matches_finite_differences():
    dout, Wd, z = _inputs(3, 4, 5, seed=1)
    dz = oracle.swiglu_bwd(dout, Wd, z)
    step = 1e-6
    fd = np.empty_like(z)
    for idx in np.ndindex(z.shape):
        keep = z[idx]
        z[idx] = keep + step
        lp = _loss(dout, Wd, z)
        z[idx] = keep - step
        lm = _loss(dout, Wd, z)
        z[idx] = keep
        fd[idx] = (lp - lm) / (2 * step)
    np.testing.assert_allclose(dz, fd, rtol=0, atol=2e-7 * max(1.0, np.max(np.abs(dz))))


def test_matches_torch_autograd():
    dout, Wd, z = _inputs(6, 16, 24, seed=2)
    zt = torch.tensor(z, requires_grad=True)
    F = Wd.shape[0]
    y = torch.nn.functional.silu(zt[:, :F]) * zt[:, F:]
    (y @ torch.tensor(Wd)).backward(torch.tensor(dout))
    np.testing.assert_allclose(oracle.swiglu_bwd(dout, Wd, z), zt.grad.numpy(), rtol=1e-12, atol=1e-13)


def test_zero_gate():
    dout, Wd, z = _inputs(4, 8, 8, seed=3)
    F = 8
    z[:, :F] = 0.0
    dz = oracle.swiglu_bwd(dout, Wd, z)
    dy = dout @ Wd.T
    np.testing.assert_allclose(dz[:, :F], dy * z[:, F:] * 0.5, rtol=1e-13, atol=1e-14)
    assert not np.any(dz[:, F:])
