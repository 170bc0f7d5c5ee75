"""Pins of the oracle's backward (CPU only): the gradients of the block are checked against things that do
not restate the oracle's chain rule.

- central finite differences of the pinned forward oracle (the loss sum(z * dz) + sum(h * dh_out), z the
  second product's output before the epilogue, so that dz and dh_out are its gradients);
- torch.autograd through torch's own fp64 composition of the block;
- closed properties: with eps = 0 the RMS normalisation is invariant to scaling h, so every row of dR is
  orthogonal to the row of h when dh_out = 0; the gradients are linear in (dz, dh_out); dh_out passes to dR
  unchanged and to dX through W1^T.
"""
import numpy as np
import pytest
import torch

import oracle

EPS = 1e-5


def _inputs(M, K1, D, N2, seed):
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K1))
    W1 = rng.standard_normal((K1, D)) / np.sqrt(K1)
    R = rng.standard_normal((M, D))
    g = rng.uniform(0.5, 1.5, D)
    W2 = rng.standard_normal((D, N2)) / np.sqrt(D)
    dz = rng.standard_normal((M, N2))
    dho = rng.standard_normal((M, D))
    return X, W1, R, g, W2, dz, dho


def _loss(X, W1, R, g, W2, dz, dho, eps):
    h, _, z = oracle.block_unfused(X, W1, R, g, W2, eps, oracle.EPI_IDENTITY, nthreads=1)
    return float(np.sum(z * dz) + np.sum(h * dho))


@pytest.mark.parametrize("eps", [EPS, 0.3])
def test_backward_matches_finite_differences(eps):
    X, W1, R, g, W2, dz, dho = _inputs(3, 4, 5, 6, seed=1)
    grads = oracle.block_bwd(X, W1, R, g, W2, eps, dz, dho, nthreads=1)
    args = [X, W1, R, g, W2]
    step = 1e-6
    for which, (a, grad) in enumerate(zip(args, [grads[0], grads[1], grads[2], grads[3], grads[4]])):
        fd = np.empty_like(a)
        for idx in np.ndindex(a.shape):
            keep = a[idx]
            a[idx] = keep + step
            lp = _loss(*args, dz, dho, eps)
            a[idx] = keep - step
            lm = _loss(*args, dz, dho, eps)
            a[idx] = keep
            fd[idx] = (lp - lm) / (2 * step)
        scale = max(1.0, np.max(np.abs(grad)))
        np.testing.assert_allclose(grad, fd, rtol=0, atol=2e-7 * scale, err_msg=f"input {which}")


def test_backward_matches_torch_autograd():
    X, W1, R, g, W2, dz, dho = _inputs(7, 16, 24, 10, seed=2)
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (X, W1, R, g, W2)]
    h = t[0] @ t[1] + t[2]
    n = torch.nn.functional.rms_norm(h, (h.shape[1],), t[3], eps=EPS)
    z = n @ t[4]
    loss = (z * torch.tensor(dz)).sum() + (h * torch.tensor(dho)).sum()
    loss.backward()
    ours = oracle.block_bwd(X, W1, R, g, W2, EPS, dz, dho)
    for name, a, b in zip(("dX", "dW1", "dR", "dgamma", "dW2"), ours, [x.grad.numpy() for x in t]):
        np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12, err_msg=name)


def test_rows_of_dR_orthogonal_to_h_when_eps_is_zero():
    X, W1, R, g, W2, dz, _ = _inputs(6, 8, 12, 9, seed=3)
    h, _, _ = oracle.block_unfused(X, W1, R, g, W2, 0.0, oracle.EPI_IDENTITY)
    _, _, dR, _, _ = oracle.block_bwd(X, W1, R, g, W2, 0.0, dz, None)
    dots = np.sum(dR * h, axis=1)
    assert np.max(np.abs(dots)) <= 1e-12 * np.max(np.abs(dR)) * np.max(np.abs(h)) * h.shape[1]
    # with eps > 0 the normalisation is no longer scale-invariant, so the rows are not orthogonal
    _, _, dR1, _, _ = oracle.block_bwd(X, W1, R, g, W2, 1.0, dz, None)
    assert np.max(np.abs(np.sum(dR1 * h, axis=1))) > 1e-3


def test_linear_in_incoming_gradients():
    X, W1, R, g, W2, dz, dho = _inputs(5, 8, 8, 6, seed=4)
    a = oracle.block_bwd(X, W1, R, g, W2, EPS, dz, dho)
    b = oracle.block_bwd(X, W1, R, g, W2, EPS, 2.0 * dz, None)
    c = oracle.block_bwd(X, W1, R, g, W2, EPS, -dz, 3.0 * dho)
    for x, y, w in zip(a, b, c):
        # a = G(dz, dho); b = G(2 dz, 0); c = G(-dz, 3 dho)  ->  a = b / 2 + (c + b / 2) / 3
        np.testing.assert_allclose(x, 0.5 * y + (w + 0.5 * y) / 3.0, rtol=1e-12, atol=1e-12)


def test_residual_gradient_path():
    """With dz = 0 only dh_out flows: dR = dh_out, dX = dh_out W1^T, dW1 = X^T dh_out, dgamma = dW2 = 0."""
    X, W1, R, g, W2, dz, dho = _inputs(4, 8, 12, 6, seed=5)
    dX, dW1, dR, dg, dW2 = oracle.block_bwd(X, W1, R, g, W2, EPS, np.zeros_like(dz), dho)
    assert np.array_equal(dR, dho)
    np.testing.assert_allclose(dX, dho @ W1.T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(dW1, X.T @ dho, rtol=1e-13, atol=1e-13)
    assert not np.any(dg) and not np.any(dW2)
