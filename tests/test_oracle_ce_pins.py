"""Pins of the oracle's cross-entropy (CPU only), none of which restates its formula: torch's own fp64
cross_entropy and logsumexp on torch's fp64 product, closed forms (uniform logits, hand-made logits with
known log-sum-exp), shift invariance, logits far beyond exp's range, and ignored rows."""
import math

import numpy as np
import pytest
import torch

import oracle


def _inputs(M, D, V, seed, ignore_every=0):
    rng = np.random.default_rng(seed)
    H = rng.standard_normal((M, D))
    W = rng.standard_normal((D, V)) * 0.5
    labels = rng.integers(0, V, size=M)
    if ignore_every:
        labels[::ignore_every] = -100
    return H, W, labels


def test_matches_torch_cross_entropy():
    H, W, labels = _inputs(37, 24, 301, seed=1, ignore_every=5)
    loss, lse = oracle.cross_entropy(H, W, labels)
    z = torch.tensor(H) @ torch.tensor(W)
    want = torch.nn.functional.cross_entropy(z, torch.tensor(labels), reduction="none", ignore_index=-100)
    np.testing.assert_allclose(loss, want.numpy(), rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=1e-13, atol=1e-13)
    assert np.all(loss[::5] == 0.0)


def test_uniform_logits_give_log_v():
    H, _, labels = _inputs(6, 8, 50, seed=2)
    loss, lse = oracle.cross_entropy(H, np.zeros((8, 50)), labels)
    np.testing.assert_allclose(lse, math.log(50), rtol=0, atol=1e-15)
    np.testing.assert_allclose(loss, math.log(50), rtol=0, atol=1e-15)


def test_hand_made_logits():
    # one row whose logits are (0, ln 2, ln 3): sum of exponentials 1 + 2 + 3 = 6
    H = np.array([[1.0]])
    W = np.array([[0.0, math.log(2.0), math.log(3.0)]])
    for label, want in [(0, math.log(6.0)), (1, math.log(3.0)), (2, math.log(2.0))]:
        loss, lse = oracle.cross_entropy(H, W, [label])
        np.testing.assert_allclose(lse, [math.log(6.0)], rtol=1e-15)
        np.testing.assert_allclose(loss, [want], rtol=1e-15)


def test_shift_invariance():
    """A constant c added to every logit (an extra hidden unit equal to 1 whose weights are all c) moves lse
    by c and leaves the loss unchanged."""
    H, W, labels = _inputs(9, 16, 70, seed=3)
    loss, lse = oracle.cross_entropy(H, W, labels)
    c = 7.25
    H2 = np.concatenate([H, np.ones((9, 1))], axis=1)
    W2 = np.concatenate([W, np.full((1, 70), c)], axis=0)
    loss2, lse2 = oracle.cross_entropy(H2, W2, labels)
    np.testing.assert_allclose(lse2, lse + c, rtol=1e-13)
    np.testing.assert_allclose(loss2, loss, rtol=1e-11, atol=1e-12)


def test_logits_beyond_exp_range():
    """Logits of 1000 overflow exp(); the log-sum-exp must still come out as 1000 + log(count of maxima)."""
    H = np.array([[1.0], [1.0]])
    W = np.array([[1000.0, 0.0, 1000.0, -5.0]])
    loss, lse = oracle.cross_entropy(H, W, [0, 1])
    assert np.all(np.isfinite(lse))
    np.testing.assert_allclose(lse, 1000.0 + math.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(loss, [math.log(2.0), 1000.0 + math.log(2.0)], rtol=1e-12)


def test_rejects_bad_labels():
    H, W, _ = _inputs(2, 4, 10, seed=4)
    with pytest.raises(RuntimeError):
        oracle.cross_entropy(H, W, [0, 10])
