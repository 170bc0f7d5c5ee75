"""Pins of the oracle's rotary position embedding (CPU only), none of which restates its formula: torch's own
fp64 "rotate half" composition, and closed properties of rotations (pair norms preserved, position 0 and
columns past n_rot untouched, composition of positions adds angles, inner products of two rotated vectors
depend only on the difference of their positions)."""
import numpy as np
import pytest
import torch

import oracle

HD = 64


def _rand(M, N, seed):
    return np.random.default_rng(seed).standard_normal((M, N))


def test_matches_torch_rotate_half():
    M, N, nrot, seq, base = 10, 6 * HD, 4 * HD, 7, 500000.0
    y = _rand(M, N, 1)
    t = torch.tensor(y, dtype=torch.float64)
    pos = torch.arange(M, dtype=torch.float64) % seq
    inv = base ** (-torch.arange(0, HD, 2, dtype=torch.float64) / HD)
    ang = torch.outer(pos, inv)
    cos = torch.cat([ang.cos(), ang.cos()], dim=1)
    sin = torch.cat([ang.sin(), ang.sin()], dim=1)
    out = t.clone()
    for h0 in range(0, nrot, HD):
        x = t[:, h0:h0 + HD]
        rot = torch.cat([-x[:, HD // 2:], x[:, :HD // 2]], dim=1)
        out[:, h0:h0 + HD] = x * cos + rot * sin
    np.testing.assert_allclose(oracle.rope_rows(y, HD, nrot, seq, base), out.numpy(), rtol=1e-13, atol=1e-13)


def test_rotation_properties():
    M, N, nrot, seq, base = 9, 3 * HD, 2 * HD, 4, 10000.0
    y = _rand(M, N, 2)
    o = oracle.rope_rows(y, HD, nrot, seq, base)
    # columns past n_rot and rows at position 0 are untouched
    assert np.array_equal(o[:, nrot:], y[:, nrot:])
    assert np.array_equal(o[0::seq], y[0::seq])
    # every rotated pair keeps its norm
    for h0 in range(0, nrot, HD):
        a, b = y[:, h0:h0 + HD // 2], y[:, h0 + HD // 2:h0 + HD]
        oa, ob = o[:, h0:h0 + HD // 2], o[:, h0 + HD // 2:h0 + HD]
        np.testing.assert_allclose(oa ** 2 + ob ** 2, a ** 2 + b ** 2, rtol=1e-12)


def test_positions_compose_and_inner_products_are_relative():
    base, seq = 500000.0, 64
    q = _rand(1, HD, 3)
    k = _rand(1, HD, 4)
    # row m of a stack of copies sits at position m
    Q = np.repeat(q, seq, axis=0)
    K = np.repeat(k, seq, axis=0)
    rq = oracle.rope_rows(Q, HD, HD, seq, base)
    rk = oracle.rope_rows(K, HD, HD, seq, base)
    dots = rq @ rk.T  # dots[p1, p2] = <R(p1) q, R(p2) k>
    for d in (0, 3, 17):
        diag = np.array([dots[p, p + d] for p in range(seq - d)])
        np.testing.assert_allclose(diag, diag[0], rtol=1e-11, atol=1e-11)
    # rotating the position-5 result by 7 more positions gives the position-12 result
    r5 = rq[5:6]
    twice = oracle.rope_rows(np.repeat(r5, 8, axis=0), HD, HD, seq, base)[7]
    np.testing.assert_allclose(twice, rq[12], rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("bad", [dict(head_dim=63), dict(n_rot=100), dict(seq_len=0), dict(base=-1.0)])
def test_rejects_bad_arguments(bad):
    args = dict(head_dim=HD, n_rot=HD, seq_len=4, base=10000.0)
    args.update(bad)
    with pytest.raises(RuntimeError):
        oracle.rope_rows(_rand(2, 2 * HD, 5), **args)
