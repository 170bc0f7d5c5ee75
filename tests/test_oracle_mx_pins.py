"""Pins of the oracle's block-scaled (MX-style) e4m3 quantiser (CPU only), none of which restates its rule:
torch's log2/ceil and float8_e4m3fn cast on the same values, closed forms at the binade edges of 448, the
round-trip error of e4m3 (unit roundoff 2^-4), the top binade being used, and block independence."""
import numpy as np
import pytest
import torch

import oracle


def _torch_reference(x: np.ndarray, block: int):
    """torch: e = ceil(log2(amax / 448)) per block (0 for amax = 0), codes = (x / 2^e) cast to e4m3fn."""
    t = torch.tensor(x, dtype=torch.float64)
    rows, cols = t.shape
    b = t.view(rows, cols // block, block)
    amax = b.abs().amax(dim=2)
    e = torch.where(amax > 0, torch.ceil(torch.log2(amax / 448.0)), torch.zeros_like(amax))
    q = (b / torch.pow(2.0, e).unsqueeze(2)).to(torch.float8_e4m3fn).view(torch.uint8).view(rows, cols)
    return q.numpy(), e.to(torch.int32).numpy()


def test_matches_torch():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((24, 256)) * np.exp(rng.uniform(-8, 8, size=(24, 1)))
    x[3, 32:64] = 0.0  # an all-zero block
    codes, exps = oracle.mx_quant_rows_e4m3(x, 32)
    tq, te = _torch_reference(x, 32)
    assert np.array_equal(exps, te)
    assert np.array_equal(codes, tq)
    assert exps[3, 1] == 0 and not codes[3, 32:64].any()


@pytest.mark.parametrize("amax,want", [(448.0, 0), (448.0 * (1 + 2 ** -40), 1), (449.0, 1), (1.0, -8), (1.75, -8),
                                       (1.7500001, -7), (224.0, -1), (3.5, -7), (0.0, 0), (2.0 ** -200, -127),
                                       (2.0 ** 200, 127)])
def test_scale_exponent_closed_forms(amax, want):
    assert oracle.mx_scale_exp(amax) == want


def test_round_trip_and_top_binade():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((16, 128)) * 3.0
    codes, exps = oracle.mx_quant_rows_e4m3(x, 32)
    dq = oracle.e4m3_decode(codes) * np.ldexp(1.0, np.repeat(exps, 32, axis=1))
    big = np.abs(x) >= np.ldexp(1.0, np.repeat(exps, 32, axis=1) - 6)  # normal range of e4m3 after scaling
    assert np.all(np.abs(dq - x)[big] <= 2.0 ** -4 * np.abs(x)[big])
    # the largest value of every block lands in the top binade (224, 448]
    scaled_max = np.abs(x).reshape(16, 4, 32).max(axis=2) / np.ldexp(1.0, exps)
    assert np.all(scaled_max > 224.0) and np.all(scaled_max <= 448.0)


def test_blocks_are_independent():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 96))
    c1, e1 = oracle.mx_quant_rows_e4m3(x, 32)
    y = x.copy()
    y[:, 32:64] *= 1000.0
    c2, e2 = oracle.mx_quant_rows_e4m3(y, 32)
    assert np.array_equal(c1[:, :32], c2[:, :32]) and np.array_equal(c1[:, 64:], c2[:, 64:])
    assert np.array_equal(e1[:, [0, 2]], e2[:, [0, 2]])
    # a block 1000 times larger moves its exponent by 9 or 10 (log2 1000 = 9.97)
    assert np.all((e2[:, 1] - e1[:, 1] >= 9) & (e2[:, 1] - e1[:, 1] <= 10))


def test_rejects_ragged_blocks():
    with pytest.raises(RuntimeError):
        oracle.mx_quant_rows_e4m3(np.zeros((2, 40)), 32)
