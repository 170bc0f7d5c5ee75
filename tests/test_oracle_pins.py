"""Pins of the fp64 CPU oracle to things other than itself (no GPU needed).

Each test ties one part of the oracle to a closed form, an invariant of the mathematics, an exhaustive code
table or an independent library routine, chosen so that a dropped term, a wrong sign or index, a misplaced
eps or a transposed operand fails at least one of them.  The block follows the CODA write-up ("CODA: new
research optimizes Transformer training with GEMM-epilogue programming"), section "CODA: the treasure hidden
in the epilogue".
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_block(rng, M, K1, D, N2, gamma=True):
    X = rng.standard_normal((M, K1))
    W1 = rng.standard_normal((K1, D)) / math.sqrt(K1)
    R = rng.standard_normal((M, D))
    g = rng.uniform(0.5, 1.5, D) if gamma else np.ones(D)
    W2 = rng.standard_normal((D, N2)) / math.sqrt(D)
    return X, W1, R, g, W2


def _normwise(a, b):
    return np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300)


# --- closed forms -------------------------------------------------------------------------------------

def test_closed_form_golden_cases():
    """Hand-derived cases (tests/golden/closed_form_block.json) hit exactly, in both orders."""
    with open(os.path.join(GOLDEN, "closed_form_block.json")) as f:
        cases = json.load(f)["cases"]
    assert len(cases) >= 5
    for c in cases:
        epi = oracle.EPI_IDENTITY if c["epi"] == "identity" else oracle.EPI_SWIGLU
        args = [np.array(c[k], dtype=np.float64) for k in ("X", "W1", "R", "gamma", "W2")]
        if "y" in c:
            y_want = np.array(c["y"], dtype=np.float64)
        else:
            y_want = np.array([[eval(e, {"exp": math.exp}) for e in c["y_expr"]]])
        for fn in (oracle.block_unfused, oracle.block_fused):
            h, r, y = fn(*args, c["eps"], epi)
            np.testing.assert_allclose(h, np.array(c["h"], dtype=np.float64), rtol=0, atol=1e-15, err_msg=c["name"])
            np.testing.assert_allclose(r, np.array(c["r"]), rtol=1e-15, atol=0, err_msg=c["name"])
            np.testing.assert_allclose(y, y_want, rtol=1e-14, atol=1e-15, err_msg=c["name"])


def test_rms_scale_closed_form():
    h = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0], [0.0, 0.0, 0.0, 2.0]])
    r = oracle.rms_scale(h, 0.0)
    np.testing.assert_allclose(r, [0.4, 1.0, 1.0], rtol=1e-15)
    r = oracle.rms_scale(h, 3.0)  # eps inside the square root
    np.testing.assert_allclose(r, [1 / math.sqrt(6.25 + 3), 0.5, 0.5], rtol=1e-15)


def test_rms_from_partials_equals_full_row():
    """Partial sums of squares over column tiles, merged, give the full-row scale (the "light reduction"
    of the write-up's epilogue section)."""
    rng = np.random.default_rng(7)
    h = rng.standard_normal((37, 96))
    for T in (1, 2, 3, 6, 96):
        tiles = np.split(h, T, axis=1)
        part = np.stack([np.sum(t * t, axis=1) for t in tiles])  # [T, M]
        r = oracle.rms_from_partials(part, 96, 1e-5)
        np.testing.assert_allclose(r, oracle.rms_scale(h, 1e-5), rtol=1e-14)
    # closed form: two tiles holding 9 and 16 for a row of width 4 -> mean 25/4 -> r = 0.4
    np.testing.assert_allclose(oracle.rms_from_partials(np.array([[9.0], [16.0]]), 4, 0.0), [0.4], rtol=1e-15)


# --- library special cases -----------------------------------------------------------------------------

@pytest.mark.parametrize("epi", [oracle.EPI_IDENTITY, oracle.EPI_SWIGLU])
@pytest.mark.parametrize("shape", [(5, 16, 8, 12), (33, 24, 40, 64), (1, 8, 8, 2)])
def test_against_torch_rms_norm_and_silu(epi, shape):
    """y = epi(rms_norm(X W1 + R; gamma, eps) W2) built from torch's own rms_norm, addmm and silu in fp64."""
    M, K1, D, N2 = shape
    rng = np.random.default_rng(sum(shape) + epi)
    X, W1, R, g, W2 = _rand_block(rng, M, K1, D, N2)
    eps = 1e-3
    tX, tW1, tR, tg, tW2 = (torch.from_numpy(a) for a in (X, W1, R, g, W2))
    h_t = torch.addmm(tR, tX, tW1)
    z_t = F.rms_norm(h_t, (D,), weight=tg, eps=eps) @ tW2
    if epi == oracle.EPI_SWIGLU:
        z_t = F.silu(z_t[:, : N2 // 2]) * z_t[:, N2 // 2:]
    for fn in (oracle.block_unfused, oracle.block_fused):
        h, r, y = fn(X, W1, R, g, W2, eps, epi)
        assert _normwise(h, h_t.numpy()) < 1e-14
        assert _normwise(y, z_t.numpy()) < 1e-12
    # the row scale itself against torch: rms_norm with unit weight is h * r
    np.testing.assert_allclose(h * r[:, None], F.rms_norm(h_t, (D,), eps=eps).numpy(), rtol=1e-12, atol=1e-14)


def test_gemm_residual_against_matmul():
    rng = np.random.default_rng(3)
    X, W1, R, _, _ = _rand_block(rng, 19, 40, 24, 8)
    h = oracle.gemm_residual(X, W1, R)
    np.testing.assert_allclose(h, X @ W1 + R, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(oracle.gemm_residual(X, W1), X @ W1, rtol=1e-13, atol=1e-13)


def test_silu_against_torch():
    xs = np.concatenate([np.linspace(-30, 30, 241), [0.0, -1e-8, 1e-8, 80.0, -80.0]])
    ref = F.silu(torch.from_numpy(xs)).numpy()
    got = np.array([oracle.silu(x) for x in xs])
    np.testing.assert_allclose(got, ref, rtol=1e-15, atol=1e-300)


# --- invariants -----------------------------------------------------------------------------------------

@pytest.mark.parametrize("epi", [oracle.EPI_IDENTITY, oracle.EPI_SWIGLU])
def test_fused_and_unfused_forms_agree(epi):
    """Moving r past the second product is exact algebra: the two fp64 orders agree to 1e-9 normwise."""
    for shape in [(7, 32, 16, 48), (64, 256, 256, 512), (3, 8, 64, 128)]:
        rng = np.random.default_rng(shape[0] * 1000 + shape[2])
        args = _rand_block(rng, *shape)
        _, _, yu = oracle.block_unfused(*args, 1e-5, epi)
        _, _, yf = oracle.block_fused(*args, 1e-5, epi)
        assert _normwise(yf, yu) < 1e-9


@pytest.mark.parametrize("eps", [1e-6, 0.5, 4.0])
def test_unit_gamma_identity_w2_row_rms(eps):
    """gamma = 1, W2 = I, identity epilogue: RMS(y_i) = 1 / sqrt(1 + eps / mean(h_i^2)) for every row."""
    rng = np.random.default_rng(11)
    M, K1, D = 40, 24, 32
    X, W1, R, _, _ = _rand_block(rng, M, K1, D, D)
    for fn in (oracle.block_unfused, oracle.block_fused):
        h, _, y = fn(X, W1, R, np.ones(D), np.eye(D), eps, oracle.EPI_IDENTITY)
        ms = np.mean(h * h, axis=1)
        np.testing.assert_allclose(np.sqrt(np.mean(y * y, axis=1)), 1 / np.sqrt(1 + eps / ms), rtol=1e-13)


@pytest.mark.parametrize("epi", [oracle.EPI_IDENTITY, oracle.EPI_SWIGLU])
def test_scale_invariance_power_of_two(epi):
    """y(cX, W1, cR, gamma, W2, c^2 eps) = y(X, W1, R, gamma, W2, eps); bit-exact for c = 2^k."""
    rng = np.random.default_rng(5)
    X, W1, R, g, W2 = _rand_block(rng, 9, 16, 24, 32)
    for c in (2.0, 0.25, 1024.0):
        for fn in (oracle.block_unfused, oracle.block_fused):
            h0, _, y0 = fn(X, W1, R, g, W2, 1e-2, epi)
            h1, _, y1 = fn(c * X, W1, c * R, g, W2, c * c * 1e-2, epi)
            assert np.array_equal(h1, c * h0)
            assert np.array_equal(y1, y0)
    # a non-power-of-two scale still agrees to rounding
    _, _, y0 = oracle.block_fused(X, W1, R, g, W2, 1e-2, epi)
    _, _, y3 = oracle.block_fused(3 * X, W1, 3 * R, g, W2, 9e-2, epi)
    assert _normwise(y3, y0) < 1e-13


@pytest.mark.parametrize("epi", [oracle.EPI_IDENTITY, oracle.EPI_SWIGLU])
def test_row_independence(epi):
    """Row i of (h, y) depends only on row i of (X, R): permuting rows permutes outputs, bit-exact."""
    rng = np.random.default_rng(9)
    X, W1, R, g, W2 = _rand_block(rng, 23, 16, 24, 32)
    perm = rng.permutation(23)
    for fn in (oracle.block_unfused, oracle.block_fused, oracle.block_roundpts):
        h, r, y = fn(X, W1, R, g, W2, 1e-5, epi)
        hp, rp, yp = fn(X[perm], W1, R[perm], g, W2, 1e-5, epi)
        assert np.array_equal(hp, h[perm]) and np.array_equal(rp, r[perm]) and np.array_equal(yp, y[perm])
        # a single row alone gives the same row
        h1, r1, y1 = fn(X[4:5], W1, R[4:5], g, W2, 1e-5, epi)
        assert np.array_equal(y1[0], y[4])


def test_gamma_fold_and_column_permutation():
    """y(gamma, W2) = y(1, diag(gamma) W2); permuting W2's columns (gate and up together) permutes y."""
    rng = np.random.default_rng(13)
    X, W1, R, g, W2 = _rand_block(rng, 11, 16, 24, 40)
    for epi in (oracle.EPI_IDENTITY, oracle.EPI_SWIGLU):
        _, _, y = oracle.block_fused(X, W1, R, g, W2, 1e-5, epi)
        _, _, yfold = oracle.block_fused(X, W1, R, np.ones(24), g[:, None] * W2, 1e-5, epi)
        assert np.array_equal(y, yfold)
        _, _, yu = oracle.block_unfused(X, W1, R, np.ones(24), g[:, None] * W2, 1e-5, epi)
        assert _normwise(yu, y) < 1e-13
    # identity: any column permutation
    perm = rng.permutation(40)
    _, _, y = oracle.block_unfused(X, W1, R, g, W2, 1e-5, oracle.EPI_IDENTITY)
    _, _, yp = oracle.block_unfused(X, W1, R, g, W2[:, perm], 1e-5, oracle.EPI_IDENTITY)
    assert np.array_equal(yp, y[:, perm])
    # SwiGLU: the same permutation of gate and up columns
    p20 = rng.permutation(20)
    _, _, y = oracle.block_unfused(X, W1, R, g, W2, 1e-5, oracle.EPI_SWIGLU)
    W2p = np.concatenate([W2[:, :20][:, p20], W2[:, 20:][:, p20]], axis=1)
    _, _, yp = oracle.block_unfused(X, W1, R, g, W2p, 1e-5, oracle.EPI_SWIGLU)
    assert np.array_equal(yp, y[:, p20])
    # swapping gate and up is NOT a symmetry (silu is applied to the first half only)
    W2s = np.concatenate([W2[:, 20:], W2[:, :20]], axis=1)
    _, _, ys = oracle.block_unfused(X, W1, R, g, W2s, 1e-5, oracle.EPI_SWIGLU)
    assert _normwise(ys, y) > 1e-3


def test_brute_force_tiny_exact_sums():
    """Tiny shapes against exactly rounded sums (math.fsum), a different summation from the oracle's."""
    rng = np.random.default_rng(17)
    M, K1, D, N2 = 3, 5, 4, 6
    X, W1, R, g, W2 = _rand_block(rng, M, K1, D, N2)
    eps = 0.1
    h = np.array([[math.fsum([X[i, k] * W1[k, j] for k in range(K1)] + [R[i, j]]) for j in range(D)] for i in range(M)])
    r = np.array([1 / math.sqrt(math.fsum(h[i] ** 2) / D + eps) for i in range(M)])
    z = np.array([[math.fsum(h[i, j] * r[i] * g[j] * W2[j, c] for j in range(D)) for c in range(N2)] for i in range(M)])
    for fn in (oracle.block_unfused, oracle.block_fused):
        ho, ro, yo = fn(X, W1, R, g, W2, eps, oracle.EPI_IDENTITY)
        assert _normwise(ho, h) < 1e-14 and _normwise(ro, r) < 1e-14 and _normwise(yo, z) < 1e-13


# --- number formats --------------------------------------------------------------------------------------

def test_bf16_round_matches_torch_cast():
    """Round-to-nearest-even to bf16 against torch's fp32 -> bf16 cast, including exact ties, subnormals,
    overflow and signed zero."""
    rng = np.random.default_rng(21)
    vals = [rng.standard_normal(4000).astype(np.float32),
            (rng.standard_normal(2000) * 1e-38).astype(np.float32),
            (rng.standard_normal(2000) * 1e37).astype(np.float32),
            np.array([0.0, -0.0, 1.0, -1.0, 3.3895e38, 3.4e38, -3.4e38, 1e-45, 9.2e-41], np.float32)]
    # exact ties: bf16 grid points plus half a bf16 ulp (representable in fp32)
    base = torch.from_numpy(rng.standard_normal(2000).astype(np.float32)).to(torch.bfloat16).to(torch.float32).numpy()
    ulp = np.spacing(base.astype(np.float32)) * 65536
    vals.append((base + ulp / 2).astype(np.float32))
    x = np.concatenate(vals).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_round(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    want = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_decode(codes)
    nan = np.isnan(want)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    assert oracle.e4m3_decode(np.uint8(0x7E)) == 448.0


def test_e4m3_encode_round_trip_and_ties():
    rng = np.random.default_rng(23)
    x = np.concatenate([rng.uniform(-448, 448, 5000), rng.standard_normal(3000) * 0.01,
                        rng.standard_normal(2000) * 1e-3, [0.0, -0.0, 448.0, -448.0, 2 ** -9, 2 ** -10, 3 * 2 ** -10]])
    # exact midpoints between neighbouring codes (ties go to the even code)
    grid = np.sort(np.unique(oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = (grid[:-1] + grid[1:]) / 2
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, want)
    # saturation and NaN
    assert oracle.e4m3_encode(np.array([1000.0, -1e9, 464.0]))[0] == 0x7E
    assert list(oracle.e4m3_encode(np.array([1000.0, -1e9]))) == [0x7E, 0xFE]
    assert oracle.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F
    # decode(encode(code)) is the identity on every finite code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)


def test_dequant_against_torch():
    rng = np.random.default_rng(29)
    t = torch.from_numpy(rng.standard_normal((12, 20)).astype(np.float32))
    q = t.to(torch.float8_e4m3fn)
    qb = q.view(torch.uint8).numpy()
    s_rows = rng.uniform(0.1, 2.0, 12).astype(np.float32)
    s_cols = rng.uniform(0.1, 2.0, 20).astype(np.float32)
    qf = q.to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.dequant_rows_e4m3(qb, s_rows), qf * s_rows.astype(np.float64)[:, None])
    np.testing.assert_array_equal(oracle.dequant_cols_e4m3(qb, s_cols), qf * s_cols.astype(np.float64)[None, :])


def test_roundpts_rounds_only_at_storage_points():
    """The round-points diagnostic equals the fused form evaluated on bf16(h * gamma) against W2, then rounded
    to bf16; and it stays within bf16 error of the exact form."""
    rng = np.random.default_rng(31)
    X, W1, R, g, W2 = _rand_block(rng, 16, 32, 32, 64)
    for epi in (oracle.EPI_IDENTITY, oracle.EPI_SWIGLU):
        h, r, y = oracle.block_roundpts(X, W1, R, g, W2, 1e-5, epi)
        hf, rf, yf = oracle.block_fused(X, W1, R, g, W2, 1e-5, epi)
        assert np.array_equal(h, hf) and np.array_equal(r, rf)
        hg = torch.from_numpy((h * g[None, :]).astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
        z = (hg @ W2) * r[:, None]
        if epi == oracle.EPI_SWIGLU:
            z = F.silu(torch.from_numpy(z[:, :32])).numpy() * z[:, 32:]
        zb = torch.from_numpy(z).to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
        # same storage roundings; only the fp64 sums' order and the fp32 hop of the reference can flip a
        # rare bf16 tie
        assert np.mean(y != zb) < 0.01
        assert _normwise(y, yf) < 2e-2
