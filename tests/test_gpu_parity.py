"""GPU parity of the fused block (and its unfused baseline) against the fp64 oracle, through the C ABI.

Small cases span several tiles and a ragged row tail and are compared element by element; the full-size
workloads run in the launch configuration the benchmark times and are compared on every row, the oracle run
chunk by chunk of rows (rows are independent, which the oracle's row-independence pin establishes).  The largest
accepted output (4 GiB of y) is compared on sampled rows that reach every row tile and every row position of an
accumulator block.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, WORKLOADS, Workload, make_inputs

from parity import (DeviceInputs, check_all_rows, check_h, check_roundpts, check_y, f64, normwise, oracle_chunk_fn,
                    oracle_rows, run_block, sample_rows_covering)

import oracle

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


SMALL = [
    WORKLOADS["tiny"],
    Workload("ragged_swiglu", M=300, K1=512, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, x_std=1.0, seed=1),
    Workload("ragged_identity", M=300, K1=384, D=768, N2=768, epi=EPI_IDENTITY, eps=1e-5, seed=2),
    Workload("one_row", M=1, K1=128, D=256, N2=256, epi=EPI_SWIGLU, eps=1e-6, seed=3),
    Workload("many_tiles", M=777, K1=1024, D=1024, N2=2048, epi=EPI_SWIGLU, eps=1e-5, seed=4),
    Workload("k128_tail", M=257, K1=128, D=256, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=5),
    # D / 256 = 17 > 16: the block runs the partial-RMS reduce as a kernel of its own instead of folding it
    Workload("wide_d_unfolded", M=260, K1=128, D=4352, N2=256, epi=EPI_SWIGLU, eps=1e-5, seed=6),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_fused_block_small(wl):
    _say(f"[gpu] fused block {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d)
    oh, orr, oy = oracle_rows(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    np.testing.assert_allclose(f64(r), orr, rtol=2e-5)
    _, _, oy_rp = oracle_rows(inp, form="roundpts")
    check_roundpts(f64(y), oy_rp)


UNFUSED_SMALL = SMALL[:3] + [SMALL[-1]]


@pytest.mark.parametrize("wl", UNFUSED_SMALL, ids=[w.name for w in UNFUSED_SMALL])
def test_unfused_block_small(wl):
    _say(f"[gpu] unfused block {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d, unfused=True)
    oh, orr, oy = oracle_rows(inp, form="unfused")
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    # the unfused GEMM1 stores T = X W1 in bf16 before the residual add (three separate operators), so its
    # row scale carries that rounding: about 2^-9 relative on T, hence a looser bound than the fused path
    np.testing.assert_allclose(f64(r), orr, rtol=2e-3)


def test_deterministic_and_in_place_residual():
    wl = SMALL[1]
    _say(f"[gpu] determinism / in-place {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    h1, y1, r1 = run_block(d)
    h2, y2, r2 = run_block(d)
    assert torch.equal(h1.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.equal(r1, r2)
    # out_h == R: the residual stream updated in place
    Rc = d.R.clone()
    h3, y3, _ = run_block(d, out_h=Rc, R=Rc)
    assert torch.equal(h3.view(torch.int16), h1.view(torch.int16))
    assert torch.equal(y3.view(torch.int16), y1.view(torch.int16))


def test_steps_one_by_one():
    """The three entry points of the steps, each against the oracle's definition of that step."""
    wl = SMALL[4]
    _say(f"[gpu] steps {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    T = wl.D // 256
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    hg = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    part = torch.full((T, wl.M), float("nan"), dtype=torch.float32, device="cuda")
    cb.coda_gemm1_residual_partial_rms(d.X, d.W1, d.R, d.gamma, h, hg, part)
    torch.cuda.synchronize()
    oh = oracle.gemm_residual(f64(inp.X), f64(inp.W1), f64(inp.R))
    check_h(f64(h), oh)
    # h * gamma with the same rule as h (gamma broadcast along the rows)
    check_h(f64(hg), oh * f64(inp.gamma)[None, :])
    opart = np.stack([np.sum(oh[:, 256 * t: 256 * (t + 1)] ** 2, axis=1) for t in range(T)])
    np.testing.assert_allclose(f64(part), opart, rtol=1e-4)
    # step 2 on the GPU's own partials, against the oracle's reduction of the same partials
    r = torch.full((wl.M,), float("nan"), dtype=torch.float32, device="cuda")
    cb.coda_partial_rms_reduce(part, wl.D, wl.eps, r)
    torch.cuda.synchronize()
    np.testing.assert_allclose(f64(r), oracle.rms_from_partials(f64(part), wl.D, wl.eps), rtol=3e-7)
    # step 3 on the GPU's hg and r: y = epi(r * (hg W2)) against the oracle's silu on the same operands
    y = torch.full((wl.M, wl.n_out), float("nan"), dtype=torch.bfloat16, device="cuda")
    cb.coda_gemm2_rowscale(hg, d.W2, r, wl.epi, y)
    torch.cuda.synchronize()
    z = (f64(hg) @ f64(inp.W2)) * f64(r)[:, None]
    half = wl.N2 // 2
    oy = np.array([[oracle.silu(v) for v in row] for row in z[:, :half]]) * z[:, half:]
    check_y(f64(y), oy)


FOLD = [SMALL[1], SMALL[3], SMALL[4],
        Workload("fold_t16", M=300, K1=256, D=4096, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=7),
        Workload("no_fold_t17", M=130, K1=128, D=4352, N2=256, epi=EPI_SWIGLU, eps=1e-5, seed=8)]


@pytest.mark.parametrize("wl", FOLD, ids=[w.name for w in FOLD])
def test_block_equals_its_three_steps(wl):
    """coda_block_fwd (the partial-RMS reduce folded into the second GEMM where D / 256 <= 16, the separate
    reduce kernel otherwise) gives the same h, r and y, bit for bit, as the three step entry points run one
    after another: the fold forms r with the reduce kernel's own expression and summation order.  The block runs
    without the split room here; where its second product's last wave then runs as 128-row halves (no_fold_t17),
    each output is still the whole tile's chain of MFMAs, so the bits are the steps' too."""
    _say(f"[gpu] block vs its steps {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    h, y, r = run_block(d, split=False)
    T = wl.D // 256
    h2 = torch.empty_like(h)
    hg = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device="cuda")
    part = torch.empty(T, wl.M, dtype=torch.float32, device="cuda")
    r2 = torch.empty(wl.M, dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y)
    cb.coda_gemm1_residual_partial_rms(d.X, d.W1, d.R, d.gamma, h2, hg, part)
    cb.coda_partial_rms_reduce(part, wl.D, wl.eps, r2)
    cb.coda_gemm2_rowscale(hg, d.W2, r2, wl.epi, y2)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    assert torch.equal(r.view(torch.int32), r2.view(torch.int32))
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16))


PANEL = [FOLD[0], FOLD[1], FOLD[3]]


@pytest.mark.parametrize("wl", PANEL, ids=[w.name for w in PANEL])
def test_panel_steps_equal_row_major_steps(wl):
    """The step entry points in the block's K-panel layout of hg give the row-major steps' h, part, hg (read
    back through the panel index), r and y bit for bit: the layout moves bytes, not arithmetic.  Step 3 with
    the folded reduce also writes the reduce kernel's r."""
    _say(f"[gpu] panel steps vs row-major steps {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    M, D, T = wl.M, wl.D, wl.D // 256
    ny = wl.N2 // 2 if wl.epi == EPI_SWIGLU else wl.N2
    dev = "cuda"
    h = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    hg = torch.empty(M, D, dtype=torch.bfloat16, device=dev)
    part = torch.empty(T, M, dtype=torch.float32, device=dev)
    r = torch.empty(M, dtype=torch.float32, device=dev)
    y = torch.empty(M, ny, dtype=torch.bfloat16, device=dev)
    cb.coda_gemm1_residual_partial_rms(d.X, d.W1, d.R, d.gamma, h, hg, part)
    cb.coda_partial_rms_reduce(part, D, wl.eps, r)
    cb.coda_gemm2_rowscale(hg, d.W2, r, wl.epi, y)
    h2 = torch.full_like(h, float("nan"))
    hgp = torch.full((D // 32, M, 32), float("nan"), dtype=torch.bfloat16, device=dev)
    part2 = torch.full_like(part, float("nan"))
    r2 = torch.full_like(r, float("nan"))
    y2 = torch.full_like(y, float("nan"))
    y3 = torch.full_like(y, float("nan"))
    cb.coda_gemm1_residual_partial_rms_panels(d.X, d.W1, d.R, d.gamma, h2, hgp, part2)
    cb.coda_gemm2_rowscale_panels(hgp, d.W2, part2, wl.eps, r2, wl.epi, y2)   # reduce folded in
    cb.coda_gemm2_rowscale_panels(hgp, d.W2, None, 0.0, r, wl.epi, y3)       # r given
    torch.cuda.synchronize()
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(h2), bits(h)) and torch.equal(bits(part2), bits(part))
    assert torch.equal(bits(hgp.permute(1, 0, 2).reshape(M, D)), bits(hg))
    assert torch.equal(bits(r2), bits(r))
    assert torch.equal(bits(y2), bits(y)) and torch.equal(bits(y3), bits(y))


def test_partial_reduce_synthetic():
    """Step 2 alone on synthetic partials: fixed-order fp32 sum, within a few fp32 ulps of the fp64 value."""
    _say("[gpu] partial reduce synthetic")
    g = torch.Generator().manual_seed(5)
    for T, M, D in [(1, 5, 256), (8, 8192, 2048), (16, 1000, 4096), (3, 257, 768)]:
        part = (torch.rand(T, M, generator=g) * 400).to(torch.float32)
        r = torch.empty(M, dtype=torch.float32, device="cuda")
        cb.coda_partial_rms_reduce(part.cuda(), D, 1e-5, r)
        torch.cuda.synchronize()
        np.testing.assert_allclose(f64(r), oracle.rms_from_partials(f64(part), D, 1e-5), rtol=4e-7)


def test_unit_gamma_identity_w2_property():
    """gamma = 1, W2 = I: RMS(y_i) = 1/sqrt(1 + eps/mean(h_i^2)) up to bf16 rounding, on every row."""
    wl = Workload("unit", M=513, K1=256, D=512, N2=512, epi=EPI_IDENTITY, eps=0.25, seed=6)
    _say(f"[gpu] unit-gamma property {wl.name}")
    inp = make_inputs(wl)
    inp.gamma = torch.ones(wl.D)
    inp.W2 = torch.eye(wl.D, dtype=torch.bfloat16)
    d = DeviceInputs(inp)
    h, y, _ = run_block(d)
    hf, yf = f64(h), f64(y)
    oh = oracle.gemm_residual(f64(inp.X), f64(inp.W1), f64(inp.R))
    want = 1 / np.sqrt(1 + wl.eps / np.mean(oh ** 2, axis=1))
    got = np.sqrt(np.mean(yf ** 2, axis=1))
    np.testing.assert_allclose(got, want, rtol=8e-3)


FULL = ["1b_attn_out_mlp_in", "1b_mlp_out_qkv", "8b_attn_out_mlp_in"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_all_rows(name):
    """Full-size workloads in the benchmark's launch configuration, every row against the oracle: h, y and r
    against the fused fp64 form, y against the storage-rounding form (the sharp bar), chunk by chunk."""
    wl = WORKLOADS[name]
    _say(f"[gpu] full size, all rows {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d)
    check_all_rows(wl.M, h, y, r, oracle_chunk_fn(inp), say=_say)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_70b_hidden_sampled_rows(unfused):
    """The 70B-style hidden size (D = 8192, SwiGLU over 2 x 28672 columns; the reduce as its own kernel) in the
    benchmark's launch configuration, on rows that reach every row tile and every row position of an accumulator
    block (every row would take the oracle minutes): h, y and r against the fused fp64 form, y against the
    storage-rounding form; the unfused baseline against the oracle's unfused form."""
    wl = WORKLOADS["70b_attn_out_mlp_in"]
    _say(f"[gpu] 70B hidden, {'unfused' if unfused else 'fused'}, sampled rows {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d, unfused=unfused)
    rows = sample_rows_covering(wl.M, n=24)
    idx = torch.as_tensor(rows, dtype=torch.long, device=y.device)
    gh, gy = f64(h[idx]), f64(y[idx])
    del h, y, d
    torch.cuda.empty_cache()
    oh, orr, oy = oracle_rows(inp, rows, form="unfused" if unfused else "fused")
    check_h(gh, oh)
    check_y(gy, oy)
    if unfused:
        # T = X W1 is stored in bf16 before the residual add (as in test_unfused_block_small)
        np.testing.assert_allclose(f64(r[rows]), orr, rtol=2e-3)
        return
    np.testing.assert_allclose(f64(r[rows]), orr, rtol=2e-5)
    _, _, oy_rp = oracle_rows(inp, rows, form="roundpts")
    check_roundpts(gy, oy_rp)


def test_largest_output_sampled_rows():
    """y at the largest size the ABI accepts, 2^31 elements (65536 x 32768 bf16, 4 GiB): store offsets up to
    2^32 - 2 bytes (past any signed 32-bit offset), 32768 second-GEMM tiles.  Checked against the oracle on
    sampled rows, the last ones among them, and for finiteness everywhere."""
    wl = Workload("largest_y", M=65536, K1=128, D=256, N2=32768, epi=EPI_IDENTITY, eps=1e-5, seed=12)
    _say(f"[gpu] largest output {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d)
    assert bool(torch.isfinite(y).all()) and bool(torch.isfinite(h).all()), "unwritten or non-finite output"
    rows = sample_rows_covering(wl.M, n=16)
    idx = torch.as_tensor(rows, dtype=torch.long, device=y.device)
    oh, orr, oy = oracle_rows(inp, rows)
    check_h(f64(h[idx]), oh)
    check_y(f64(y[idx]), oy)
    np.testing.assert_allclose(f64(r[rows]), orr, rtol=2e-5)

