"""GPU tests of the half-tile form of the second GEMM's last wave, through the C ABI.

Where the second product's 256 x 256 output tiles leave a last wave that fills at most half of the CUs and that wave is
not split along K (bf16 blocks; the rule is halves_plan in csrc/launch.h), each tile of the wave runs as two 128-row
halves over the whole of K, in a launch of its own after the whole tiles.  Every output is the same chain of MFMAs as
in a whole tile, so the block's h, r and y equal those of the three step entry points (which always run whole tiles)
bit for bit.  Checked here:
- the rule written out, on the shapes below, which take the halves or do not;
- shapes that take them (every tile in halves; a whole wave and a tail in halves; a ragged last row tile of more than
  128 rows; SwiGLU and identity epilogues; the reduce folded in and as a kernel of its own), fused and unfused, every
  element against the oracle, and the fused block against its three steps bit for bit;
- a shape whose last wave the split along K takes when the workspace has the room for it and the halves take when it
  has not: both against the oracle, the halves bit for bit against the steps;
- the block with the rotary embedding and the forward that keeps z on a shape that takes the halves;
- full size: the 1B MLP-out -> QKV block (384 tiles: 256 whole, the last 128 in halves) against its steps bit for bit
  (its every row against the oracle is in test_gpu_parity.py).
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, WORKLOADS, Workload, make_inputs

from parity import DeviceInputs, check_h, check_roundpts, check_y, f64, oracle_rows, run_block

import oracle

pytestmark = pytest.mark.gpu

PLAN_CUS = 256


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()
    if torch.cuda.get_device_properties(0).multi_processor_count != PLAN_CUS:
        pytest.skip("the shapes below are chosen for 256 CUs")


def _halves(wl: Workload):
    """The half-tile rule written out, for a second GEMM whose last wave is not split along K: (whole tiles, tiles
    run in halves).  A last wave of at most half of the CUs, more than 64 rows, and a last row tile that is whole or
    has more than 128 rows."""
    tiles = -(-wl.M // 256) * (wl.N2 // 256)
    rem, tail = tiles % PLAN_CUS, wl.M % 256
    if wl.M <= 64 or rem == 0 or 2 * rem > PLAN_CUS or (tail and tail <= 128):
        return tiles, 0
    return tiles - rem, rem


HALVES = [
    # 2 x 40 = 80 tiles: all of them in halves (160 workgroups)
    Workload("halves_all", M=512, K1=256, D=256, N2=10240, epi=EPI_IDENTITY, eps=1e-5, seed=81),
    # 10 x 36 = 360 tiles: 256 whole, 104 in halves; SwiGLU
    Workload("halves_tail_swiglu", M=2560, K1=256, D=512, N2=9216, epi=EPI_SWIGLU, eps=1e-5, seed=82),
    # 11 x 24 = 264 tiles: 256 whole, 8 in halves; the last row tile has 200 rows (its second half 72)
    Workload("halves_ragged", M=2760, K1=128, D=256, N2=6144, epi=EPI_IDENTITY, eps=1e-5, seed=83),
    # D / 256 = 17: the reduce is a kernel of its own; 2 tiles in halves of 128 and 2 rows
    Workload("halves_no_fold", M=130, K1=128, D=4352, N2=512, epi=EPI_SWIGLU, eps=1e-5, seed=84),
]
# a last row tile of 40 rows: its second half would be empty, so the wave stays whole
WHOLE = Workload("halves_short_tail", M=2600, K1=128, D=256, N2=6144, epi=EPI_IDENTITY, eps=1e-5, seed=85)


def test_rule_on_the_shapes():
    assert [_halves(w) for w in HALVES] == [(0, 80), (256, 104), (256, 8), (0, 2)]
    assert _halves(WHOLE) == (264, 0)
    assert _halves(WORKLOADS["1b_mlp_out_qkv"]) == (256, 128)
    assert _halves(WORKLOADS["1b_attn_out_mlp_in"]) == (2048, 0)
    assert _halves(WORKLOADS["tiny"]) == (2, 0)


def _steps(d: DeviceInputs):
    """h, r, y of the three step entry points (whole tiles, the reduce as a kernel of its own)."""
    wl = d.wl
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device="cuda")
    hg = torch.empty_like(h)
    part = torch.empty(wl.D // 256, wl.M, dtype=torch.float32, device="cuda")
    r = torch.empty(wl.M, dtype=torch.float32, device="cuda")
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device="cuda")
    cb.coda_gemm1_residual_partial_rms(d.X, d.W1, d.R, d.gamma, h, hg, part)
    cb.coda_partial_rms_reduce(part, wl.D, wl.eps, r)
    cb.coda_gemm2_rowscale(hg, d.W2, r, wl.epi, y)
    torch.cuda.synchronize()
    return h, r, y


def _same_bits(a: torch.Tensor, b: torch.Tensor) -> bool:
    t = torch.int32 if a.dtype == torch.float32 else torch.int16
    return torch.equal(a.view(t), b.view(t))


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("wl", HALVES + [WHOLE], ids=[w.name for w in HALVES + [WHOLE]])
def test_halves_against_oracle_and_steps(wl, unfused):
    _say(f"[gpu] halves {'unfused' if unfused else 'fused'} {wl} rule {_halves(wl)}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    # no split room: the K split cannot take the last wave, the halves take it where the rule says so
    h, y, r = run_block(d, unfused=unfused, split=False)
    form = "unfused" if unfused else "fused"
    oh, orr, oy = oracle_rows(inp, form=form)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    np.testing.assert_allclose(f64(r), orr, rtol=2e-3 if unfused else 2e-5)
    if not unfused:
        check_roundpts(f64(y), oracle_rows(inp, form="roundpts")[2])
        h2, r2, y2 = _steps(d)
        assert _same_bits(h, h2) and _same_bits(r, r2) and _same_bits(y, y2)


def test_split_along_k_comes_first():
    """halves_no_fold's 2 tiles over K = D = 4352: with the split room the K split takes them (both pieces' tickets
    taken), without it the halves do; both against the oracle, the halves bit for bit against the steps."""
    wl = HALVES[3]
    _say(f"[gpu] halves vs K split {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    box = []
    h1, y1, r1 = run_block(d, split=True, ws_out=box)
    ws = box[0]
    total = cb.coda_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, 0)
    base = total - cb.coda_workspace_split_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, 0)
    assert total > base
    assert bool((ws[base: base + 8].view(torch.int32).cpu() == 2).all()), "the K split did not take the wave"
    h0, y0, r0 = run_block(d, split=False)
    oh, orr, oy = oracle_rows(inp)
    for h, y, r in ((h1, y1, r1), (h0, y0, r0)):
        check_h(f64(h), oh)
        check_y(f64(y), oy)
        np.testing.assert_allclose(f64(r), orr, rtol=2e-5)
    h2, r2, y2 = _steps(d)
    assert _same_bits(h0, h2) and _same_bits(r0, r2) and _same_bits(y0, y2)


def test_halves_rope_block():
    """coda_block_fwd_rope on halves_ragged (no K split: K = 256): the rotation against the oracle's, the columns past
    the rotated span equal to the plain block's bit for bit."""
    wl = HALVES[2]
    seq_len, n_rot, base = 48, 512, 10000.0
    _say(f"[gpu] halves rope {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((wl.M, wl.N2), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_IDENTITY, device="cuda")
    cb.coda_block_fwd_rope(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, seq_len, n_rot, base, h, y, ws)
    torch.cuda.synchronize()
    oh, _, oy = oracle_rows(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oracle.rope_rows(oy, 64, n_rot, seq_len, base))
    _, y_plain, _ = run_block(d)
    assert _same_bits(y[:, n_rot:], y_plain[:, n_rot:])


def test_halves_save_z():
    """The forward that keeps z on halves_tail_swiglu: y equal to coda_block_fwd's, z equal to the identity-epilogue
    block's y (the same tile grid, the same halves), bit for bit."""
    wl = HALVES[1]
    _say(f"[gpu] halves save z {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    _, y_plain, _ = run_block(d)
    _, z_plain, _ = run_block(DeviceInputs(make_inputs(wl.with_(epi=EPI_IDENTITY))))
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device="cuda")
    y = torch.full((wl.M, wl.N2 // 2), float("nan"), dtype=torch.bfloat16, device="cuda")
    z = torch.full((wl.M, wl.N2), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_SWIGLU, device="cuda")
    cb.coda_block_fwd_save_z(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, h, y, z, ws)
    torch.cuda.synchronize()
    assert _same_bits(y, y_plain)
    assert _same_bits(z, z_plain)


@pytest.mark.timeout(300)
def test_halves_full_size_equals_steps():
    """The 1B MLP-out -> QKV block with the default workspace: its last 128 tiles in halves; h, r, y equal to the
    three steps' bit for bit, and the same run to run."""
    wl = WORKLOADS["1b_mlp_out_qkv"]
    _say(f"[gpu] halves full size {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    h, y, r = run_block(d)
    _, y_again, _ = run_block(d)
    h2, r2, y2 = _steps(d)
    assert _same_bits(h, h2) and _same_bits(r, r2) and _same_bits(y, y2)
    assert _same_bits(y, y_again)
