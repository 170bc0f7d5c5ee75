"""GPU tests of the GEMM kernels' small-row form (at most 64 rows: each SIMD holds one wave of the tile's first 128
rows, which computes the first two 32-row blocks, and the waves of rows 128 .. 255 skip the product), through the
C ABI.

- The small form gives the general form's results bit for bit: a block on 64 rows against the same block on those
  64 rows plus one (65 rows take the general form), h, r and y compared on the 64 rows, for both epilogues, the
  fused and the unfused block, with and without the split of the second product's K (D = 2048).
- Against the oracle on every element at 1, 17 and 64 rows, fused and unfused, and the block with the rotary
  embedding.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, Workload, make_inputs

from parity import DeviceInputs, check_h, check_roundpts, check_y, f64, oracle_rows, run_block

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


def _first_rows(inp, n):
    """The same inputs restricted to the first n rows."""
    sub = DeviceInputs(inp)
    sub.X, sub.R = sub.X[:n].contiguous(), sub.R[:n].contiguous()
    sub.wl = inp.wl.with_(M=n)
    return sub


SHAPES = [(512, 1024), (2048, 512)]  # (D, N2); D = 2048 splits the second product's K


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("epi", [EPI_IDENTITY, EPI_SWIGLU], ids=["identity", "swiglu"])
@pytest.mark.parametrize("shape", SHAPES, ids=[f"D{d}_N{n}" for d, n in SHAPES])
def test_small_form_equals_general_form(shape, epi, unfused):
    D, N2 = shape
    wl = Workload("small_vs_general", M=65, K1=256, D=D, N2=N2, epi=epi, eps=1e-5, seed=71)
    _say(f"[gpu] small form vs general form {wl} unfused={unfused}")
    inp = make_inputs(wl)
    h65, y65, r65 = run_block(DeviceInputs(inp), unfused=unfused)
    h64, y64, r64 = run_block(_first_rows(inp, 64), unfused=unfused)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    assert torch.equal(bits(h64), bits(h65[:64]))
    assert torch.equal(bits(r64), bits(r65[:64]))
    assert torch.equal(bits(y64), bits(y65[:64]))


SMALL = [
    Workload("small_one_row", M=1, K1=384, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=72),
    Workload("small_17_rows", M=17, K1=256, D=768, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=73),
    Workload("small_64_rows", M=64, K1=512, D=1024, N2=2048, epi=EPI_SWIGLU, eps=1e-6, seed=74),
]


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_rows_against_oracle(wl, unfused):
    _say(f"[gpu] small rows {wl} unfused={unfused}")
    inp = make_inputs(wl)
    h, y, r = run_block(DeviceInputs(inp), unfused=unfused)
    oh, orr, oy = oracle_rows(inp, form="unfused" if unfused else "fused")
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    np.testing.assert_allclose(f64(r), orr, rtol=2e-3 if unfused else 2e-5)
    if not unfused:
        check_roundpts(f64(y), oracle_rows(inp, form="roundpts")[2])


def test_small_rows_rope_block():
    wl = Workload("small_rope", M=40, K1=256, D=512, N2=768, epi=EPI_IDENTITY, eps=1e-5, seed=75)
    seq_len, n_rot, base = 16, 512, 10000.0
    _say(f"[gpu] small rows rope {wl}")
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
