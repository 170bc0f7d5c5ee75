"""Canary guard regions around every output and the workspace of the entry points (GPU), and the CODA_SYNC_CHECK
debugging mode.

Each output tensor and the workspace is a view into a larger buffer whose 4 KiB before and after are filled with a
byte pattern; after the call (and a synchronisation) the pattern must be intact, so a kernel that writes past a
tile edge, a masked row or the end of a buffer is caught even when the written values would look plausible.
Ragged shapes (a last row tile that is mostly masked) make such writes likely to show.
"""
import os
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import (CE_WORKLOADS, EPI_IDENTITY, EPI_SWIGLU, SwigluBwdWorkload, Workload,
                                             make_ce_inputs, make_grads, make_inputs, make_swiglu_bwd_inputs)

pytestmark = pytest.mark.gpu

GUARD = 4096
PATTERN = 0x5A


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


class Guarded:
    """A tensor of the given shape and dtype inside a byte buffer with GUARD bytes of PATTERN on each side."""

    def __init__(self, shape, dtype, fill=float("nan")):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.buf = torch.full((GUARD + n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.buf[GUARD: GUARD + n].view(dtype).view(*shape)
        if dtype != torch.uint8:
            self.t.fill_(fill)

    def intact(self):
        torch.cuda.synchronize()
        return bool((self.buf[:GUARD] == PATTERN).all()) and bool((self.buf[-GUARD:] == PATTERN).all())


def _check(named):
    bad = [k for k, g in named.items() if not g.intact()]
    assert not bad, f"guard bytes overwritten next to: {bad}"


BLOCKS = [
    Workload("guard_swiglu", M=300, K1=512, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=51),
    Workload("guard_identity_wide_d", M=130, K1=128, D=4352, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=52),
]


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("wl", BLOCKS, ids=[w.name for w in BLOCKS])
def test_block_writes_stay_inside(wl, unfused):
    _say(f"[gpu] guards {'unfused' if unfused else 'fused'} {wl.name}")
    inp = make_inputs(wl)
    X, W1, R, g, W2 = (t.cuda() for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    h = Guarded((wl.M, wl.D), torch.bfloat16)
    y = Guarded((wl.M, wl.n_out), torch.bfloat16)
    ws = Guarded((cb.coda_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, int(unfused)),), torch.uint8)
    fn = cb.coda_block_unfused if unfused else cb.coda_block_fwd
    fn(X, W1, R, g, W2, wl.eps, wl.epi, h.t, y.t, ws.t)
    _check({"out_h": h, "out_y": y, "workspace": ws})
    assert bool(torch.isfinite(y.t).all())


@pytest.mark.parametrize("mx", [False, True], ids=["per_row", "block_scaled"])
def test_fp8_block_writes_stay_inside(mx):
    wl = Workload("guard_fp8", M=300, K1=512, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, fp8=True, seed=53)
    _say(f"[gpu] guards fp8 {'mx' if mx else 'per-row'}")
    inp = make_inputs(wl)
    args = [t.cuda() for t in (inp.Xq, inp.sx, inp.W1q, inp.sw1, inp.R, inp.gamma, inp.W2q, inp.sw2)]
    h = Guarded((wl.M, wl.D), torch.bfloat16)
    y = Guarded((wl.M, wl.n_out), torch.bfloat16)
    ws = Guarded((cb.coda_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 2 if mx else 1, 0),), torch.uint8)
    (cb.coda_block_fwd_fp8_mx if mx else cb.coda_block_fwd_fp8)(*args, wl.eps, wl.epi, h.t, y.t, ws.t)
    _check({"out_h": h, "out_y": y, "workspace": ws})


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_bwd_writes_stay_inside(unfused):
    wl = Workload("guard_bwd", M=384, K1=512, D=512, N2=768, epi=EPI_IDENTITY, eps=1e-5, w1_std=0.05, w2_std=0.05,
                  seed=54)
    _say(f"[gpu] guards bwd {'unfused' if unfused else 'fused'}")
    inp = make_inputs(wl)
    dz, dho = (t.cuda() for t in make_grads(wl))
    X, W1, R, g, W2 = (t.cuda() for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device="cuda")
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device="cuda")
    wsf = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device="cuda")
    cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, wsf)
    r = cb.workspace_r(wsf, wl.M, wl.D)
    outs = {"dX": Guarded((wl.M, wl.K1), torch.bfloat16), "dW1": Guarded((wl.K1, wl.D), torch.float32),
            "dR": Guarded((wl.M, wl.D), torch.bfloat16), "dgamma": Guarded((wl.D,), torch.float32),
            "dW2": Guarded((wl.D, wl.N2), torch.float32),
            "workspace": Guarded((cb.coda_bwd_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, int(unfused)),), torch.uint8)}
    fn = cb.coda_block_bwd_unfused if unfused else cb.coda_block_bwd
    fn(X, W1, h, r, g, W2, dz, dho, *(outs[k].t for k in ("dX", "dW1", "dR", "dgamma", "dW2", "workspace")))
    _check(outs)


def test_ce_and_swiglu_bwd_writes_stay_inside():
    _say("[gpu] guards ce and swiglu bwd")
    from gemm_epilogue_fusion_amd.inputs import CeWorkload
    wl = CeWorkload("guard_ce", M=300, D=256, V=1024, ignore_every=7, seed=55)
    H, W, labels = (t.cuda() for t in make_ce_inputs(wl))
    loss, lse = Guarded((wl.M,), torch.float32), Guarded((wl.M,), torch.float32)
    ws = Guarded((cb.coda_ce_workspace_bytes(wl.M, wl.D, wl.V, 0),), torch.uint8)
    cb.coda_ce_fwd(H, W, labels, loss.t, lse.t, ws.t)
    _check({"loss": loss, "lse": lse, "workspace": ws})
    sw = SwigluBwdWorkload("guard_swiglu_bwd", M=300, D=384, F=768, seed=56)
    dout, Wd, z = (t.cuda() for t in make_swiglu_bwd_inputs(sw))
    dz = Guarded((sw.M, 2 * sw.F), torch.bfloat16)
    cb.coda_swiglu_bwd(dout, Wd, z, dz.t)
    _check({"dz": dz})


def test_sync_check_mode_gives_the_same_results():
    """CODA_SYNC_CHECK=1 synchronises and checks after every launch; the results are the normal path's bit for
    bit, and the entry point still returns success."""
    wl = BLOCKS[0]
    _say("[gpu] CODA_SYNC_CHECK")
    inp = make_inputs(wl)
    X, W1, R, g, W2 = (t.cuda() for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    outs = []
    for mode in ("0", "1"):
        os.environ["CODA_SYNC_CHECK"] = mode
        try:
            h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device="cuda")
            y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device="cuda")
            ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device="cuda")
            cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws)
            torch.cuda.synchronize()
            outs.append((h, y))
        finally:
            os.environ.pop("CODA_SYNC_CHECK", None)
    assert torch.equal(outs[0][0].view(torch.int16), outs[1][0].view(torch.int16))
    assert torch.equal(outs[0][1].view(torch.int16), outs[1][1].view(torch.int16))
