"""Shared helpers of the parity tests: error metrics, GPU runs through the C ABI and oracle runs.

Tolerances (the contract of the fused block; bf16 outputs):
  y  : normwise max relative error  max|g - o| / max|o|        <= 2e-2  (fp8 operands: 6e-2)
       mean absolute error relative to the output's scale    mean|g - o| / max|o| <= 1e-3
  h  : normwise max relative error                             <= 1e-2, and elementwise
       |g - o| <= 1e-2 |o| + 1e-2 rms(o_row)
Elementwise relative error is not used for y: near zero it is unbounded even for an exact pipeline whose
only error is the final bf16 rounding.  The sharper detector compares with the oracle's storage-rounding
form (h, gamma*W2 and y rounded to bf16 where the kernels round), against which a correct kernel differs
only by fp32 accumulation order.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, BlockInputs

Y_NORMWISE = 2e-2
Y_NORMWISE_FP8 = 6e-2
Y_MAE_REL = 1e-3
H_NORMWISE = 1e-2
H_ELEM_REL = 1e-2
# against the storage-rounding oracle: a few bf16 ulps at the largest magnitude, tiny on average
RP_NORMWISE = 1.6e-2
RP_MAE_REL = 1e-4


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def normwise(g: np.ndarray, o: np.ndarray) -> float:
    return float(np.max(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def mae_rel(g: np.ndarray, o: np.ndarray) -> float:
    return float(np.mean(np.abs(g - o)) / max(np.max(np.abs(o)), 1e-30))


def check_y(g: np.ndarray, o: np.ndarray, fp8: bool = False, what: str = "y") -> dict:
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    nw, mr = normwise(g, o), mae_rel(g, o)
    lim = Y_NORMWISE_FP8 if fp8 else Y_NORMWISE
    assert nw <= lim, f"{what}: normwise max rel error {nw:.3e} > {lim}"
    if not fp8:
        assert mr <= Y_MAE_REL, f"{what}: MAE/max|o| {mr:.3e} > {Y_MAE_REL}"
    return {"normwise": nw, "mae_rel": mr, "mae_abs": float(np.mean(np.abs(g - o)))}


def check_h(g: np.ndarray, o: np.ndarray) -> dict:
    assert np.all(np.isfinite(g)), "h: non-finite values"
    nw = normwise(g, o)
    assert nw <= H_NORMWISE, f"h: normwise {nw:.3e} > {H_NORMWISE}"
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    bound = H_ELEM_REL * np.abs(o) + H_ELEM_REL * rms
    bad = np.abs(g - o) > bound
    assert not bad.any(), f"h: {int(bad.sum())} elements outside |dh| <= 1e-2|h| + 1e-2 rms(h_row)"
    return {"normwise": nw}


def check_roundpts(g: np.ndarray, o_rp: np.ndarray, what: str = "y") -> dict:
    nw, mr = normwise(g, o_rp), mae_rel(g, o_rp)
    assert nw <= RP_NORMWISE, f"{what} vs storage-rounding oracle: normwise {nw:.3e} > {RP_NORMWISE}"
    assert mr <= RP_MAE_REL, f"{what} vs storage-rounding oracle: MAE/max {mr:.3e} > {RP_MAE_REL}"
    return {"rp_normwise": nw, "rp_mae_rel": mr}


class DeviceInputs:
    """The inputs of one workload copied to the GPU once."""

    def __init__(self, inp: BlockInputs, device="cuda"):
        self.inp = inp
        self.wl = inp.wl
        self.X = inp.X.to(device)
        self.W1 = inp.W1.to(device)
        self.R = inp.R.to(device)
        self.gamma = inp.gamma.to(device)
        self.W2 = inp.W2.to(device)


def run_block(d: DeviceInputs, unfused: bool = False, poison: bool = True, out_h=None, R=None):
    """One call of coda_block_fwd (or coda_block_unfused) on fresh, NaN-poisoned outputs and workspace."""
    wl = d.wl
    dev = d.X.device
    h = out_h if out_h is not None else torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=int(unfused), device=dev)
    if poison:
        if out_h is None:
            h.fill_(float("nan"))
        y.fill_(float("nan"))
        ws.fill_(0xFF)
    fn = cb.coda_block_unfused if unfused else cb.coda_block_fwd
    fn(d.X, d.W1, d.R if R is None else R, d.gamma, d.W2, wl.eps, wl.epi, h, y, ws)
    torch.cuda.synchronize()
    r = cb.workspace_r(ws, wl.M, wl.D).clone()
    return h, y, r


def oracle_rows(inp: BlockInputs, rows=None, form: str = "fused"):
    """Oracle (h, r, y) in fp64 for the given rows (all rows if None); rows are independent."""
    wl = inp.wl
    X, R = inp.X, inp.R
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long)
        X, R = X[idx], R[idx]
    fn = {"fused": oracle.block_fused, "unfused": oracle.block_unfused, "roundpts": oracle.block_roundpts}[form]
    return fn(f64(X), f64(inp.W1), f64(R), f64(inp.gamma), f64(inp.W2), wl.eps, wl.epi)


def sample_rows(M: int, n: int = 48, seed: int = 0) -> np.ndarray:
    """First rows, last rows (the ragged tail) and a seeded spread in between, sorted and unique."""
    rng = np.random.default_rng(seed)
    picks = set(range(min(8, M))) | set(range(max(0, M - 8), M))
    picks |= set(int(v) for v in rng.choice(M, size=min(n, M), replace=False))
    return np.array(sorted(picks))
