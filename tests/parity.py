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


def run_block(d: DeviceInputs, unfused: bool = False, poison: bool = True, out_h=None, R=None, split: bool = True,
              ws_out: list = None):
    """One call of coda_block_fwd (or coda_block_unfused) on fresh, NaN-poisoned outputs and workspace.  split=False
    gives the call a workspace without the room to split the second product's last wave (whole tiles only);
    ws_out, if given, receives the workspace."""
    wl = d.wl
    dev = d.X.device
    h = out_h if out_h is not None else torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=int(unfused), device=dev, split=split)
    if ws_out is not None:
        ws_out.append(ws)
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


def sample_rows_covering(M: int, n: int = 48, seed: int = 0) -> np.ndarray:
    """sample_rows plus, for every 256-row tile, one row in each 128-row half, chosen so that the sample covers
    every value of row % 32 (a lane's row inside a 32-row accumulator block) and every 32-row block of each half:
    a tile placed wrongly, or a row mapping wrong inside a tile, cannot hide in unsampled rows."""
    picks = set(int(v) for v in sample_rows(M, n, seed))
    tiles = (M + 255) // 256
    for t in range(tiles):
        for half in (0, 1):
            off = 128 * half + 32 * ((t + half) % 4) + (t + 16 * half) % 32
            row = 256 * t + off
            if row < M:
                picks.add(row)
    for res in range(32):  # every residue mod 32 at least once, whatever the tile count
        if not any(p % 32 == res for p in picks):
            cand = [m for m in range(res, M, 32)]
            if cand:
                picks.add(cand[(res * 7919) % len(cand)])
    return np.array(sorted(picks))


class Gauge:
    """Running normwise and mean absolute errors of a result compared chunk by chunk of rows, so that every row
    of a full-size output can be checked without holding the oracle's whole fp64 output at once."""

    def __init__(self, what: str):
        self.what = what
        self.max_err = 0.0
        self.max_ref = 0.0
        self.sum_err = 0.0
        self.n = 0

    def add(self, g: np.ndarray, o: np.ndarray) -> None:
        assert np.all(np.isfinite(g)), f"{self.what}: non-finite values"
        d = np.abs(g - o)
        if d.size:
            self.max_err = max(self.max_err, float(d.max()))
            self.max_ref = max(self.max_ref, float(np.abs(o).max()))
            self.sum_err += float(d.sum())
            self.n += d.size

    def normwise(self) -> float:
        return self.max_err / max(self.max_ref, 1e-30)

    def mae_rel(self) -> float:
        return self.sum_err / max(self.n, 1) / max(self.max_ref, 1e-30)


def check_h_local(g: np.ndarray, o: np.ndarray) -> None:
    """The elementwise half of check_h (|dh| <= 1e-2 |h| + 1e-2 rms(h_row)): a property of each row alone."""
    rms = np.sqrt(np.mean(o * o, axis=1, keepdims=True))
    bad = np.abs(g - o) > H_ELEM_REL * np.abs(o) + H_ELEM_REL * rms
    assert not bad.any(), f"h: {int(bad.sum())} elements outside |dh| <= 1e-2|h| + 1e-2 rms(h_row)"


def check_all_rows(M: int, h: torch.Tensor, y: torch.Tensor, r, oracle_chunk, fp8: bool = False,
                   chunk: int = 1024, say=print, r_rtol: float = 2e-5) -> dict:
    """Every row of a GPU result against the oracle, chunk by chunk (rows are independent, so the oracle can run
    on row ranges).  h, y (bf16) and r (fp32, or None) are the GPU's results; oracle_chunk(a, b) returns a dict
    with the oracle's 'h', 'y' (fp64) and optionally 'r' and 'y_rp' (the storage-rounding form) for rows a..b-1.
    Applies the contract of check_h / check_y / check_roundpts to the whole output, and prints one progress line
    per chunk."""
    hc, yc = h.detach().cpu(), y.detach().cpu()
    rc = r.detach().cpu() if r is not None else None
    gh, gy, grp = Gauge("h"), Gauge("y"), Gauge("y vs storage-rounding oracle")
    for a in range(0, M, chunk):
        b = min(M, a + chunk)
        o = oracle_chunk(a, b)
        hg = f64(hc[a:b])
        gh.add(hg, o["h"])
        check_h_local(hg, o["h"])
        yg = f64(yc[a:b])
        gy.add(yg, o["y"])
        if "y_rp" in o:
            grp.add(yg, o["y_rp"])
        if rc is not None and "r" in o:
            np.testing.assert_allclose(f64(rc[a:b]), o["r"], rtol=r_rtol)
        say(f"    rows {a}..{b - 1} of {M}: y normwise so far {gy.normwise():.3e}")
    out = {"h_normwise": gh.normwise(), "y_normwise": gy.normwise(), "y_mae_rel": gy.mae_rel()}
    assert out["h_normwise"] <= H_NORMWISE, f"h: normwise {out['h_normwise']:.3e} > {H_NORMWISE}"
    lim = Y_NORMWISE_FP8 if fp8 else Y_NORMWISE
    assert out["y_normwise"] <= lim, f"y: normwise max rel error {out['y_normwise']:.3e} > {lim}"
    if not fp8:
        assert out["y_mae_rel"] <= Y_MAE_REL, f"y: MAE/max|o| {out['y_mae_rel']:.3e} > {Y_MAE_REL}"
    if grp.n:
        out["rp_normwise"], out["rp_mae_rel"] = grp.normwise(), grp.mae_rel()
        assert out["rp_normwise"] <= RP_NORMWISE, f"y vs storage-rounding oracle: normwise {out['rp_normwise']:.3e}"
        assert out["rp_mae_rel"] <= RP_MAE_REL, f"y vs storage-rounding oracle: MAE/max {out['rp_mae_rel']:.3e}"
    say("    all rows: " + ", ".join(f"{k} {v:.3e}" for k, v in out.items()))
    return out


def oracle_chunk_fn(inp: BlockInputs, roundpts: bool = True):
    """oracle_chunk for check_all_rows on a bf16 workload: the fused fp64 form (h, r, y) and, if asked, the
    storage-rounding form's y, for a row range."""
    wl = inp.wl
    W1, g, W2 = f64(inp.W1), f64(inp.gamma), f64(inp.W2)

    def fn(a, b):
        X, R = f64(inp.X[a:b]), f64(inp.R[a:b])
        oh, orr, oy = oracle.block_fused(X, W1, R, g, W2, wl.eps, wl.epi)
        out = {"h": oh, "r": orr, "y": oy}
        if roundpts:
            out["y_rp"] = oracle.block_roundpts(X, W1, R, g, W2, wl.eps, wl.epi)[2]
        return out

    return fn
