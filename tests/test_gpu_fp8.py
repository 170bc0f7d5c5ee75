"""GPU parity of the fused block with OCP e4m3 operands (and its unfused baseline) against the fp64 oracle.

The oracle runs on the dequantised inputs (code * scale, exact in fp64); the contract tolerance for e4m3 is
a normwise max relative error of 6e-2 on y (h keeps the bf16 rule).  The method-internal quantisers are byte
work and are checked bit for bit: given the h the GPU stored (bf16) and gamma, the kernels' steps are fully
determined in fp32 (a = h * gamma; per row: amax, s = amax / 448, its reciprocal, a times it, clamp to +-448,
round to nearest even e4m3; block-scaled: the power-of-two exponent of each 32-value block and a / 2^e), so an
fp32 emulation of those steps in numpy, with the oracle's e4m3 encoder for the last rounding, must reproduce
every code and every scale.  As an end-to-end check the same quantisers applied to the oracle's own h (rounded
to bf16 as stored) must agree on at least 99% of the codes (the rest sit where the GPU's fp32-accumulated h is
one bf16 step from the oracle's), and the block-scaled y must match the oracle's y computed through its own
quantised operand to the storage-rounding bar.  The full-size workload is compared on every row.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, WORKLOADS, Workload, make_inputs

from parity import check_all_rows, check_h, check_roundpts, check_y, f64

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


def _u8(t):
    return t.view(torch.uint8).numpy()


def _oracle_fp8(inp, rows=None, form="fused"):
    wl = inp.wl
    Xq, sx, R = inp.Xq, inp.sx, inp.R
    if rows is not None:
        idx = torch.as_tensor(rows, dtype=torch.long)
        Xq, sx, R = Xq[idx], sx[idx], R[idx]
    X = oracle.dequant_rows_e4m3(_u8(Xq), sx.numpy())
    W1 = oracle.dequant_cols_e4m3(_u8(inp.W1q), inp.sw1.numpy())
    W2 = oracle.dequant_cols_e4m3(_u8(inp.W2q), inp.sw2.numpy())
    fn = oracle.block_fused if form == "fused" else oracle.block_unfused
    return fn(X, W1, f64(R), f64(inp.gamma), W2, wl.eps, wl.epi)


def _align256(x):
    return (x + 255) // 256 * 256


def _oracle_a32(oh, gamma):
    """a = bf16(h) * gamma in fp32 from the oracle's fp64 h (the kernels multiply the stored bf16 h in fp32)."""
    hb = oracle.bf16_round(oh).astype(np.float32)
    return (hb * gamma.numpy().astype(np.float32)[None, :]).astype(np.float32)


def _panels_to_rows(flat, M, D, P=64):
    """The fused paths keep the e4m3 operand in the workspace as K panels [D / P][M][P] (element (m, k) at
    ((k / P) * M + m) * P + k % P); this returns it as [M, D]."""
    return flat.view(D // P, M, P).permute(1, 0, 2).reshape(M, D)


def _gpu_a32(h, gamma):
    """a = h * gamma in fp32 from the GPU's stored bf16 h: the quantisers' input exactly as the kernels form it
    (bf16 -> fp32 is exact, the product is one fp32 rounding)."""
    hb = h.detach().cpu().float().numpy()
    return hb * gamma.numpy().astype(np.float32)[None, :]


def _rowq_fp32(a):
    """The per-row quantiser's steps in fp32: s = amax / 448 (1 for an all-zero row), inv = 1 / s, q = e4m3 of
    a * inv clamped to +-448 (the last rounding by the oracle's encoder; the fp32 value is exact in fp64)."""
    amax = np.max(np.abs(a), axis=1).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    inv = (np.float32(1.0) / s).astype(np.float32)
    quot = np.clip(a * inv[:, None], np.float32(-448.0), np.float32(448.0)).astype(np.float32)
    return oracle.e4m3_encode(quot.astype(np.float64)), s


def _ws_rowq(ws, M, D):
    """The per-row e4m3 path's workspace after a call: part, r, the codes (K panels of 64), s_a [M], s_a * r [M]."""
    off_r = _align256((D // 256) * M * 4)
    off_q = off_r + _align256(M * 4)
    off_s = off_q + _align256(M * D)
    off_rs = off_s + _align256(M * 4)
    wsc = ws.cpu()
    f32 = lambda off: wsc[off: off + 4 * M].view(torch.float32).numpy()
    return {"r": f32(off_r), "q": _panels_to_rows(wsc[off_q: off_q + M * D], M, D).numpy(), "s": f32(off_s),
            "rs": f32(off_rs)}


def _check_rowq_exact(w, h, gamma):
    """Codes, scales and the epilogue row scale s * r of the per-row quantiser, bit for bit from the GPU's h."""
    want_q, want_s = _rowq_fp32(_gpu_a32(h, gamma))
    assert np.array_equal(w["s"].view(np.uint32), want_s.view(np.uint32)), \
        f"row scales: {int(np.sum(w['s'] != want_s))} differ"
    bad = w["q"] != want_q
    assert not bad.any(), f"codes: {int(bad.sum())} of {bad.size} differ (first at {np.argwhere(bad)[0]})"
    rs = (w["s"] * w["r"]).astype(np.float32)
    assert np.array_equal(w["rs"].view(np.uint32), rs.view(np.uint32)), "s_a * r differs from its fp32 product"


def _run_fp8(inp, unfused=False):
    wl = inp.wl
    dev = "cuda"
    args = [t.to(dev) for t in (inp.Xq, inp.sx, inp.W1q, inp.sw1, inp.R, inp.gamma, inp.W2q, inp.sw2)]
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((wl.M, wl.n_out), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=int(unfused), device=dev, fp8=1)
    ws.fill_(0xFF)
    fn = cb.coda_block_unfused_fp8 if unfused else cb.coda_block_fwd_fp8
    fn(*args, wl.eps, wl.epi, h, y, ws)
    torch.cuda.synchronize()
    return h, y, ws


FP8_SMALL = [
    Workload("fp8_ragged_swiglu", M=300, K1=512, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, fp8=True, seed=7),
    Workload("fp8_identity", M=257, K1=256, D=768, N2=512, epi=EPI_IDENTITY, eps=1e-5, fp8=True, seed=8),
    Workload("fp8_one_row", M=1, K1=256, D=256, N2=256, epi=EPI_SWIGLU, eps=1e-6, fp8=True, seed=9),
    # rows wider than the quantiser keeps in registers (D > 4096): the tail chunks are read twice
    Workload("fp8_wide_rows", M=40, K1=256, D=4608, N2=512, epi=EPI_IDENTITY, eps=1e-5, fp8=True, seed=10),
]


@pytest.mark.parametrize("wl", FP8_SMALL, ids=[w.name for w in FP8_SMALL])
def test_fp8_fused_small(wl):
    _say(f"[gpu] fp8 fused {wl}")
    inp = make_inputs(wl)
    h, y, ws = _run_fp8(inp)
    oh, orr, oy = _oracle_fp8(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)
    w = _ws_rowq(ws, wl.M, wl.D)
    np.testing.assert_allclose(w["r"], orr, rtol=2e-5)
    _check_rowq_exact(w, h, inp.gamma)
    # end to end: the same quantiser applied to the oracle's own h (rounded to bf16 as stored)
    q_oracle, s_oracle = _rowq_fp32(_oracle_a32(oh, inp.gamma))
    np.testing.assert_allclose(w["s"], s_oracle, rtol=2.0 ** -7)
    assert np.mean(w["q"] == q_oracle) >= 0.99


@pytest.mark.parametrize("wl", FP8_SMALL[:2], ids=[w.name for w in FP8_SMALL[:2]])
def test_fp8_unfused_small(wl):
    _say(f"[gpu] fp8 unfused {wl}")
    inp = make_inputs(wl)
    h, y, _ = _run_fp8(inp, unfused=True)
    oh, _, oy = _oracle_fp8(inp, form="unfused")
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)


def _oracle_fp8_chunks(inp):
    """oracle_chunk for check_all_rows: the fused fp64 form on the dequantised inputs, for a row range."""
    wl = inp.wl
    W1 = oracle.dequant_cols_e4m3(_u8(inp.W1q), inp.sw1.numpy())
    W2 = oracle.dequant_cols_e4m3(_u8(inp.W2q), inp.sw2.numpy())
    g = f64(inp.gamma)

    def fn(a, b):
        X = oracle.dequant_rows_e4m3(_u8(inp.Xq[a:b]), inp.sx[a:b].numpy())
        oh, orr, oy = oracle.block_fused(X, W1, f64(inp.R[a:b]), g, W2, wl.eps, wl.epi)
        return {"h": oh, "r": orr, "y": oy}

    return fn


@pytest.mark.timeout(600)
def test_fp8_full_size_all_rows():
    wl = WORKLOADS["1b_attn_out_mlp_in_fp8"]
    _say(f"[gpu] fp8 full size, all rows {wl}")
    inp = make_inputs(wl)
    h, y, ws = _run_fp8(inp)
    w = _ws_rowq(ws, wl.M, wl.D)
    _check_rowq_exact(w, h, inp.gamma)
    check_all_rows(wl.M, h, y, torch.from_numpy(w["r"]), _oracle_fp8_chunks(inp), fp8=True, say=_say)


# ---- block-scaled (MX-style) A operand of the second GEMM: coda_block_fwd_fp8_mx ----

def _run_fp8_mx(inp):
    wl = inp.wl
    dev = "cuda"
    args = [t.to(dev) for t in (inp.Xq, inp.sx, inp.W1q, inp.sw1, inp.R, inp.gamma, inp.W2q, inp.sw2)]
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((wl.M, wl.n_out), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev, fp8=2)
    ws.fill_(0xFF)
    cb.coda_block_fwd_fp8_mx(*args, wl.eps, wl.epi, h, y, ws)
    torch.cuda.synchronize()
    return h, y, ws


def _mx_scales_from_workspace(wsc, M, D, off):
    """The scale bytes in the kernels' layout: byte (((kt*tiles_m + tm)*2 + wm)*64 + 32h + j)*4 + mb holds the
    scale of row tm*256 + wm*128 + mb*32 + j, columns 64 kt + 32 h .. +31.  Returns exponents [M, D/32]."""
    tiles_m = (M + 255) // 256
    raw = wsc[off: off + (D // 64) * tiles_m * 512].numpy()
    m = np.arange(M)[:, None]
    kb = np.arange(D // 32)[None, :]
    kt, h = kb // 2, kb % 2
    tm, r = m // 256, m % 256
    idx = ((((kt * tiles_m + tm) * 2 + r // 128) * 64 + 32 * h + r % 32) * 4 + (r // 32) % 4)
    return raw[idx].astype(np.int32) - 127


def _check_mx_exact(q, e, h, gamma):
    """Codes and block exponents of the block-scaled quantiser, bit for bit: the oracle's block quantiser applied
    to a = h * gamma formed in fp32 from the GPU's stored h (a / 2^e is exact in fp32 and in fp64 alike)."""
    want_q, want_e = oracle.mx_quant_rows_e4m3(_gpu_a32(h, gamma).astype(np.float64), 32)
    bad_e = e != want_e
    assert not bad_e.any(), f"block exponents: {int(bad_e.sum())} of {bad_e.size} differ"
    bad = q != want_q
    assert not bad.any(), f"codes: {int(bad.sum())} of {bad.size} differ (first at {np.argwhere(bad)[0]})"


def _oracle_mx_y(inp, oh, orr, rows=None):
    """y through the oracle's own block-scaled operand: a = bf16(h) * gamma (fp32), quantised by the oracle,
    dequantised, times the dequantised W2, times r, the epilogue, then bf16 (the kernels' storage roundings)."""
    wl = inp.wl
    a = _oracle_a32(oh, inp.gamma)
    codes, exps = oracle.mx_quant_rows_e4m3(a.astype(np.float64), 32)
    A = oracle.e4m3_decode(codes) * np.ldexp(1.0, np.repeat(exps, 32, axis=1))
    W2 = oracle.dequant_cols_e4m3(_u8(inp.W2q), inp.sw2.numpy())
    z = orr[:, None] * (A @ W2)
    if wl.epi == EPI_SWIGLU:
        half = wl.N2 // 2
        g = z[:, :half]
        z = g / (1.0 + np.exp(-g)) * z[:, half:]
    return oracle.bf16_round(z), codes, exps


@pytest.mark.parametrize("wl", FP8_SMALL, ids=[w.name for w in FP8_SMALL])
def test_fp8_mx_small(wl):
    _say(f"[gpu] fp8 block-scaled {wl}")
    inp = make_inputs(wl)
    h, y, ws = _run_fp8_mx(inp)
    oh, orr, oy = _oracle_fp8(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)
    M, D = wl.M, wl.D
    off_r = _align256((D // 256) * M * 4)
    off_q = off_r + _align256(M * 4)
    off_s = off_q + _align256(M * D)
    wsc = ws.cpu()
    np.testing.assert_allclose(wsc[off_r: off_r + 4 * M].view(torch.float32).numpy(), orr, rtol=2e-5)
    y_mx, codes, exps = _oracle_mx_y(inp, oh, orr)
    check_roundpts(f64(y), y_mx)
    q = _panels_to_rows(wsc[off_q: off_q + M * D], M, D).numpy()
    e = _mx_scales_from_workspace(wsc, M, D, off_s)
    _check_mx_exact(q, e, h, inp.gamma)
    # end to end: the oracle's quantiser on the oracle's own h
    assert np.mean(q == codes) >= 0.99
    assert np.mean(e == exps) >= 0.99


@pytest.mark.timeout(600)
def test_fp8_mx_full_size_all_rows():
    wl = WORKLOADS["1b_attn_out_mlp_in_fp8"]
    _say(f"[gpu] fp8 block-scaled full size, all rows {wl}")
    inp = make_inputs(wl)
    h, y, ws = _run_fp8_mx(inp)
    M, D = wl.M, wl.D
    off_r = _align256((D // 256) * M * 4)
    off_q = off_r + _align256(M * 4)
    off_s = off_q + _align256(M * D)
    wsc = ws.cpu()
    q = _panels_to_rows(wsc[off_q: off_q + M * D], M, D).numpy()
    _check_mx_exact(q, _mx_scales_from_workspace(wsc, M, D, off_s), h, inp.gamma)
    base = _oracle_fp8_chunks(inp)

    def chunk(a, b):
        o = base(a, b)
        o["y_rp"] = _oracle_mx_y(inp, o["h"], o["r"])[0]
        return o

    r = wsc[off_r: off_r + 4 * M].view(torch.float32)
    check_all_rows(M, h, y, r, chunk, fp8=True, say=_say)


# ---- seeded random shapes: the per-row, block-scaled and unfused e4m3 paths, each against the oracle ----

def _fp8_random_shapes(n: int = 10, seed: int = 4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 3, 63, 65, 255, 257]) if i < 2 else rng.integers(1, 320))
        K1 = 256 * int(rng.integers(1, 3))
        D = 256 * int(rng.integers(1, 4))
        N2 = 256 * int(rng.integers(1, 4))
        epi = EPI_SWIGLU if rng.integers(0, 2) else EPI_IDENTITY
        out.append(Workload(f"fp8rand{i}_M{M}_K{K1}_D{D}_N{N2}_{'swiglu' if epi else 'id'}", M=M, K1=K1, D=D,
                            N2=N2, epi=epi, eps=1e-5, fp8=True, seed=200 + i))
    return out


FP8_RANDOM = _fp8_random_shapes()


@pytest.mark.parametrize("wl", FP8_RANDOM, ids=[w.name for w in FP8_RANDOM])
def test_fp8_random_shape(wl):
    _say(f"[gpu] fp8 random shape {wl}")
    inp = make_inputs(wl)
    oh, orr, oy = _oracle_fp8(inp)
    # per-row scales: end to end, r, and the quantiser bit for bit
    h, y, ws = _run_fp8(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)
    w = _ws_rowq(ws, wl.M, wl.D)
    np.testing.assert_allclose(w["r"], orr, rtol=2e-5)
    _check_rowq_exact(w, h, inp.gamma)
    # block-scaled A operand: end to end, the storage-rounding bar through the oracle's own quantiser, and the
    # codes and exponents bit for bit
    h, y, ws = _run_fp8_mx(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)
    M, D = wl.M, wl.D
    off_r = _align256((D // 256) * M * 4)
    off_q = off_r + _align256(M * 4)
    off_s = off_q + _align256(M * D)
    wsc = ws.cpu()
    check_roundpts(f64(y), _oracle_mx_y(inp, oh, orr)[0])
    q = _panels_to_rows(wsc[off_q: off_q + M * D], M, D).numpy()
    _check_mx_exact(q, _mx_scales_from_workspace(wsc, M, D, off_s), h, inp.gamma)
    # the unfused baseline against the oracle's unfused form
    h, y, _ = _run_fp8(inp, unfused=True)
    ouh, _, ouy = _oracle_fp8(inp, form="unfused")
    check_h(f64(h), ouh)
    check_y(f64(y), ouy, fp8=True)
