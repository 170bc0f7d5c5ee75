"""GPU parity of the block with a rotary position embedding in the second product's epilogue.

coda_block_fwd_rope (the rotation fused into K3's epilogue) and coda_block_fwd + coda_rope_rows (the rotation as
a separate pass) are compared with oracle.rope_rows applied to the fp64 oracle block (identity epilogue), on the
same bf16-valued inputs, to the bf16 contract of the block (normwise 2e-2, MAE 1e-3 of max|o|).  Cases: several
row and column tiles with a ragged last row tile, a rotated span that ends inside a tile, a sequence length that
is not a multiple of the row tile (positions wrap inside tiles), the degenerate cases (no rotated columns:
bit-identical to coda_block_fwd; seq_len 1: every position is 0, the rotation is the identity), and the
1B QKV shape (q and k heads rotated, v heads not) on every row.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, WORKLOADS, Workload, make_inputs

from parity import DeviceInputs, check_all_rows, check_h, check_y, f64, oracle_chunk_fn, oracle_rows, run_block

import oracle

pytestmark = pytest.mark.gpu

HEAD = 64


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


def _run_rope(d: DeviceInputs, seq_len, n_rot, base):
    wl = d.wl
    dev = d.X.device
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((wl.M, wl.N2), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_IDENTITY, device=dev)
    ws.fill_(0xFF)
    cb.coda_block_fwd_rope(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, seq_len, n_rot, base, h, y, ws)
    torch.cuda.synchronize()
    return h, y


def _run_separate(d: DeviceInputs, seq_len, n_rot, base):
    h, y, _ = run_block(d)
    cb.coda_rope_rows(y, seq_len, n_rot, base)
    torch.cuda.synchronize()
    return h, y


# (workload, seq_len, n_rope_cols, rope_base)
CASES = [
    (Workload("rope_ragged", M=640, K1=512, D=512, N2=768, epi=EPI_IDENTITY, eps=1e-5, w1_std=0.05,
              w2_std=0.05, seed=31), 200, 320, 10000.0),
    (Workload("rope_all_cols", M=512, K1=256, D=256, N2=512, epi=EPI_IDENTITY, eps=1e-6, w1_std=1 / 16,
              w2_std=1 / 16, seed=32), 96, 512, 500000.0),
    (Workload("rope_long_seq", M=384, K1=512, D=256, N2=1024, epi=EPI_IDENTITY, eps=1e-5, w1_std=0.05,
              w2_std=1 / 16, seed=33), 4096, 768, 10000.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0].name for c in CASES])
@pytest.mark.parametrize("path", ["fused", "separate"])
def test_rope_small(case, path):
    wl, seq_len, n_rot, base = case
    _say(f"rope {path} {wl.name} M={wl.M} K1={wl.K1} D={wl.D} N2={wl.N2} seq={seq_len} n_rot={n_rot}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    run = _run_rope if path == "fused" else _run_separate
    h, y = run(d, seq_len, n_rot, base)
    oh, _, oy = oracle_rows(inp)
    oy = oracle.rope_rows(oy, HEAD, n_rot, seq_len, base)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    # the columns past the rotated span are the plain block's, bit for bit
    _, y_plain, _ = run_block(d)
    assert torch.equal(y[:, n_rot:], y_plain[:, n_rot:])


def test_rope_no_rotated_columns_is_the_plain_block():
    wl = CASES[0][0]
    d = DeviceInputs(make_inputs(wl))
    _, y_plain, _ = run_block(d)
    _, y = _run_rope(d, 200, 0, 10000.0)
    assert torch.equal(y, y_plain)
    y2 = y_plain.clone()
    cb.coda_rope_rows(y2, 200, 0, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(y2, y_plain)


def test_rope_seq_len_one_is_the_identity():
    """Every position is 0, so every angle is 0 and the rotation is the identity: the output equals the plain
    block's to within one bf16 rounding."""
    wl = CASES[1][0]
    d = DeviceInputs(make_inputs(wl))
    _, y_plain, _ = run_block(d)
    _, y = _run_rope(d, 1, wl.N2, 500000.0)
    a, b = f64(y), f64(y_plain)
    assert np.all(np.abs(a - b) <= 2.0 ** -8 * np.abs(b))


def test_rope_fused_matches_separate_pass():
    """The two paths differ only in where bf16 rounding happens (before or after the rotation): at most a
    few bf16 half-ulps of the row's largest value (the inputs' two roundings and the two outputs')."""
    wl, seq_len, n_rot, base = CASES[0]
    d = DeviceInputs(make_inputs(wl))
    _, yf = _run_rope(d, seq_len, n_rot, base)
    _, ys = _run_separate(d, seq_len, n_rot, base)
    a, b = f64(yf), f64(ys)
    rowmax = np.max(np.abs(b), axis=1, keepdims=True)
    assert np.max(np.abs(a - b) / rowmax) <= 4 * 2.0 ** -8


@pytest.mark.timeout(600)
def test_rope_full_size_all_rows():
    """The 1B QKV shape (q and k heads rotated, v heads not), every row: the oracle block and its rotation
    chunk by chunk of rows, each chunk's rows at their own positions (row index mod seq_len)."""
    wl = WORKLOADS["1b_mlp_out_qkv"]
    seq_len, n_rot, base = 2048, 2560, 500000.0
    _say(f"rope fused full size, all rows {wl.name} seq={seq_len} n_rot={n_rot}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y = _run_rope(d, seq_len, n_rot, base)
    base_chunk = oracle_chunk_fn(inp, roundpts=False)

    def chunk(a, b):
        o = base_chunk(a, b)
        # row a + k sits at position (a + k) mod seq_len = (p0 + k) mod seq_len: rotate a block whose row index
        # starts p0 rows in and keep those rows
        p0 = a % seq_len
        buf = np.zeros((p0 + (b - a), o["y"].shape[1]), np.float64)
        buf[p0:] = o["y"]
        o["y"] = oracle.rope_rows(buf, HEAD, n_rot, seq_len, base)[p0:]
        return o

    check_all_rows(wl.M, h, y, None, chunk, say=_say)


def _random_cases(n: int = 8, seed: int = 313):
    """Seeded block shapes (identity epilogue) with a random rotated span (a multiple of the 64-column head, up to
    all of N2), sequence length and base."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 600))
        K1 = 128 * int(rng.integers(1, 5))
        D = 256 * int(rng.integers(1, 3))
        N2 = 256 * int(rng.integers(1, 5))
        n_rot = 64 * int(rng.integers(0, N2 // 64 + 1))
        seq = int(rng.choice([1, 7, 128, 333, 8192]))
        base = float(rng.choice([10000.0, 500000.0]))
        wl = Workload(f"roperand{i}_M{M}_K{K1}_D{D}_N{N2}_rot{n_rot}_seq{seq}", M=M, K1=K1, D=D, N2=N2,
                      epi=EPI_IDENTITY, eps=1e-5, w1_std=0.05, w2_std=0.05, seed=330 + i)
        out.append((wl, seq, n_rot, base))
    return out


RANDOM = _random_cases()


@pytest.mark.parametrize("case", RANDOM, ids=[c[0].name for c in RANDOM])
@pytest.mark.parametrize("path", ["fused", "separate"])
def test_rope_random_shape(case, path):
    wl, seq_len, n_rot, base = case
    _say(f"rope random {path} {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    run = _run_rope if path == "fused" else _run_separate
    h, y = run(d, seq_len, n_rot, base)
    oh, _, oy = oracle_rows(inp)
    oy = oracle.rope_rows(oy, HEAD, n_rot, seq_len, base)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
