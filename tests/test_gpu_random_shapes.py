"""GPU parity of the fused block and its unfused baseline on seeded random shapes: row counts that end anywhere in
a row tile (including a single row), every K1 multiple of 128, hidden sizes on both sides of the folded-reduce
limit (D / 256 <= 16, else the reduce runs as its own kernel), both epilogues.  Each case is compared element by
element with the oracle: h, y and r against the fused fp64 form and y against the storage-rounding form for the
fused block, h and y against the oracle's unfused form for the baseline."""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, Workload, make_inputs

from parity import DeviceInputs, check_h, check_roundpts, check_y, f64, oracle_rows, run_block

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


def _shapes(n: int = 14, seed: int = 2024):
    """n seeded shapes of at most about 0.6 GFLOP each (the oracle's fp64 cost), plus one past the fold limit."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 31, 33, 127, 129, 255, 257]) if i < 2 else rng.integers(1, 320))
        K1 = 128 * int(rng.integers(1, 5))
        D = 256 * int(rng.integers(1, 4))
        N2 = 256 * int(rng.integers(1, 4))
        epi = int(rng.integers(0, 2))
        out.append(Workload(f"rand{i}_M{M}_K{K1}_D{D}_N{N2}_{'swiglu' if epi else 'id'}", M=M, K1=K1, D=D, N2=N2,
                            epi=EPI_SWIGLU if epi else EPI_IDENTITY, eps=1e-5, seed=100 + i))
    out.append(Workload("rand_unfolded_M77_K128_D4352_N256", M=77, K1=128, D=4352, N2=256, epi=EPI_SWIGLU,
                        eps=1e-5, seed=99))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_random_shape(wl):
    _say(f"[gpu] random shape {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r = run_block(d)
    oh, orr, oy = oracle_rows(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    np.testing.assert_allclose(f64(r), orr, rtol=2e-5)
    check_roundpts(f64(y), oracle_rows(inp, form="roundpts")[2])
    hu, yu, ru = run_block(d, unfused=True)
    uh, ur, uy = oracle_rows(inp, form="unfused")
    check_h(f64(hu), uh)
    check_y(f64(yu), uy)
    np.testing.assert_allclose(f64(ru), ur, rtol=2e-3)
