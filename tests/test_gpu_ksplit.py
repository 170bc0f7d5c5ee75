"""GPU tests of the split of the GEMMs' last waves of tiles, through the C ABI.

Where a GEMM's 256 x 256 output tiles leave a last wave that fills at most a quarter of the CUs, each tile of that wave
is computed as two halves of K whose fp32 sums are added before the epilogue, in either GEMM of the bf16 blocks
(coda_workspace_bytes in include/coda.h describes the room this takes in the workspace).  Checked here:
- the split is taken where it is planned: after a call every split tile of either GEMM holds ticket 2 (both halves
  ran and each took its ticket), and the workspace's split room matches the rule written out here;
- small shapes with the second GEMM's tiles split (a ragged row tile, SwiGLU and identity epilogues, the path with
  the reduce as a kernel of its own), the first GEMM's, or both, and a shape with a whole wave plus a split tail,
  fused and unfused, against the oracle (every element on the small shapes; rows covering every row tile on the
  tail shape), and against the same block run on whole tiles (a workspace without the split room): y within the
  fp32 summation-order difference, h and r equal bit for bit where the first GEMM is not split;
- outputs bit-identical run to run, whichever half finishes second;
- full size: a last wave of 32 tiles in the second GEMM (a QKV projection with 2 key-value heads of 64 after the 1B
  hidden size: 8192 rows, D = 2048, 2048 + 2 x 128 output columns, 288 tiles), the 1B MLP-out -> QKV block on
  1024 rows (both GEMMs' tiles split) and 3072 rows over K1 = 4096 (a last wave of 96 tiles): tickets, run-to-run identity, a row in every row tile against the oracle and
  every row against the whole-tile run; the 1B MLP-out -> QKV shape itself (384 tiles, a last wave of 128) is not
  split;
- the block with the rotary embedding and the forward that keeps z take the same split;
- seeded random shapes that split either GEMM or both, into 2, 4 and 8 pieces, every element against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, WORKLOADS, Workload, make_inputs

from parity import (DeviceInputs, check_h, check_roundpts, check_y, f64, mae_rel, normwise, oracle_rows, run_block,
                    sample_rows_covering)

import oracle

pytestmark = pytest.mark.gpu

SLOT_BYTES = 512 * 128 * 4  # one workgroup's fp32 accumulators
PLAN_CUS = 256              # the split room is planned for MI355X's CU count
# y of the split and whole-tile runs: the same products summed in another fp32 order, then rounded to bf16
CLOSE_NORMWISE = 1e-2
CLOSE_MAE_REL = 1e-4


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()
    if torch.cuda.get_device_properties(0).multi_processor_count != PLAN_CUS:
        pytest.skip("the split room is planned for 256 CUs")


def _plan(tiles: int, K: int):
    """The split rule written out: (split tiles, log2 of the pieces per tile).  A last wave that fills at most a
    quarter of the CUs (three eighths where K >= 4096) splits in two where K gives two pieces of at least 512 (K a
    multiple of 256); in more, up to 8, while all pieces stay within half of the CUs and each keeps at least 1024 of
    K (a multiple of 128)."""
    rem = tiles % PLAN_CUS
    if rem == 0 or (4 * rem > PLAN_CUS and not (8 * rem <= 3 * PLAN_CUS and K >= 4096)) or K % 256 or K // 2 < 512:
        return 0, 0
    g = 1
    while g < 3 and 2 * (rem << (g + 1)) <= PLAN_CUS and K % (128 << (g + 1)) == 0 and (K >> (g + 1)) >= 1024:
        g += 1
    return rem, g


def _plans(wl: Workload):
    """(the first GEMM's plan, over K1; the second's, over D)."""
    rt = (wl.M + 255) // 256
    return _plan(rt * (wl.D // 256), wl.K1), _plan(rt * (wl.N2 // 256), wl.D)


def _al(x: int) -> int:
    return (x + 255) // 256 * 256


def _room(plan) -> int:
    t, g = plan
    S = 1 << g
    return _al(4 * t * (S - 1)) + t * (2 * S - 2) * SLOT_BYTES if t else 0


def _tickets(ws: torch.Tensor, wl: Workload, unfused: bool = False):
    """The tickets after a call: (the first GEMM's, the second GEMM's), S - 1 per split tile.  The split room follows
    the workspace's base part: the second GEMM's tickets and slots, then the first GEMM's."""
    total = cb.coda_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, int(unfused))
    base = total - cb.coda_workspace_split_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, int(unfused))
    p1, p2 = _plans(wl)
    n = lambda p: p[0] * ((1 << p[1]) - 1)
    g2 = ws[base: base + 4 * n(p2)].view(torch.int32).cpu()
    o1 = base + _room(p2)
    g1 = ws[o1: o1 + 4 * n(p1)].view(torch.int32).cpu()
    return g1, g2


def _both_tickets_taken(ws, wl, unfused=False) -> bool:
    return all(bool((g == 2).all()) for g in _tickets(ws, wl, unfused))


def _run(d: DeviceInputs, unfused=False, split=True):
    box = []
    h, y, r = run_block(d, unfused=unfused, split=split, ws_out=box)
    return h, y, r, box[0]


# a QKV projection with 2 key-value heads of 64 at the 1B hidden size: 32 x 9 = 288 tiles, a last wave of 32
QKV_2KV = Workload("1b_qkv_2kv", M=8192, K1=2048, D=2048, N2=2304, epi=EPI_IDENTITY, eps=1e-5, seed=65)

# the 1B MLP-out -> QKV block on 1024 rows (an eighth of the rows, as one GPU of eight holds them): the first GEMM's
# 4 x 8 = 32 tiles and the second's 4 x 12 = 48 tiles are all split
QKV_ROWS1024 = Workload("1b_mlp_out_qkv_1024_rows", M=1024, K1=8192, D=2048, N2=3072, epi=EPI_IDENTITY, eps=1e-5,
                        seed=66)

SMALL = [
    Workload("split_swiglu_ragged", M=300, K1=256, D=1024, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=61),
    Workload("split_identity_one_row_tile", M=64, K1=128, D=2048, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=62),
    # D / 256 = 17: the reduce is a kernel of its own, the second product reads r; halves of K = 2176
    Workload("split_no_fold", M=130, K1=128, D=4352, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=63),
    # the first GEMM split (4 tiles over K1 = 2048), the second not (D = 512)
    Workload("split_first_gemm", M=300, K1=2048, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=67),
    # both GEMMs split: 8 tiles over K1 = 1024, 4 tiles over D = 1024
    Workload("split_both_gemms", M=260, K1=1024, D=1024, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=68),
    # the second GEMM's 2 tiles in 4 pieces each (K = D = 4096, the tree's two levels)
    Workload("split_four_pieces", M=130, K1=256, D=4096, N2=512, epi=EPI_IDENTITY, eps=1e-5, seed=69),
    # the first GEMM's one tile in 8 pieces (K1 = 8192, three levels), on 64 rows (the small-row form)
    Workload("split_eight_pieces", M=64, K1=8192, D=256, N2=256, epi=EPI_IDENTITY, eps=1e-5, seed=70),
]


def test_plan_matches_the_written_rule():
    for wl in SMALL + FULL + [WORKLOADS["1b_mlp_out_qkv"], WORKLOADS["1b_attn_out_mlp_in"], WORKLOADS["tiny"]]:
        p1, p2 = _plans(wl)
        for unfused in (False, True):
            assert cb.coda_workspace_split_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, 0, int(unfused)) == \
                _room(p1) + _room(p2), (wl.name, unfused)
    none = ((0, 0), (0, 0))
    assert _plans(WORKLOADS["1b_mlp_out_qkv"]) == none   # 256 tiles; a last wave of 128 tiles: over a quarter
    assert _plans(WORKLOADS["1b_attn_out_mlp_in"]) == none
    assert _plans(QKV_2KV) == ((0, 0), (32, 1))
    assert _plans(QKV_ROWS1024) == ((32, 2), (48, 1))      # the first GEMM in 4 pieces of 2048
    assert _plans(ROWS3072) == ((96, 1), (12, 1))
    assert [_plans(w) for w in SMALL] == [((0, 0), (8, 1)), ((0, 0), (2, 1)), ((0, 0), (2, 1)), ((4, 1), (0, 0)),
                                          ((8, 1), (4, 1)), ((0, 0), (2, 2)), ((1, 3), (0, 0))]


@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_split_small_against_oracle(wl, unfused):
    _say(f"[gpu] split {'unfused' if unfused else 'fused'} {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    (t1, _), (t2, _) = _plans(wl)
    assert t1 + t2 > 0
    h, y, r, ws = _run(d, unfused)
    assert _both_tickets_taken(ws, wl, unfused), "a split tile did not take both tickets"
    form = "unfused" if unfused else "fused"
    oh, orr, oy = oracle_rows(inp, form=form)
    check_h(f64(h), oh)
    check_y(f64(y), oy)
    if unfused:
        np.testing.assert_allclose(f64(r), orr, rtol=2e-3)
    else:
        np.testing.assert_allclose(f64(r), orr, rtol=2e-5)
        check_roundpts(f64(y), oracle_rows(inp, form="roundpts")[2])
    # the same block on whole tiles: the outputs differ only by the order of the fp32 sums (h and r not at all where
    # the first GEMM is not split)
    h0, y0, r0, _ = _run(d, unfused, split=False)
    if t1 == 0:
        assert torch.equal(h.view(torch.int16), h0.view(torch.int16))
        assert torch.equal(r.view(torch.int32), r0.view(torch.int32))
    else:
        assert normwise(f64(h), f64(h0)) <= CLOSE_NORMWISE
        np.testing.assert_allclose(f64(r), f64(r0), rtol=1e-5)
    g, w = f64(y), f64(y0)
    assert normwise(g, w) <= CLOSE_NORMWISE and mae_rel(g, w) <= CLOSE_MAE_REL


def test_split_is_deterministic():
    """The half that finishes second adds the other's fp32 slot to its own accumulators; fp32 addition is
    commutative, so the result does not depend on the order in which the halves finish."""
    wl = SMALL[0]
    _say(f"[gpu] split determinism {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    ys = [_run(d)[1] for _ in range(4)]
    for y in ys[1:]:
        assert torch.equal(y.view(torch.int16), ys[0].view(torch.int16))


def test_split_tail_after_a_whole_wave():
    """264 tiles: 256 whole tiles, then the last 8 (in the tile order) split; rows covering every row tile
    against the oracle, every row against the whole-tile run."""
    wl = Workload("split_tail", M=2048, K1=256, D=1024, N2=8448, epi=EPI_IDENTITY, eps=1e-5, seed=64)
    _say(f"[gpu] split tail {wl}")
    assert _plans(wl) == ((0, 0), (8, 1))
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h, y, r, ws = _run(d)
    assert _both_tickets_taken(ws, wl)
    rows = sample_rows_covering(wl.M, n=64, seed=5)
    oh, orr, oy = oracle_rows(inp, rows)
    hg, yg = f64(h), f64(y)
    check_h(hg[rows], oh)
    check_y(yg[rows], oy)
    np.testing.assert_allclose(f64(r)[rows], orr, rtol=2e-5)
    _, y0, _, _ = _run(d, split=False)
    w = f64(y0)
    assert normwise(yg, w) <= CLOSE_NORMWISE and mae_rel(yg, w) <= CLOSE_MAE_REL


# 3072 rows over K1 = 4096: the first GEMM's 96 tiles, three eighths of the CUs, split in two (K >= 4096); the
# second GEMM's 12 tiles in two
ROWS3072 = Workload("rows3072_k1_4096", M=3072, K1=4096, D=2048, N2=256, epi=EPI_IDENTITY, eps=1e-5, seed=71)
FULL = [QKV_2KV, QKV_ROWS1024, ROWS3072]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_split_full_size(wl, unfused):
    _say(f"[gpu] split full size {'unfused' if unfused else 'fused'} {wl}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h1, y1, r1, ws = _run(d, unfused)
    assert _both_tickets_taken(ws, wl, unfused)
    del ws
    _, y2, _, _ = _run(d, unfused)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # a row in every row tile (the split tiles are the last in the tile order, in the last row tiles), the ends
    rows = np.array(sorted({0, 1, 2, 3, wl.M - 2, wl.M - 1} | {256 * t + (37 * t) % 256 for t in range(wl.M // 256)}))
    oh, orr, oy = oracle_rows(inp, rows, form="unfused" if unfused else "fused")
    check_h(f64(h1)[rows], oh)
    check_y(f64(y1)[rows], oy)
    np.testing.assert_allclose(f64(r1)[rows], orr, rtol=2e-3 if unfused else 2e-5)
    _, y0, _, _ = _run(d, unfused, split=False)
    g, w = f64(y1), f64(y0)
    assert normwise(g, w) <= CLOSE_NORMWISE and mae_rel(g, w) <= CLOSE_MAE_REL


def test_split_rope_block():
    """coda_block_fwd_rope on a split shape: ticket 2 on every tile, the rotation against the oracle's, the
    columns past the rotated span equal to the plain (also split) block's bit for bit."""
    wl = SMALL[1]
    seq_len, n_rot, base = 48, 256, 10000.0
    _say(f"[gpu] split rope {wl.name}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device="cuda")
    y = torch.full((wl.M, wl.N2), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_IDENTITY, device="cuda")
    ws.fill_(0xFF)
    cb.coda_block_fwd_rope(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, seq_len, n_rot, base, h, y, ws)
    torch.cuda.synchronize()
    assert _both_tickets_taken(ws, wl)
    oh, _, oy = oracle_rows(inp)
    check_h(f64(h), oh)
    check_y(f64(y), oracle.rope_rows(oy, 64, n_rot, seq_len, base))
    _, y_plain, _ = run_block(d)
    assert torch.equal(y[:, n_rot:].view(torch.int16), y_plain[:, n_rot:].view(torch.int16))


def test_split_save_z():
    """The forward that keeps z on a split shape: y equal to coda_block_fwd's, z equal to the identity-epilogue
    block's y (the same tiles, split the same way), bit for bit."""
    wl = SMALL[0]
    _say(f"[gpu] split save z {wl.name}")
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
    assert torch.equal(y.view(torch.int16), y_plain.view(torch.int16))
    # SwiGLU tiles hold 128 gate and the matching 128 up columns, identity tiles 256 contiguous columns: the tile
    # grid is the same, the accumulation per column too, so z is the identity block's y bit for bit
    assert torch.equal(z.view(torch.int16), z_plain.view(torch.int16))


def _split_shapes(n: int = 10, seed: int = 4096):
    """n seeded shapes whose first or second GEMM (or both) splits, in 2, 4 or 8 pieces, at most about 0.5 G
    multiply-adds each (the oracle's fp64 cost)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        M = int(rng.integers(1, 600))
        if len(out) % 3 == 2:  # a long first product over a narrow D: eight pieces where its tiles are few
            K1, D = 8192, 256 * int(rng.choice([1, 2]))
        else:
            K1 = int(rng.choice([256, 1024, 2048, 4096, 8192]))
            D = 256 * int(rng.choice([1, 2, 4, 8, 16]))
        N2 = 256 * int(rng.integers(1, 5))
        epi = int(rng.integers(0, 2))
        wl = Workload(f"split_rand{len(out)}_M{M}_K{K1}_D{D}_N{N2}_{'swiglu' if epi else 'id'}", M=M, K1=K1, D=D,
                      N2=N2, epi=EPI_SWIGLU if epi else EPI_IDENTITY, eps=1e-5, seed=300 + len(out))
        (t1, _), (t2, _) = _plans(wl)
        if t1 + t2 == 0 or M * (K1 * D + D * N2) > 5e8:
            continue
        out.append(wl)
    return out


SPLIT_RANDOM = _split_shapes()


def test_split_random_shapes_cover_every_piece_count():
    lgs = {g for wl in SPLIT_RANDOM for (t, g) in _plans(wl) if t}
    assert lgs == {1, 2, 3}, lgs


@pytest.mark.parametrize("wl", SPLIT_RANDOM, ids=[w.name for w in SPLIT_RANDOM])
def test_split_random_shape(wl):
    """Fused and unfused, every element against the oracle, both GEMMs' tickets, and the whole-tile run."""
    _say(f"[gpu] split random shape {wl} plans {_plans(wl)}")
    inp = make_inputs(wl)
    d = DeviceInputs(inp)
    for unfused in (False, True):
        h, y, r, ws = _run(d, unfused)
        assert _both_tickets_taken(ws, wl, unfused)
        oh, orr, oy = oracle_rows(inp, form="unfused" if unfused else "fused")
        check_h(f64(h), oh)
        check_y(f64(y), oy)
        np.testing.assert_allclose(f64(r), orr, rtol=2e-3 if unfused else 2e-5)
        _, y0, _, _ = _run(d, unfused, split=False)
        g, w = f64(y), f64(y0)
        assert normwise(g, w) <= CLOSE_NORMWISE and mae_rel(g, w) <= CLOSE_MAE_REL
