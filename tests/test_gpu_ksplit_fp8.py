"""GPU tests of the split of the GEMMs' last waves of tiles in the e4m3 blocks, through the C ABI.

The e4m3 blocks (coda_block_fwd_fp8 with per-row scales, coda_block_fwd_fp8_mx with block-scaled A operand, and
coda_block_unfused_fp8) split their products' last waves as the bf16 blocks do, by a rule of their own (an e4m3 K
value costs the MFMAs half a bf16 one, the exchange of the pieces' sums the same; coda_workspace_bytes in
include/coda.h states it).
A piece of a block-scaled tile starts its A scales as many K steps in as its A codes.  Checked here:
- the room each block's workspace gets matches the rule written out here, and after a call every split tile's
  tickets read 2 (all its pieces ran);
- small shapes that split the second GEMM (with the reduce folded in and as a kernel of its own), the first, both,
  and in 4 and 8 pieces: h and y against the oracle on every element, the quantisers' codes and scales bit for bit
  from the GPU's own h, the block-scaled y against the oracle's own block-scaled operand at the storage-rounding
  bar, and the same block on whole tiles (a workspace without the split room): h, r, codes and scales equal bit for
  bit where the first GEMM is not split, y within the fp32 summation-order difference;
- outputs bit-identical run to run;
- full size: a QKV projection with one key-value head of 128 (multi-query attention) at the 8B hidden size in e4m3
  (8192 rows, D = 4096, 4096 + 2 x 128 output columns: 544 tiles in the second GEMM, a last wave of 32 split in two):
  every row of the per-row block against the oracle, a row in every row tile of the block-scaled one, and every row
  of both against their whole-tile runs; the 1B shape with 2 key-value heads (a last wave of 32 over K = 2048) is
  not split.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, Workload, make_inputs

from parity import check_all_rows, check_h, check_roundpts, check_y, f64, mae_rel, normwise, sample_rows_covering
from test_gpu_fp8 import (_align256, _check_mx_exact, _check_rowq_exact, _mx_scales_from_workspace, _oracle_fp8,
                          _oracle_fp8_chunks, _oracle_mx_y, _panels_to_rows, _ws_rowq)

pytestmark = pytest.mark.gpu

SLOT_BYTES = 512 * 128 * 4  # one workgroup's fp32 accumulators
PLAN_CUS = 256              # the split room is planned for MI355X's CU count
CLOSE_NORMWISE = 1e-2       # y of the split and whole-tile runs: the same products summed in another fp32 order
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


def _plan8(tiles: int, K: int):
    """The split rule for e4m3 operands written out: (split tiles, log2 of the pieces per tile).  A last wave that
    fills at most an eighth of the CUs (three eighths where K >= 8192) splits in two where K gives two pieces of at
    least 2048 (K a multiple of 512); in more, up to 8, while all pieces stay within half of the CUs and each keeps
    at least 2048 of K (a multiple of 256)."""
    rem = tiles % PLAN_CUS
    if rem == 0 or (8 * rem > PLAN_CUS and not (8 * rem <= 3 * PLAN_CUS and K >= 8192)) or K % 512 or K // 2 < 2048:
        return 0, 0
    g = 1
    while g < 3 and 2 * (rem << (g + 1)) <= PLAN_CUS and K % (256 << (g + 1)) == 0 and (K >> (g + 1)) >= 2048:
        g += 1
    return rem, g


def _plans(wl: Workload):
    """(the first GEMM's plan, over K1; the second's, over D)."""
    rt = (wl.M + 255) // 256
    return _plan8(rt * (wl.D // 256), wl.K1), _plan8(rt * (wl.N2 // 256), wl.D)


def _room(plan) -> int:
    t, g = plan
    S = 1 << g
    return _align256(4 * t * (S - 1)) + t * (2 * S - 2) * SLOT_BYTES if t else 0


KINDS = {"fused": (1, 0), "mx": (2, 0), "unfused": (1, 1)}  # (fp8 argument, unfused)


def _tickets_all_taken(ws: torch.Tensor, wl: Workload, kind: str) -> bool:
    """Every split tile's S - 1 tickets read 2 after a call.  The split room follows the workspace's base part: the
    second GEMM's tickets and slots, then the first GEMM's."""
    fp8, unfused = KINDS[kind]
    total = cb.coda_workspace_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, fp8, unfused)
    base = total - cb.coda_workspace_split_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, fp8, unfused)
    p1, p2 = _plans(wl)
    n = lambda p: p[0] * ((1 << p[1]) - 1)
    g2 = ws[base: base + 4 * n(p2)].view(torch.int32).cpu()
    o1 = base + _room(p2)
    g1 = ws[o1: o1 + 4 * n(p1)].view(torch.int32).cpu()
    return bool((g1 == 2).all()) and bool((g2 == 2).all())


def _run8(inp, kind: str, split: bool = True):
    """One call of the e4m3 block `kind` on NaN-poisoned outputs and a 0xFF-filled workspace."""
    wl = inp.wl
    dev = "cuda"
    fp8, unfused = KINDS[kind]
    args = [t.to(dev) for t in (inp.Xq, inp.sx, inp.W1q, inp.sw1, inp.R, inp.gamma, inp.W2q, inp.sw2)]
    h = torch.full((wl.M, wl.D), float("nan"), dtype=torch.bfloat16, device=dev)
    y = torch.full((wl.M, wl.n_out), float("nan"), dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=unfused, device=dev, fp8=fp8, split=split)
    ws.fill_(0xFF)
    fn = {"fused": cb.coda_block_fwd_fp8, "mx": cb.coda_block_fwd_fp8_mx, "unfused": cb.coda_block_unfused_fp8}[kind]
    fn(*args, wl.eps, wl.epi, h, y, ws)
    torch.cuda.synchronize()
    return h, y, ws


def _mx_parts(ws: torch.Tensor, M: int, D: int):
    """r, the block-scaled codes [M, D] and their exponents [M, D/32] from the block-scaled path's workspace."""
    off_r = _align256((D // 256) * M * 4)
    off_q = off_r + _align256(M * 4)
    off_s = off_q + _align256(M * D)
    wsc = ws.cpu()
    r = wsc[off_r: off_r + 4 * M].view(torch.float32).numpy()
    q = _panels_to_rows(wsc[off_q: off_q + M * D], M, D).numpy()
    return r, q, _mx_scales_from_workspace(wsc, M, D, off_s)


# a QKV projection with one key-value head of 128 at the 8B hidden size, e4m3: 32 x 17 = 544 tiles, a last wave of 32
QKV_MQA_E4M3 = Workload("8b_qkv_mqa_e4m3", M=8192, K1=2048, D=4096, N2=4352, epi=EPI_IDENTITY, eps=1e-5, fp8=True,
                        seed=75)
# the 1B QKV projection with 2 key-value heads of 64: a last wave of 32 tiles over K = 2048, not split in e4m3
QKV_2KV_E4M3 = Workload("1b_qkv_2kv_e4m3", M=8192, K1=2048, D=2048, N2=2304, epi=EPI_IDENTITY, eps=1e-5, fp8=True,
                        seed=77)

SMALL = [
    # the second GEMM's 8 tiles in two over K = 4096 (the block-scaled path folds the reduce in)
    Workload("e4m3_split_second", M=300, K1=256, D=4096, N2=1024, epi=EPI_SWIGLU, eps=1e-5, fp8=True, seed=71),
    # the first GEMM's 4 tiles in two over K1 = 4096, the second not (D = 512)
    Workload("e4m3_split_first", M=300, K1=4096, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, fp8=True, seed=72),
    # both: 32 tiles over K1 = 4096 and 4 tiles over D = 4096, in two
    Workload("e4m3_split_both", M=260, K1=4096, D=4096, N2=512, epi=EPI_IDENTITY, eps=1e-5, fp8=True, seed=73),
    # the second GEMM's 2 tiles in four over K = D = 8192 (D / 256 = 32: the reduce is a kernel of its own)
    Workload("e4m3_split_four_pieces", M=130, K1=256, D=8192, N2=512, epi=EPI_IDENTITY, eps=1e-5, fp8=True,
             seed=74),
    # the first GEMM's one tile in eight over K1 = 16384
    Workload("e4m3_split_eight_pieces", M=64, K1=16384, D=256, N2=256, epi=EPI_IDENTITY, eps=1e-5, fp8=True,
             seed=76),
]

EXPECTED = {  # (first GEMM's plan, second GEMM's plan)
    "e4m3_split_second": ((0, 0), (8, 1)),
    "e4m3_split_first": ((4, 1), (0, 0)),
    "e4m3_split_both": ((32, 1), (4, 1)),
    "e4m3_split_four_pieces": ((0, 0), (2, 2)),
    "e4m3_split_eight_pieces": ((1, 3), (0, 0)),
    "8b_qkv_mqa_e4m3": ((0, 0), (32, 1)),
    "1b_qkv_2kv_e4m3": ((0, 0), (0, 0)),
}


def test_plan_matches_the_written_rule():
    for wl in SMALL + [QKV_MQA_E4M3, QKV_2KV_E4M3]:
        assert _plans(wl) == EXPECTED[wl.name], wl.name
        p1, p2 = _plans(wl)
        for kind, (fp8, unfused) in KINDS.items():
            got = cb.coda_workspace_split_bytes(wl.M, wl.K1, wl.D, wl.N2, wl.epi, fp8, unfused)
            assert got == _room(p1) + _room(p2), (wl.name, kind)


def _check_against_whole_tiles(wl, kind, hs, ys, wss, hw, yw, wsw):
    """The split run against the whole-tile run of the same block: bit-identical h, r and quantised operand where
    the first GEMM is not split, y within the fp32 summation-order difference."""
    p1, p2 = _plans(wl)
    if p1[0] == 0:
        assert torch.equal(hs, hw), "h differs from the whole-tile run"
        if kind == "mx":
            for a, b in zip(_mx_parts(wss, wl.M, wl.D), _mx_parts(wsw, wl.M, wl.D)):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), "r / codes / scales differ"
        elif kind == "fused":
            a, b = _ws_rowq(wss, wl.M, wl.D), _ws_rowq(wsw, wl.M, wl.D)
            for k in ("r", "q", "s", "rs"):
                assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), f"{k} differs"
        g, o = f64(ys), f64(yw)
        assert normwise(g, o) <= CLOSE_NORMWISE and mae_rel(g, o) <= CLOSE_MAE_REL
    else:  # h itself takes another fp32 summation order: at most a bf16 rounding apart
        assert normwise(f64(hs), f64(hw)) <= 2.0 ** -7


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_split_small_against_oracle(wl, kind):
    _say(f"[gpu] e4m3 split {kind} {wl.name} M={wl.M} K1={wl.K1} D={wl.D} N2={wl.N2} plans={_plans(wl)}")
    inp = make_inputs(wl)
    h, y, ws = _run8(inp, kind)
    assert _tickets_all_taken(ws, wl, kind)
    oh, orr, oy = _oracle_fp8(inp, form="unfused" if kind == "unfused" else "fused")
    check_h(f64(h), oh)
    check_y(f64(y), oy, fp8=True)
    if kind == "fused":
        w = _ws_rowq(ws, wl.M, wl.D)
        np.testing.assert_allclose(w["r"], orr, rtol=2e-5)
        _check_rowq_exact(w, h, inp.gamma)
    elif kind == "mx":
        r, q, e = _mx_parts(ws, wl.M, wl.D)
        np.testing.assert_allclose(r, orr, rtol=2e-5)
        _check_mx_exact(q, e, h, inp.gamma)
        check_roundpts(f64(y), _oracle_mx_y(inp, oh, orr)[0])
    hw, yw, wsw = _run8(inp, kind, split=False)
    _check_against_whole_tiles(wl, kind, h, y, ws, hw, yw, wsw)
    h2, y2, _ = _run8(inp, kind)
    assert torch.equal(h, h2) and torch.equal(y, y2), "split outputs differ run to run"


@pytest.mark.timeout(600)
def test_split_full_size_per_row_all_rows():
    wl = QKV_MQA_E4M3
    _say(f"[gpu] e4m3 split full size, per-row scales, all rows {wl.name}")
    inp = make_inputs(wl)
    h, y, ws = _run8(inp, "fused")
    assert _tickets_all_taken(ws, wl, "fused")
    w = _ws_rowq(ws, wl.M, wl.D)
    _check_rowq_exact(w, h, inp.gamma)
    hw, yw, wsw = _run8(inp, "fused", split=False)
    _check_against_whole_tiles(wl, "fused", h, y, ws, hw, yw, wsw)
    h2, y2, _ = _run8(inp, "fused")
    assert torch.equal(h, h2) and torch.equal(y, y2)
    check_all_rows(wl.M, h, y, torch.from_numpy(w["r"]), _oracle_fp8_chunks(inp), fp8=True, say=_say)


@pytest.mark.timeout(600)
def test_split_full_size_block_scaled():
    wl = QKV_MQA_E4M3
    _say(f"[gpu] e4m3 split full size, block-scaled {wl.name}")
    inp = make_inputs(wl)
    h, y, ws = _run8(inp, "mx")
    assert _tickets_all_taken(ws, wl, "mx")
    r, q, e = _mx_parts(ws, wl.M, wl.D)
    _check_mx_exact(q, e, h, inp.gamma)
    hw, yw, wsw = _run8(inp, "mx", split=False)
    _check_against_whole_tiles(wl, "mx", h, y, ws, hw, yw, wsw)
    rows = sample_rows_covering(wl.M)
    oh, orr, oy = _oracle_fp8(inp, rows=rows)
    g = f64(y)[rows]
    check_h(f64(h)[rows], oh)
    check_y(g, oy, fp8=True)
    check_roundpts(g, _oracle_mx_y(inp, oh, orr)[0])
    np.testing.assert_allclose(r[rows], orr, rtol=2e-5)
