"""GPU parity of the cross-entropy of a vocabulary projection (coda_ce_fwd, logits never stored) and of its
unfused baseline (coda_ce_unfused, bf16 logits stored and read back) against the fp64 oracle.

Bars (derived from the arithmetic, written here):
  fused   : |loss - o| and |lse - o| <= 5e-5 + 2^-18 max|z_row|.  The logits are fp32 sums of D bf16 products
            (accumulation error a few tens of fp32 ulps of the row's largest logit at these D), lse carries
            that error, and exp2 and the sums of V fp32 terms add a few 1e-7 relative.  Dropping a single
            256-column tile of the vocabulary moves lse by log(1 + 1/T) >= 2e-3 at T = 501, well above the bar
            (max|z_row| is about 4 there).
  unfused : the logits are rounded to bf16 first (unit roundoff 2^-8: relative error at most 2^-8 each), so
            lse moves by at most 2^-8 max|z_row| and the loss by twice that: |loss - o| <= 2^-7 max|z_row| + 5e-5.
Cases: one tile, several row and column tiles with a ragged last row tile, logits of size ~20 (exp's range
exercised), labels on tile edges, ignored rows (-100), a label >= V (NaN), and the 1B LM-head shape on about 120
sampled rows: two in every 256-row tile, together covering every row position of a 32-row accumulator block.
"""
import sys

import numpy as np
import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import CE_WORKLOADS, CeWorkload, make_ce_inputs

from parity import f64, sample_rows_covering

import oracle

pytestmark = pytest.mark.gpu

ATOL = 5e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


def _run(H, W, labels, unfused=False):
    M, V = H.shape[0], W.shape[1]
    dev = "cuda"
    loss = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((M,), float("nan"), dtype=torch.float32, device=dev)
    ws = cb.alloc_ce_workspace(M, H.shape[1], V, unfused=int(unfused), device=dev)
    ws.fill_(0xFF)
    fn = cb.coda_ce_unfused if unfused else cb.coda_ce_fwd
    fn(H.to(dev), W.to(dev), labels.to(dev), loss, lse, ws)
    torch.cuda.synchronize()
    return loss.cpu().double().numpy(), lse.cpu().double().numpy()


SMALL = [
    CeWorkload("one_tile", M=64, D=128, V=256, seed=41),
    CeWorkload("ragged", M=300, D=256, V=768, ignore_every=7, seed=42),
    CeWorkload("many_tiles", M=777, D=512, V=2560, ignore_every=50, seed=43),
    CeWorkload("wide_logits", M=260, D=384, V=1024, w_std=1.0, seed=44),
]


def _edge_labels(labels, V):
    lab = labels.clone()
    edges = [e % V for e in (0, 255, 256, 257, V - 256, V - 1, 511)] + [-100]
    lab[:len(edges)] = torch.tensor(edges, dtype=torch.int32)
    return lab


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_ce_small(wl, unfused):
    _say(f"[gpu] ce {'unfused' if unfused else 'fused'} {wl}")
    H, W, labels = make_ce_inputs(wl)
    labels = _edge_labels(labels, wl.V)
    loss, lse = _run(H, W, labels, unfused)
    oloss, olse = oracle.cross_entropy(f64(H), f64(W), labels.numpy())
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    assert np.all(loss[labels.numpy() < 0] == 0.0)
    if unfused:
        zmax = np.max(np.abs(f64(H) @ f64(W)), axis=1)
        bound = 2.0 ** -7 * zmax + ATOL
        assert np.all(np.abs(loss - oloss) <= bound), np.max(np.abs(loss - oloss) - bound)
        assert np.all(np.abs(lse - olse) <= bound)
    else:
        _check_fused(loss, lse, oloss, olse, f64(H), f64(W))


def _check_fused(loss, lse, oloss, olse, H, W):
    bound = ATOL + 2.0 ** -18 * np.max(np.abs(H @ W), axis=1)
    err = np.maximum(np.abs(loss - oloss), np.abs(lse - olse))
    _say(f"    max error {np.max(err):.3e}, max error / bar {np.max(err / bound):.3f}")
    assert np.all(err <= bound), f"max error / bar {np.max(err / bound):.3f}"


def test_ce_label_out_of_range_is_nan():
    wl = SMALL[1]
    H, W, labels = make_ce_inputs(wl)
    labels[3] = wl.V
    labels[4] = wl.V + 1000
    for unfused in (False, True):
        loss, lse = _run(H, W, labels, unfused)
        assert np.isnan(loss[3]) and np.isnan(loss[4])
        assert np.all(np.isfinite(lse)) and np.all(np.isfinite(np.delete(loss, [3, 4])))


def test_ce_deterministic():
    wl = SMALL[2]
    H, W, labels = make_ce_inputs(wl)
    a = _run(H, W, labels)
    b = _run(H, W, labels)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_ce_full_size_sampled_rows():
    wl = CE_WORKLOADS["1b_lm_head"]
    _say(f"[gpu] ce full size {wl}")
    H, W, labels = make_ce_inputs(wl)
    loss, lse = _run(H, W, labels)
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    rows = sample_rows_covering(wl.M, n=16, seed=3)
    Hs, Wd = f64(H[rows]), f64(W)
    oloss, olse = oracle.cross_entropy(Hs, Wd, labels[rows].numpy())
    _check_fused(loss[rows], lse[rows], oloss, olse, Hs, Wd)


def _random_shapes(n: int = 8, seed: int = 555):
    """Seeded shapes within the cross-entropy's rules (D a multiple of 128, V of 256, any M), some with ignored
    labels."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 255, 257]) if i < 2 else rng.integers(1, 700))
        D = 128 * int(rng.integers(1, 5))
        V = 256 * int(rng.integers(1, 13))
        ign = int(rng.choice([0, 3, 11]))
        out.append(CeWorkload(f"cerand{i}_M{M}_D{D}_V{V}_ign{ign}", M=M, D=D, V=V, ignore_every=ign, seed=500 + i))
    return out


RANDOM = _random_shapes()


@pytest.mark.parametrize("wl", RANDOM, ids=[w.name for w in RANDOM])
@pytest.mark.parametrize("unfused", [False, True], ids=["fused", "unfused"])
def test_ce_random_shape(wl, unfused):
    _say(f"[gpu] ce random {'unfused' if unfused else 'fused'} {wl}")
    H, W, labels = make_ce_inputs(wl)
    loss, lse = _run(H, W, labels, unfused)
    oloss, olse = oracle.cross_entropy(f64(H), f64(W), labels.numpy())
    assert np.all(np.isfinite(loss)) and np.all(np.isfinite(lse))
    assert np.all(loss[labels.numpy() < 0] == 0.0)
    if unfused:
        bound = 2.0 ** -7 * np.max(np.abs(f64(H) @ f64(W)), axis=1) + ATOL
        assert np.all(np.abs(loss - oloss) <= bound) and np.all(np.abs(lse - olse) <= bound)
    else:
        _check_fused(loss, lse, oloss, olse, f64(H), f64(W))
