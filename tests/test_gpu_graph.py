"""The entry points under HIP graph capture (torch.cuda.CUDAGraph) and on concurrent streams.  A captured
block, replayed several times with other eager GPU work and synchronisations in between, gives the eager
result bit for bit on every replay, and follows new data copied into its static inputs.  The library enqueues
only kernels (no memset, no allocation, no host synchronisation), which is what makes a call capturable.  Two
blocks in flight on streams of their own with their own workspaces give what each gives alone.
"""
import sys

import torch
import pytest

from gemm_epilogue_fusion_amd import binding as cb
from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, EPI_SWIGLU, WORKLOADS, Workload, make_grads, make_inputs

from parity import DeviceInputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cb.load()


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _capture(fn):
    """Capture fn() (after one eager warm-up call on a side stream, as torch requires) into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


CASES = [WORKLOADS["tiny"],
         Workload("graph_ragged_swiglu", M=300, K1=512, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=21),
         # every tile of the second product split along K: the tickets are cleared by the first kernel of each replay
         Workload("graph_split_swiglu", M=300, K1=256, D=1024, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=23),
         # every tile of the second product as two 128-row halves: two launches of the second GEMM's kernels
         Workload("graph_halves", M=512, K1=256, D=256, N2=2048, epi=EPI_IDENTITY, eps=1e-5, seed=24)]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_block_graph_replays_match_eager(wl):
    _say(f"[gpu] graph replay of the block {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    dev = d.X.device
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
    call = lambda: cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, h, y, ws)
    call()
    torch.cuda.synchronize()
    h_ref, y_ref = h.clone(), y.clone()
    g = _capture(call)
    # other eager work between replays: the unfused baseline on its own buffers and a torch reduction
    hu = torch.empty_like(h)
    yu = torch.empty_like(y)
    wsu = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=1, device=dev)
    for i in range(3):
        h.fill_(float("nan"))
        y.fill_(float("nan"))
        g.replay()
        cb.coda_block_unfused(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, hu, yu, wsu)
        _ = float(yu.float().abs().sum())
        torch.cuda.synchronize()
        assert torch.equal(_bits(h), _bits(h_ref)), f"replay {i}: h differs from the eager call"
        assert torch.equal(_bits(y), _bits(y_ref)), f"replay {i}: y differs from the eager call"
    # new data in the static inputs: the replay computes on it
    X2 = (torch.randn(wl.M, wl.K1, generator=torch.Generator().manual_seed(99))).to(torch.bfloat16).to(dev)
    d.X.copy_(X2)
    h2 = torch.empty_like(h)
    y2 = torch.empty_like(y)
    ws2 = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
    cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, h2, y2, ws2)
    g.replay()
    torch.cuda.synchronize()
    assert not torch.equal(_bits(y2), _bits(y_ref))
    assert torch.equal(_bits(h), _bits(h2)) and torch.equal(_bits(y), _bits(y2))


def test_backward_graph_replays_match_eager():
    wl = Workload("graph_bwd", M=256, K1=256, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=22)
    _say(f"[gpu] graph replay of the backward {wl.name}")
    d = DeviceInputs(make_inputs(wl))
    dev = d.X.device
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
    cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, h, y, ws)
    r = cb.workspace_r(ws, wl.M, wl.D).clone()
    dz, dho = (t.to(dev) for t in make_grads(wl))
    outs = (torch.empty(wl.M, wl.K1, dtype=torch.bfloat16, device=dev),
            torch.empty(wl.K1, wl.D, dtype=torch.float32, device=dev),
            torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev),
            torch.empty(wl.D, dtype=torch.float32, device=dev),
            torch.empty(wl.D, wl.N2, dtype=torch.float32, device=dev))
    wsb = cb.alloc_bwd_workspace(wl.M, wl.K1, wl.D, wl.N2, device=dev)
    call = lambda: cb.coda_block_bwd(d.X, d.W1, h, r, d.gamma, d.W2, dz, dho, *outs, wsb)
    call()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]
    g = _capture(call)
    for i in range(3):
        for o in outs:
            o.fill_(float("nan"))
        g.replay()
        cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, torch.empty_like(h), torch.empty_like(y),
                          cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev))
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(_bits(o), _bits(ref)), f"replay {i}: a gradient differs from the eager call"


def test_concurrent_streams_distinct_workspaces():
    """Blocks in flight at once on several streams, each with its own workspace (the documented condition for
    concurrent calls), give the results each gives alone, bit for bit."""
    wls = [Workload("stream_a", M=513, K1=256, D=512, N2=1024, epi=EPI_SWIGLU, eps=1e-5, seed=31),
           Workload("stream_b", M=300, K1=384, D=768, N2=512, epi=0, eps=1e-5, seed=32),
           # the second product split along K: each call's tickets and slots live in its own workspace
           Workload("stream_c_split", M=200, K1=256, D=2048, N2=512, epi=0, eps=1e-5, seed=33),
           # the second product's 4 tiles as 128-row halves
           Workload("stream_d_halves", M=450, K1=256, D=512, N2=512, epi=0, eps=1e-5, seed=34)]
    _say("[gpu] concurrent streams " + ", ".join(w.name for w in wls))
    runs = []
    for wl in wls:
        d = DeviceInputs(make_inputs(wl))
        dev = d.X.device
        ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
        outs = [(torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev),
                 torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)) for _ in range(2)]
        runs.append((wl, d, ws, outs))
    for wl, d, ws, outs in runs:  # alone, one after the other
        cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, outs[0][0], outs[0][1], ws)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in runs]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    for _ in range(3):  # interleaved launches on the streams
        for s, (wl, d, ws, outs) in zip(streams, runs):
            with torch.cuda.stream(s):
                cb.coda_block_fwd(d.X, d.W1, d.R, d.gamma, d.W2, wl.eps, wl.epi, outs[1][0], outs[1][1], ws)
    torch.cuda.synchronize()
    for wl, d, ws, outs in runs:
        assert torch.equal(_bits(outs[0][0]), _bits(outs[1][0])), wl.name
        assert torch.equal(_bits(outs[0][1]), _bits(outs[1][1])), wl.name
