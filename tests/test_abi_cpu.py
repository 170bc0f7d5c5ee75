"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function include/coda.h
declares, and rejects bad arguments with the documented status before enqueuing anything.

Pointers here are fake, aligned integers: validation never dereferences them, and no test below reaches a
launch on a machine that has a GPU.
"""
import ctypes
import os
import re

import pytest
import torch

from gemm_epilogue_fusion_amd import binding as cb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, INVALID, UNSUPPORTED, ALIAS, WORKSPACE, HIP = 0, 1, 2, 3, 4, 5


@pytest.fixture(scope="module")
def lib():
    return cb.load()


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "coda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(coda_\w+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = _declared_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), f"libcoda.so does not export {n}"
    assert set(names) == set(cb.EXPORTS)


def test_version_and_strings(lib):
    assert lib.coda_abi_version() == 1
    assert lib.coda_status_string(0) == b"CODA_OK"
    assert lib.coda_status_string(4) == b"CODA_ERR_WORKSPACE"
    assert lib.coda_status_string(99) == b"CODA_ERR_UNKNOWN"


# fake, 256-byte aligned, non-overlapping "device" addresses
BASE = 1 << 40
GB = 1 << 32


def _args(M=512, K1=256, D=256, N2=512, epi=0, eps=1e-5, ws_bytes=None, **over):
    a = dict(X=BASE, W1=BASE + GB, R=BASE + 2 * GB, gamma=BASE + 3 * GB, W2=BASE + 4 * GB, eps=eps, epi=epi,
             out_h=BASE + 5 * GB, out_y=BASE + 6 * GB, M=M, K1=K1, D=D, N2=N2, ws=BASE + 7 * GB)
    a.update(over)
    need = cb.load().coda_workspace_bytes(a["M"], a["K1"], a["D"], a["N2"], a["epi"], 0, 1)  # fits both paths
    a["ws_bytes"] = need if ws_bytes is None else ws_bytes
    return a


def _call(lib, a, fn="coda_block_fwd"):
    return getattr(lib, fn)(a["X"], a["W1"], a["R"], a["gamma"], a["W2"], a["eps"], a["epi"], a["out_h"],
                            a["out_y"], a["M"], a["K1"], a["D"], a["N2"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["coda_block_fwd", "coda_block_unfused"])
@pytest.mark.parametrize("case,over,want", [
    ("null_X", dict(X=0), INVALID),
    ("null_out_y", dict(out_y=0), INVALID),
    ("misaligned_W2", dict(W2=BASE + 4 * GB + 8), INVALID),
    ("M_zero", dict(M=0), INVALID),
    ("K1_negative", dict(K1=-64), INVALID),
    ("K1_not_128", dict(K1=192), UNSUPPORTED),
    ("D_not_256", dict(D=320), UNSUPPORTED),
    ("N2_not_256", dict(N2=384), UNSUPPORTED),
    # largest sizes: each dimension at most 2^30, each matrix at most 2^31 elements (32-bit row and element
    # indices in the kernels), checked before any pointer range is formed
    ("M_above_2e30", dict(M=(1 << 30) + 1), UNSUPPORTED),
    ("y_above_2e31_elements", dict(M=1 << 20, N2=1 << 12), UNSUPPORTED),
    ("W2_above_2e31_elements", dict(D=1 << 16, N2=1 << 16), UNSUPPORTED),
    ("bad_epi", dict(epi=7), INVALID),
    ("eps_negative", dict(eps=-1.0), INVALID),
    ("eps_nan", dict(eps=float("nan")), INVALID),
    ("eps_inf", dict(eps=float("inf")), INVALID),
    ("out_y_on_X", dict(out_y=BASE + 16), ALIAS),
    ("out_h_on_W1", dict(out_h=BASE + GB), ALIAS),
    ("out_y_on_out_h", dict(out_y=BASE + 5 * GB + 256), ALIAS),
    ("ws_on_gamma", dict(ws=BASE + 3 * GB), ALIAS),
    ("out_h_partly_on_R", dict(out_h=BASE + 2 * GB + 256), ALIAS),
    ("null_workspace", dict(ws=0), WORKSPACE),
    ("small_workspace", dict(ws_bytes=1024), WORKSPACE),
    ("misaligned_workspace", dict(ws=BASE + 7 * GB + 16), WORKSPACE),
])
def test_validation(lib, fn, case, over, want):
    a = _args()
    over = dict(over)
    ws_bytes = over.pop("ws_bytes", None)
    a.update(over)
    if ws_bytes is not None:
        a["ws_bytes"] = ws_bytes
    assert _call(lib, a, fn) == want, lib.coda_last_error()
    assert lib.coda_last_error() != b""


def test_unfused_hidden_limit(lib):
    a = _args(D=8448)
    assert _call(lib, a, "coda_block_unfused") == UNSUPPORTED


def test_workspace_bytes(lib):
    # part [D/256][M] + r [M], each 256-byte aligned; then h*gamma [M, D] bf16 (fused) or T and n (unfused)
    assert lib.coda_workspace_bytes(8192, 2048, 2048, 16384, 1, 0, 0) == 8 * 8192 * 4 + 8192 * 4 + 8192 * 2048 * 2
    assert lib.coda_workspace_bytes(8192, 2048, 2048, 16384, 1, 0, 1) == 8 * 8192 * 4 + 8192 * 4 + 2 * 8192 * 2048 * 2
    assert lib.coda_workspace_bytes(5, 128, 256, 256, 0, 0, 0) == 256 + 256 + 5 * 256 * 2
    assert lib.coda_workspace_r_offset(8192, 2048) == 8 * 8192 * 4
    assert lib.coda_workspace_bytes(0, 64, 256, 256, 0, 0, 0) == 0


def test_step_entry_points_validate(lib):
    assert lib.coda_partial_rms_reduce(0, 8, 100, 2048, 1e-5, BASE, None) == INVALID
    assert lib.coda_partial_rms_reduce(BASE, 0, 100, 2048, 1e-5, BASE + GB, None) == INVALID
    assert lib.coda_partial_rms_reduce(BASE, 8, 100, 2048, -1.0, BASE + GB, None) == INVALID
    assert lib.coda_partial_rms_reduce(BASE, 8, 100, 2048, 1e-5, BASE + 256, None) == ALIAS
    g1 = lambda **o: lib.coda_gemm1_residual_partial_rms(
        o.get("X", BASE), BASE + GB, BASE + 2 * GB, BASE + 3 * GB, o.get("h", BASE + 4 * GB), o.get("hg", BASE + 5 * GB),
        BASE + 6 * GB, 100, o.get("K1", 256), 256, None)
    assert g1(K1=192) == UNSUPPORTED
    assert g1(X=0) == INVALID
    assert g1(hg=BASE + 4 * GB + 512) == ALIAS   # out_hg overlapping out_h
    assert g1(hg=BASE + 2 * GB) == ALIAS         # out_hg on R (only out_h may alias R)
    assert lib.coda_gemm2_rowscale(BASE, BASE + GB, BASE + 2 * GB, 2, BASE + 4 * GB, 100, 256, 512, None) == INVALID
    assert lib.coda_gemm2_rowscale(BASE, BASE + GB, BASE + 2 * GB, 0, BASE + 16, 100, 256, 512, None) == ALIAS


def test_panel_step_entry_points_validate(lib):
    g1 = lambda **o: lib.coda_gemm1_residual_partial_rms_panels(
        o.get("X", BASE), BASE + GB, BASE + 2 * GB, BASE + 3 * GB, o.get("h", BASE + 4 * GB), o.get("hg", BASE + 5 * GB),
        BASE + 6 * GB, 100, o.get("K1", 256), 256, None)
    assert g1(K1=192) == UNSUPPORTED
    assert g1(X=0) == INVALID
    assert g1(hg=BASE + 4 * GB + 512) == ALIAS
    # step 3: hg, W2, part, eps, r, epi, y, M, D, N2
    g3 = lambda **o: lib.coda_gemm2_rowscale_panels(
        BASE, BASE + GB, o.get("part", BASE + 2 * GB), o.get("eps", 1e-5), o.get("r", BASE + 3 * GB), o.get("epi", 1),
        o.get("y", BASE + 4 * GB), 100, o.get("D", 256), 512, None)
    assert g3(epi=2) == INVALID
    assert g3(eps=-1.0) == INVALID
    assert g3(eps=float("nan")) == INVALID
    assert g3(D=4352) == UNSUPPORTED                  # the folded reduce takes D <= 4096
    assert g3(r=BASE + 2 * GB + 64) == ALIAS          # r (an output when folding) on part
    assert g3(y=BASE + 3 * GB) == ALIAS               # out_y on r
    assert g3(y=BASE + 16) == ALIAS                   # out_y on hg
    assert g3(D=192) == UNSUPPORTED


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_no_gpu_reports_hip_error(lib):
    """With no GPU, a call that passes validation fails at the launch with CODA_ERR_HIP (no crash)."""
    a = _args()
    assert _call(lib, a) == HIP
    assert b"launch" in lib.coda_last_error()
    # the allowed exact alias out_h == R passes validation and also reaches the launch
    a = _args(out_h=BASE + 2 * GB)
    assert _call(lib, a) == HIP


def test_binding_rejects_host_tensors():
    X = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        cb.coda_block_fwd(X, torch.zeros(64, 256, dtype=torch.bfloat16), torch.zeros(4, 256, dtype=torch.bfloat16),
                          torch.ones(256), torch.zeros(256, 256, dtype=torch.bfloat16), 1e-5, 0,
                          torch.zeros(4, 256, dtype=torch.bfloat16), torch.zeros(4, 256, dtype=torch.bfloat16),
                          torch.zeros(1024, dtype=torch.uint8))


def _call8(lib, a, fn="coda_block_fwd_fp8", sx=BASE + 8 * GB, sw1=BASE + 9 * GB, sw2=BASE + 10 * GB):
    return getattr(lib, fn)(a["X"], sx, a["W1"], sw1, a["R"], a["gamma"], a["W2"], sw2, a["eps"], a["epi"],
                            a["out_h"], a["out_y"], a["M"], a["K1"], a["D"], a["N2"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["coda_block_fwd_fp8", "coda_block_unfused_fp8", "coda_block_fwd_fp8_mx"])
def test_fp8_validation(lib, fn):
    a = _args(M=512, K1=256, D=256, N2=512)
    assert _call8(lib, a, fn, sx=0) == INVALID
    assert _call8(lib, a, fn, sw2=BASE + 10 * GB + 4) == INVALID          # misaligned scale
    assert _call8(lib, _args(K1=384), fn) == UNSUPPORTED                  # e4m3 K step is 256
    assert _call8(lib, a, fn, sw1=BASE + 5 * GB) == ALIAS                  # a scale vector under out_h
    small = dict(a)
    small["ws_bytes"] = 1024
    assert _call8(lib, small, fn) == WORKSPACE


def test_workspace_split_bytes(lib):
    """The room to split each GEMM's last wave, planned for 256 CUs: none where the tiles fill whole waves, the last
    wave fills more than a quarter of the CUs or K (D for the second GEMM, K1 for the first) is below 1024; else, for
    S pieces per tile, S - 1 int32 tickets per tile of the last wave (256-byte aligned) and 2 S - 2 fp32 slots of
    256 KiB per such tile, the second GEMM's room first.  The e4m3 blocks have a rule of their own (an eighth of the
    CUs, three eighths from K = 8192; pieces of at least 2048).  coda_workspace_bytes includes it."""
    al = lambda x: (x + 255) // 256 * 256
    slot = 512 * 128 * 4
    base = lambda M, D, unfused=0: al(D // 256 * M * 4) + al(M * 4) + (2 if unfused else 1) * al(M * D * 2)
    f = lib.coda_workspace_split_bytes
    assert f(8192, 2048, 2048, 16384, 1, 0, 0) == 0          # 32 x 64 tiles: whole waves
    assert f(8192, 8192, 2048, 3072, 0, 0, 0) == 0           # 32 x 12 = 384 tiles: a last wave of 128, over a quarter
    assert lib.coda_workspace_bytes(8192, 8192, 2048, 3072, 0, 0, 0) == base(8192, 2048)
    tail32 = al(32 * 4) + 64 * slot                           # 32 x 9 = 288 tiles: a last wave of 32
    assert f(8192, 2048, 2048, 2304, 0, 0, 0) == tail32
    assert lib.coda_workspace_bytes(8192, 2048, 2048, 2304, 0, 0, 0) == base(8192, 2048) + tail32
    assert f(8192, 2048, 2048, 2304, 0, 0, 1) == tail32       # the unfused bf16 block: the same room
    assert lib.coda_workspace_bytes(8192, 2048, 2048, 2304, 0, 0, 1) == base(8192, 2048, 1) + tail32
    # e4m3 blocks (their own rule): a last wave of at most an eighth of the CUs (three eighths from K = 8192), pieces
    # of at least 2048 of K
    assert f(8192, 2048, 2048, 2304, 0, 1, 0) == 0            # 32 tiles over K = 2048: none
    assert f(8192, 2048, 2048, 2304, 0, 2, 0) == 0
    assert f(8192, 2048, 4096, 4352, 0, 1, 0) == tail32       # 32 x 17 = 544 tiles, K = 4096: a last wave of 32
    assert f(8192, 2048, 4096, 4352, 0, 2, 0) == tail32
    assert f(8192, 2048, 4096, 4352, 0, 1, 1) == tail32
    base8 = al(16 * 8192 * 4) + al(8192 * 4) + al(8192 * 4096) + 2 * al(8192 * 4)  # the fused e4m3 block's base
    assert lib.coda_workspace_bytes(8192, 2048, 4096, 4352, 0, 1, 0) == base8 + tail32
    assert f(8192, 2048, 4096, 4608, 0, 1, 0) == 0            # 32 x 18 = 576 tiles: a last wave of 64
    assert f(8192, 2048, 4096, 4608, 0, 0, 0) == al(64 * 4) + 128 * slot  # (bf16: a quarter, split)
    assert f(300, 256, 4096, 1024, 1, 1, 0) == al(8 * 4) + 16 * slot
    assert f(64, 8192, 256, 256, 0, 1, 0) == al(3 * 4) + 6 * slot   # one tile over K1 = 8192 in four of 2048
    assert f(64, 16384, 256, 256, 0, 1, 0) == al(7 * 4) + 14 * slot  # over K1 = 16384 in eight
    assert f(3072, 4096, 2048, 2048, 0, 1, 0) == 0            # 96 tiles: three eighths only from K = 8192
    assert f(3072, 8192, 2048, 2048, 0, 1, 0) == al(96 * 4) + 192 * slot
    assert f(256 * 65, 256, 1024, 256, 0, 0, 0) == 0            # 65 tiles: the last wave is over a quarter
    assert f(256 * 64, 256, 1024, 256, 0, 0, 0) == al(64 * 4) + 128 * slot  # 64 tiles: exactly a quarter
    assert f(300, 256, 768, 1024, 1, 0, 0) == 0                 # K = 768
    assert f(300, 256, 1024, 1024, 1, 0, 0) == al(8 * 4) + 16 * slot
    assert f(130, 128, 4352, 256, 0, 0, 0) == al(4) + 2 * slot  # one tile, K = 4352 (halves of 2176)
    # the first GEMM too (its tiles ceil(M/256) x D/256 over K1): 300 rows, K1 = 2048, D = 512 -> 4 tiles split
    assert f(300, 2048, 512, 512, 0, 0, 0) == al(4 * 4) + 8 * slot
    # more than two pieces (a tree of S - 1 tickets and 2 S - 2 slots per tile) where all of them stay within half of
    # the CUs and each keeps 1024 of K: 1024 rows of the 1B MLP-out -> QKV block: the second GEMM's 48 tiles in two
    # (K = 2048), then the first GEMM's 32 tiles in four (K1 = 8192; eight would be 256 pieces)
    assert f(1024, 8192, 2048, 3072, 0, 0, 0) == al(48 * 4) + 96 * slot + al(32 * 3 * 4) + 32 * 6 * slot
    # one tile over K = 4096: four pieces of 1024; over K1 = 8192: eight of 1024
    assert f(130, 256, 4096, 512, 0, 0, 0) == al(2 * 3 * 4) + 2 * 6 * slot
    assert f(64, 8192, 256, 256, 0, 0, 0) == al(7 * 4) + 14 * slot
    # over K >= 4096 a last wave of up to three eighths of the CUs splits too: 3072 rows, D = 2048 -> 96 tiles of the
    # first GEMM over K1 = 4096 or 8192 (in two: four would pass half of the CUs), none over K1 = 2048
    assert f(3072, 4096, 2048, 2048, 0, 0, 0) == al(96 * 4) + 192 * slot
    assert f(3072, 8192, 2048, 2048, 0, 0, 0) == al(96 * 4) + 192 * slot
    assert f(3072, 2048, 2048, 2048, 0, 0, 0) == 0
    assert f(256 * 104, 256, 4096, 256, 0, 0, 0) == 0           # 104 tiles: over three eighths
    assert f(0, 256, 2048, 3072, 0, 0, 0) == 0                  # invalid dimensions
    assert f(8192, 256, 2048, 3000, 0, 0, 0) == 0


def test_fp8_workspace_bytes(lib):
    M, D = 8192, 2048
    a = lambda x: (x + 255) // 256 * 256
    base = a(8 * M * 4) + a(M * 4)
    assert lib.coda_workspace_bytes(M, 2048, D, 16384, 1, 1, 0) == base + a(M * D) + 2 * a(M * 4)
    assert lib.coda_workspace_bytes(M, 2048, D, 16384, 1, 1, 1) == base + a(M * D * 2) + a(M * D) + a(M * 4)
    # block-scaled: the codes and one scale byte per 32 values, rows padded to the 256-row tile
    assert lib.coda_workspace_bytes(M, 2048, D, 16384, 1, 2, 0) == base + a(M * D) + a(D // 32 * M)
    assert lib.coda_workspace_bytes(300, 256, 512, 512, 0, 2, 0) == a(2 * 300 * 4) + a(300 * 4) + a(300 * 512) + a(16 * 512)
    assert lib.coda_workspace_bytes(M, 2048, D, 16384, 1, 2, 1) == 0   # no unfused block-scaled form
    assert lib.coda_workspace_bytes(M, 2048, D, 16384, 1, 3, 0) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_fp8_mx_no_gpu_reports_hip_error(lib):
    a = _args(M=512, K1=256, D=256, N2=512)
    assert _call8(lib, a, "coda_block_fwd_fp8_mx") == HIP


# ---- backward entry points ----
def _bargs(M=256, K1=256, D=256, N2=512, unfused=0, **over):
    a = dict(X=BASE, W1=BASE + GB, h=BASE + 2 * GB, r=BASE + 3 * GB, gamma=BASE + 3 * GB + (1 << 20),
             W2=BASE + 4 * GB, dz=BASE + 5 * GB, dh_out=BASE + 6 * GB, dX=BASE + 7 * GB, dW1=BASE + 8 * GB,
             dR=BASE + 9 * GB, dgamma=BASE + 10 * GB, dW2=BASE + 11 * GB, M=M, K1=K1, D=D, N2=N2,
             ws=BASE + 12 * GB)
    a.update(over)
    a["ws_bytes"] = cb.load().coda_bwd_workspace_bytes(a["M"], a["K1"], a["D"], a["N2"], 1)  # fits both paths
    return a


def _bcall(lib, a, fn="coda_block_bwd"):
    return getattr(lib, fn)(a["X"], a["W1"], a["h"], a["r"], a["gamma"], a["W2"], a["dz"], a["dh_out"], a["dX"],
                            a["dW1"], a["dR"], a["dgamma"], a["dW2"], a["M"], a["K1"], a["D"], a["N2"], a["ws"],
                            a["ws_bytes"], None)


@pytest.mark.parametrize("fn", ["coda_block_bwd", "coda_block_bwd_unfused", "coda_block_bwd_w2t"])
@pytest.mark.parametrize("case,over,want", [
    ("null_dz", dict(dz=0), INVALID),
    ("null_out_dW2", dict(dW2=0), INVALID),
    ("misaligned_r", dict(r=BASE + 3 * GB + 4), INVALID),
    ("M_not_128", dict(M=320), UNSUPPORTED),
    ("K1_not_256", dict(K1=384), UNSUPPORTED),
    ("D_not_256", dict(D=320), UNSUPPORTED),
    ("out_dR_on_h", dict(dR=BASE + 2 * GB), ALIAS),
    ("out_dX_on_out_dR", dict(dX=BASE + 9 * GB + 512), ALIAS),
    ("ws_on_dz", dict(ws=BASE + 5 * GB), ALIAS),
    ("null_workspace", dict(ws=0), WORKSPACE),
])
def test_bwd_validation(lib, fn, case, over, want):
    a = _bargs(**over)
    assert _bcall(lib, a, fn) == want, lib.coda_last_error()
    assert lib.coda_last_error() != b""


def _ksplit(rows, cols, k):
    # the fp32 weight-gradient products split K until they have >= 256 workgroups (at most 8 ranges, each
    # range a multiple of 128)
    tiles = -(-rows // 256) * (cols // 256)
    s = 1
    while s < 8 and tiles * s < 256 and k % (128 * s * 2) == 0:
        s *= 2
    return s


@pytest.mark.parametrize("M,K1,D,N2", [(8192, 2048, 2048, 16384), (8192, 8192, 2048, 3072), (256, 256, 256, 512)])
def test_bwd_workspace_bytes(lib, M, K1, D, N2):
    al = lambda x: (x + 255) // 256 * 256
    fused = al(M * D * 2) + al((D // 256) * M * 4) + al(-(-M // 256) * D * 4) + al(M * 4) + 2 * al(M * D * 2)
    s1, s2 = _ksplit(D, K1, M), _ksplit(D, N2, M)
    slabs = max(s1 * D * K1 * 4 if s1 > 1 else 0, s2 * D * N2 * 4 if s2 > 1 else 0)
    shared = max(slabs, D * N2 * 2)  # the split-K slabs and the transposed W2 share one region
    assert lib.coda_bwd_workspace_bytes(M, K1, D, N2, 0) == fused + al(shared)
    assert lib.coda_bwd_workspace_bytes(M, K1, D, N2, 1) == fused + al(M * D * 2) + al(shared)


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_bwd_no_gpu_reports_hip_error(lib):
    a = _bargs()
    assert _bcall(lib, a) == HIP
    a = _bargs(dh_out=0)  # dh_out is optional
    assert _bcall(lib, a) == HIP


def _rcall(lib, a, seq_len=2048, n_rot=256, base=10000.0):
    return lib.coda_block_fwd_rope(a["X"], a["W1"], a["R"], a["gamma"], a["W2"], a["eps"], seq_len, n_rot, base,
                                   a["out_h"], a["out_y"], a["M"], a["K1"], a["D"], a["N2"], a["ws"], a["ws_bytes"],
                                   None)


@pytest.mark.parametrize("case,kw,want", [
    ("seq_len_zero", dict(seq_len=0), INVALID),
    ("n_rot_not_64", dict(n_rot=96), INVALID),
    ("n_rot_negative", dict(n_rot=-64), INVALID),
    ("n_rot_past_N2", dict(n_rot=576), INVALID),
    ("base_zero", dict(base=0.0), INVALID),
    ("base_negative", dict(base=-1.0), INVALID),
    ("base_nan", dict(base=float("nan")), INVALID),
    ("base_inf", dict(base=float("inf")), INVALID),
])
def test_rope_validation(lib, case, kw, want):
    assert _rcall(lib, _args(), **kw) == want, lib.coda_last_error()
    y = BASE + 6 * GB
    assert lib.coda_rope_rows(y, 100, 512, kw.get("seq_len", 2048), kw.get("n_rot", 256), kw.get("base", 1e4),
                              None) == want


def test_rope_block_rules(lib):
    # the block's own rules come first, and only the identity epilogue's workspace is needed
    assert _rcall(lib, _args(N2=384)) == UNSUPPORTED
    assert _rcall(lib, _args(out_y=BASE + 16)) == ALIAS
    a = _args()
    a["ws_bytes"] = lib.coda_workspace_bytes(a["M"], a["K1"], a["D"], a["N2"], 0, 0, 0) - 1
    assert _rcall(lib, a) == WORKSPACE
    assert lib.coda_rope_rows(0, 100, 512, 2048, 256, 1e4, None) == INVALID
    assert lib.coda_rope_rows(BASE, 0, 512, 2048, 256, 1e4, None) == INVALID


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_rope_no_gpu_reports_hip_error(lib):
    assert _rcall(lib, _args()) == HIP
    assert _rcall(lib, _args(), n_rot=0) == HIP
    assert lib.coda_rope_rows(BASE, 100, 512, 2048, 256, 1e4, None) == HIP


def _ccall(lib, fn="coda_ce_fwd", M=300, D=256, V=768, H=BASE, W=BASE + GB, labels=BASE + 2 * GB,
           loss=BASE + 3 * GB, lse=BASE + 4 * GB, ws=BASE + 5 * GB, ws_bytes=None, unfused=0):
    if ws_bytes is None:
        ws_bytes = lib.coda_ce_workspace_bytes(M, D, V, unfused) if M >= 1 and V >= 256 else 1 << 20
    return getattr(lib, fn)(H, W, labels, loss, lse, M, D, V, ws, ws_bytes, None)


@pytest.mark.parametrize("fn,unfused", [("coda_ce_fwd", 0), ("coda_ce_unfused", 1)])
@pytest.mark.parametrize("case,kw,want", [
    ("null_H", dict(H=0), INVALID),
    ("null_labels", dict(labels=0), INVALID),
    ("misaligned_loss", dict(loss=BASE + 3 * GB + 4), INVALID),
    ("M_zero", dict(M=0), INVALID),
    ("D_not_128", dict(D=192), UNSUPPORTED),
    ("V_not_256", dict(V=1000), UNSUPPORTED),
    ("loss_on_H", dict(loss=BASE + 64), ALIAS),
    ("lse_on_loss", dict(lse=BASE + 3 * GB + 256), ALIAS),
    ("ws_on_labels", dict(ws=BASE + 2 * GB), ALIAS),
    ("null_workspace", dict(ws=0), WORKSPACE),
    ("small_workspace", dict(ws_bytes=100), WORKSPACE),
])
def test_ce_validation(lib, fn, unfused, case, kw, want):
    assert _ccall(lib, fn, unfused=unfused, **kw) == want, lib.coda_last_error()


def test_ce_workspace_bytes(lib):
    al = lambda x: (x + 255) // 256 * 256
    M, D, V = 8192, 2048, 128256
    # the panel copy of H [M, D] bf16 first, then the per-tile pairs and label logits (or the bf16 logits)
    assert lib.coda_ce_workspace_bytes(M, D, V, 0) == al(M * D * 2) + 2 * al(V // 256 * M * 4) + al(M * 4)
    assert lib.coda_ce_workspace_bytes(M, D, V, 1) == al(M * D * 2) + al(M * V * 2)
    assert lib.coda_ce_workspace_bytes(0, D, V, 0) == 0
    assert lib.coda_ce_workspace_bytes(M, 0, V, 0) == 0


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_ce_no_gpu_reports_hip_error(lib):
    assert _ccall(lib) == HIP
    assert _ccall(lib, "coda_ce_unfused", unfused=1) == HIP


def _scall(lib, fn="coda_swiglu_bwd", M=300, D=256, F=512, dout=BASE, Wd=BASE + GB, z=BASE + 2 * GB,
           dz=BASE + 3 * GB, ws=BASE + 4 * GB, ws_bytes=1 << 30):
    return getattr(lib, fn)(dout, Wd, z, dz, M, D, F, ws, ws_bytes, None)


@pytest.mark.parametrize("fn", ["coda_swiglu_bwd", "coda_swiglu_bwd_unfused"])
@pytest.mark.parametrize("case,kw,want", [
    ("null_dout", dict(dout=0), INVALID),
    ("misaligned_z", dict(z=BASE + 2 * GB + 8), INVALID),
    ("M_zero", dict(M=0), INVALID),
    ("D_not_128", dict(D=192), UNSUPPORTED),
    ("F_not_256", dict(F=640), UNSUPPORTED),
    ("dz_on_z", dict(dz=BASE + 2 * GB + 256), ALIAS),
])
def test_swiglu_bwd_validation(lib, fn, case, kw, want):
    assert _scall(lib, fn, **kw) == want, lib.coda_last_error()


def test_swiglu_bwd_workspace(lib):
    assert lib.coda_swiglu_bwd_workspace_bytes(8192, 8192, 0) == 0
    assert lib.coda_swiglu_bwd_workspace_bytes(8192, 8192, 1) == 8192 * 8192 * 2
    assert _scall(lib, "coda_swiglu_bwd_unfused", ws=0) == WORKSPACE
    assert _scall(lib, "coda_swiglu_bwd_unfused", ws_bytes=100) == WORKSPACE
    assert _scall(lib, "coda_swiglu_bwd_unfused", ws=BASE + 2 * GB) == ALIAS  # workspace on z


@pytest.mark.skipif(torch.cuda.device_count() > 0, reason="would launch on fake pointers")
def test_swiglu_bwd_no_gpu_reports_hip_error(lib):
    assert _scall(lib, "coda_swiglu_bwd", ws=0, ws_bytes=0) == HIP  # the fused form needs no workspace
    assert _scall(lib, "coda_swiglu_bwd_unfused") == HIP


def test_save_z_validation(lib):
    a = _args(epi=1)
    z = BASE + 8 * GB
    call = lambda **o: lib.coda_block_fwd_save_z(a["X"], a["W1"], a["R"], a["gamma"], a["W2"], a["eps"], a["out_h"],
                                                 a["out_y"], o.get("z", z), a["M"], a["K1"], a["D"], o.get("N2", a["N2"]),
                                                 a["ws"], a["ws_bytes"], None)
    assert call(z=0) == INVALID
    assert call(z=BASE + 16) == ALIAS            # on X
    assert call(z=BASE + 6 * GB + 64) == ALIAS   # on out_y
    assert call(N2=384) == UNSUPPORTED


def test_noalloc_limits(lib):
    """coda_block_fwd_noalloc: a workspace beyond the library's fixed scratch is refused before anything touches the
    device; bad arguments within the limit are refused with the block's own codes."""
    f = lib.coda_block_fwd_noalloc
    args = lambda M, D, N2=512, epi=0, **o: [o.get("X", BASE), BASE + GB, BASE + 2 * GB, BASE + 3 * GB, BASE + 4 * GB,
                                             o.get("eps", 1e-5), epi, BASE + 5 * GB, BASE + 6 * GB, M, 256, D, N2, None]
    assert lib.coda_workspace_bytes(16384, 256, 4096, 512, 0, 0, 0) > cb.NOALLOC_SCRATCH_BYTES
    assert f(*args(16384, 4096)) == WORKSPACE
    assert b"scratch" in lib.coda_last_error()
    if torch.cuda.device_count() == 0:
        # within the limit the scratch's address is looked up first: with no device that is a HIP error
        assert f(*args(512, 256)) == HIP
