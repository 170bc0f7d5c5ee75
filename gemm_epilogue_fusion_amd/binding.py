"""ctypes binding of libcoda.so (include/coda.h) for torch tensors.

Argument marshalling only: every step of the block runs in the library's HIP kernels.  Each function has the
name of the C entry point it calls, takes device tensors (torch is used for device memory and streams),
checks dtype / shape / device / contiguity on the host, passes raw pointers, sizes and the current HIP
stream, and raises CodaError with the library's own message on a non-zero status.  There is no fallback: if
the library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcoda.so")

EPI_IDENTITY = 0
EPI_SWIGLU = 1

STATUS = {0: "CODA_OK", 1: "CODA_ERR_INVALID_ARG", 2: "CODA_ERR_UNSUPPORTED", 3: "CODA_ERR_ALIAS",
          4: "CODA_ERR_WORKSPACE", 5: "CODA_ERR_HIP", 6: "CODA_ERR_INTERNAL"}

# every symbol include/coda.h declares
EXPORTS = ("coda_abi_version", "coda_status_string", "coda_last_error", "coda_workspace_bytes",
           "coda_workspace_split_bytes",
           "coda_workspace_r_offset", "coda_block_fwd", "coda_block_unfused", "coda_block_fwd_fp8",
           "coda_block_unfused_fp8", "coda_block_fwd_fp8_mx",
           "coda_gemm1_residual_partial_rms", "coda_partial_rms_reduce", "coda_gemm2_rowscale",
           "coda_gemm1_residual_partial_rms_panels", "coda_gemm2_rowscale_panels",
           "coda_bwd_workspace_bytes", "coda_block_bwd", "coda_block_bwd_unfused", "coda_block_bwd_w2t",
           "coda_block_fwd_rope",
           "coda_rope_rows", "coda_ce_workspace_bytes", "coda_ce_fwd", "coda_ce_unfused",
           "coda_block_fwd_save_z", "coda_swiglu_bwd_workspace_bytes", "coda_swiglu_bwd", "coda_swiglu_bwd_unfused",
           "coda_block_fwd_noalloc")


class CodaError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}: {detail}")


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libcoda.so (built by gemm_epilogue_fusion_amd.build); raises if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m gemm_epilogue_fusion_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i64, f32, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int, ctypes.c_size_t
    lib.coda_abi_version.argtypes, lib.coda_abi_version.restype = [], i32
    lib.coda_status_string.argtypes, lib.coda_status_string.restype = [i32], ctypes.c_char_p
    lib.coda_last_error.argtypes, lib.coda_last_error.restype = [], ctypes.c_char_p
    lib.coda_workspace_bytes.argtypes = [i64, i64, i64, i64, i32, i32, i32]
    lib.coda_workspace_bytes.restype = sz
    lib.coda_workspace_split_bytes.argtypes = [i64, i64, i64, i64, i32, i32, i32]
    lib.coda_workspace_split_bytes.restype = sz
    lib.coda_workspace_r_offset.argtypes, lib.coda_workspace_r_offset.restype = [i64, i64], sz
    block = [vp, vp, vp, vp, vp, f32, i32, vp, vp, i64, i64, i64, i64, vp, sz, vp]
    for name in ("coda_block_fwd", "coda_block_unfused"):
        getattr(lib, name).argtypes = block
        getattr(lib, name).restype = i32
    lib.coda_block_fwd_noalloc.argtypes = [vp, vp, vp, vp, vp, f32, i32, vp, vp, i64, i64, i64, i64, vp]
    lib.coda_block_fwd_noalloc.restype = i32
    block8 = [vp, vp, vp, vp, vp, vp, vp, vp, f32, i32, vp, vp, i64, i64, i64, i64, vp, sz, vp]
    for name in ("coda_block_fwd_fp8", "coda_block_unfused_fp8", "coda_block_fwd_fp8_mx"):
        getattr(lib, name).argtypes = block8
        getattr(lib, name).restype = i32
    lib.coda_gemm1_residual_partial_rms.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.coda_gemm1_residual_partial_rms.restype = i32
    lib.coda_partial_rms_reduce.argtypes = [vp, i64, i64, i64, f32, vp, vp]
    lib.coda_partial_rms_reduce.restype = i32
    lib.coda_gemm2_rowscale.argtypes = [vp, vp, vp, i32, vp, i64, i64, i64, vp]
    lib.coda_gemm2_rowscale.restype = i32
    lib.coda_gemm1_residual_partial_rms_panels.argtypes = [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
    lib.coda_gemm1_residual_partial_rms_panels.restype = i32
    lib.coda_gemm2_rowscale_panels.argtypes = [vp, vp, vp, f32, vp, i32, vp, i64, i64, i64, vp]
    lib.coda_gemm2_rowscale_panels.restype = i32
    lib.coda_block_fwd_rope.argtypes = [vp, vp, vp, vp, vp, f32, i64, i64, f32, vp, vp, i64, i64, i64, i64, vp, sz, vp]
    lib.coda_block_fwd_rope.restype = i32
    lib.coda_rope_rows.argtypes, lib.coda_rope_rows.restype = [vp, i64, i64, i64, i64, f32, vp], i32
    lib.coda_bwd_workspace_bytes.argtypes, lib.coda_bwd_workspace_bytes.restype = [i64, i64, i64, i64, i32], sz
    bwd = [vp] * 13 + [i64, i64, i64, i64, vp, sz, vp]
    for name in ("coda_block_bwd", "coda_block_bwd_unfused", "coda_block_bwd_w2t"):
        getattr(lib, name).argtypes = bwd
        getattr(lib, name).restype = i32
    lib.coda_ce_workspace_bytes.argtypes, lib.coda_ce_workspace_bytes.restype = [i64, i64, i64, i32], sz
    for name in ("coda_ce_fwd", "coda_ce_unfused"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
        getattr(lib, name).restype = i32
    lib.coda_block_fwd_save_z.argtypes = [vp, vp, vp, vp, vp, f32, vp, vp, vp, i64, i64, i64, i64, vp, sz, vp]
    lib.coda_block_fwd_save_z.restype = i32
    lib.coda_swiglu_bwd_workspace_bytes.argtypes, lib.coda_swiglu_bwd_workspace_bytes.restype = [i64, i64, i32], sz
    for name in ("coda_swiglu_bwd", "coda_swiglu_bwd_unfused"):
        getattr(lib, name).argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, sz, vp]
        getattr(lib, name).restype = i32
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        detail = load().coda_last_error().decode(errors="replace")
        raise CodaError(status, where, detail)


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def coda_abi_version() -> int:
    return load().coda_abi_version()


def coda_workspace_bytes(M: int, K1: int, D: int, N2: int, epi_kind: int, fp8: int = 0, unfused: int = 0) -> int:
    return load().coda_workspace_bytes(M, K1, D, N2, epi_kind, fp8, unfused)


def coda_workspace_r_offset(M: int, D: int) -> int:
    return load().coda_workspace_r_offset(M, D)


def coda_workspace_split_bytes(M: int, K1: int, D: int, N2: int, epi_kind: int, fp8: int = 0,
                               unfused: int = 0) -> int:
    return load().coda_workspace_split_bytes(M, K1, D, N2, epi_kind, fp8, unfused)


def alloc_workspace(M: int, K1: int, D: int, N2: int, epi_kind: int, unfused: int = 0, device="cuda", fp8: int = 0,
                    split: bool = True):
    """The workspace of a block entry point; split=False leaves out the room for splitting the products' last
    waves (the block then runs them as whole tiles)."""
    n = coda_workspace_bytes(M, K1, D, N2, epi_kind, fp8, unfused)
    if n == 0:
        raise ValueError("no workspace size for these dimensions")
    if not split:
        n -= coda_workspace_split_bytes(M, K1, D, N2, epi_kind, fp8, unfused)
    return torch.empty(n, dtype=torch.uint8, device=device)


def _block(name: str, X, W1, R, gamma, W2, eps, epi_kind, out_h, out_y, workspace, stream):
    M, K1 = X.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    ny = N2 if epi_kind == EPI_IDENTITY else N2 // 2
    args = (_dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
            _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
            _dev(W2, "W2", torch.bfloat16, (D, N2)))
    h = _dev(out_h, "out_h", torch.bfloat16, (M, D))
    y = _dev(out_y, "out_y", torch.bfloat16, (M, ny))
    ws = _dev(workspace, "workspace", torch.uint8)
    st = getattr(load(), name)(*args, float(eps), int(epi_kind), h, y, M, K1, D, N2, ws, workspace.numel(),
                               _stream(stream))
    _check(st, name)


def coda_block_fwd(X, W1, R, gamma, W2, eps: float, epi_kind: int, out_h, out_y, workspace, stream=None):
    """Fused block: out_h = bf16(X W1 + R); out_y = bf16(epi(r * (h diag(gamma) W2)))."""
    _block("coda_block_fwd", X, W1, R, gamma, W2, eps, epi_kind, out_h, out_y, workspace, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # CODA_NOALLOC_SCRATCH_BYTES of include/coda.h


def coda_block_fwd_noalloc(X, W1, R, gamma, W2, eps: float, epi_kind: int, out_h, out_y, stream=None):
    """coda_block_fwd on the library's fixed per-device scratch (no workspace; nothing allocated); calls on one
    device must not overlap."""
    M, K1 = X.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    ny = N2 if epi_kind == EPI_IDENTITY else N2 // 2
    args = (_dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
            _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
            _dev(W2, "W2", torch.bfloat16, (D, N2)))
    h = _dev(out_h, "out_h", torch.bfloat16, (M, D))
    y = _dev(out_y, "out_y", torch.bfloat16, (M, ny))
    st = load().coda_block_fwd_noalloc(*args, float(eps), int(epi_kind), h, y, M, K1, D, N2, _stream(stream))
    _check(st, "coda_block_fwd_noalloc")


def coda_block_unfused(X, W1, R, gamma, W2, eps: float, epi_kind: int, out_h, out_y, workspace, stream=None):
    """Unfused three-kernel baseline with the same outputs."""
    _block("coda_block_unfused", X, W1, R, gamma, W2, eps, epi_kind, out_h, out_y, workspace, stream)


def coda_block_fwd_rope(X, W1, R, gamma, W2, eps: float, seq_len: int, n_rope_cols: int, rope_base: float, out_h,
                        out_y, workspace, stream=None):
    """Fused block (identity epilogue) with a rotary embedding of the first n_rope_cols output columns."""
    M, K1 = X.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    args = (_dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
            _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
            _dev(W2, "W2", torch.bfloat16, (D, N2)))
    st = load().coda_block_fwd_rope(*args, float(eps), int(seq_len), int(n_rope_cols), float(rope_base),
                                    _dev(out_h, "out_h", torch.bfloat16, (M, D)),
                                    _dev(out_y, "out_y", torch.bfloat16, (M, N2)), M, K1, D, N2,
                                    _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(st, "coda_block_fwd_rope")


def coda_rope_rows(y, seq_len: int, n_rope_cols: int, rope_base: float, stream=None):
    """In-place rotary embedding of bf16 y [M,N] (the separate-pass counterpart)."""
    M, N = y.shape
    st = load().coda_rope_rows(_dev(y, "y", torch.bfloat16), M, N, int(seq_len), int(n_rope_cols), float(rope_base),
                               _stream(stream))
    _check(st, "coda_rope_rows")


def _block_fp8(name: str, Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, workspace, stream):
    M, K1 = Xq.shape
    D = W1q.shape[1]
    N2 = W2q.shape[1]
    ny = N2 if epi_kind == EPI_IDENTITY else N2 // 2
    e4 = torch.float8_e4m3fn
    args = (_dev(Xq, "Xq", e4, (M, K1)), _dev(sx, "sx", torch.float32, (M,)),
            _dev(W1q, "W1q", e4, (K1, D)), _dev(sw1, "sw1", torch.float32, (D,)),
            _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
            _dev(W2q, "W2q", e4, (D, N2)), _dev(sw2, "sw2", torch.float32, (N2,)))
    h = _dev(out_h, "out_h", torch.bfloat16, (M, D))
    y = _dev(out_y, "out_y", torch.bfloat16, (M, ny))
    ws = _dev(workspace, "workspace", torch.uint8)
    st = getattr(load(), name)(*args, float(eps), int(epi_kind), h, y, M, K1, D, N2, ws, workspace.numel(),
                               _stream(stream))
    _check(st, name)


def coda_block_fwd_fp8(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps: float, epi_kind: int, out_h, out_y, workspace,
                       stream=None):
    """Fused block with e4m3 operands (dequantised value = code * scale; sx per row, sw1 / sw2 per column)."""
    _block_fp8("coda_block_fwd_fp8", Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, workspace,
               stream)


def coda_block_fwd_fp8_mx(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps: float, epi_kind: int, out_h, out_y, workspace,
                          stream=None):
    """Fused e4m3 block whose second GEMM takes a block-scaled (32 values per power-of-two scale) A operand
    quantised in the first GEMM's epilogue; workspace from alloc_workspace(..., fp8=2)."""
    _block_fp8("coda_block_fwd_fp8_mx", Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, workspace,
               stream)


def coda_block_unfused_fp8(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps: float, epi_kind: int, out_h, out_y, workspace,
                           stream=None):
    """Unfused three-kernel baseline with e4m3 operands."""
    _block_fp8("coda_block_unfused_fp8", Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y,
               workspace, stream)


def coda_gemm1_residual_partial_rms(X, W1, R, gamma, out_h, out_hg, part, stream=None):
    """Step 1: out_h = bf16(X W1 + R), out_hg = bf16((X W1 + R) * gamma), part [D/256, M] partial sums of squares."""
    M, K1 = X.shape
    D = W1.shape[1]
    st = load().coda_gemm1_residual_partial_rms(
        _dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
        _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
        _dev(out_h, "out_h", torch.bfloat16, (M, D)), _dev(out_hg, "out_hg", torch.bfloat16, (M, D)),
        _dev(part, "part", torch.float32, (D // 256, M)), M, K1, D, _stream(stream))
    _check(st, "coda_gemm1_residual_partial_rms")


def coda_partial_rms_reduce(part, D: int, eps: float, r, stream=None):
    T, M = part.shape
    st = load().coda_partial_rms_reduce(_dev(part, "part", torch.float32, (T, M)), T, M, D, float(eps),
                                        _dev(r, "r", torch.float32, (M,)), _stream(stream))
    _check(st, "coda_partial_rms_reduce")


def coda_gemm2_rowscale(hg, W2, r, epi_kind: int, out_y, stream=None):
    """Step 3: out_y = bf16(epi(r * (hg W2)))."""
    M, D = hg.shape
    N2 = W2.shape[1]
    ny = N2 if epi_kind == EPI_IDENTITY else N2 // 2
    st = load().coda_gemm2_rowscale(
        _dev(hg, "hg", torch.bfloat16, (M, D)), _dev(W2, "W2", torch.bfloat16, (D, N2)),
        _dev(r, "r", torch.float32, (M,)), int(epi_kind), _dev(out_y, "out_y", torch.bfloat16, (M, ny)),
        M, D, N2, _stream(stream))
    _check(st, "coda_gemm2_rowscale")


def coda_gemm1_residual_partial_rms_panels(X, W1, R, gamma, out_h, out_hg_panels, part, stream=None):
    """Step 1 with hg written in K panels: out_hg_panels [D/32, M, 32] holds hg[m, 32 p + j] at [p, m, j]."""
    M, K1 = X.shape
    D = W1.shape[1]
    st = load().coda_gemm1_residual_partial_rms_panels(
        _dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
        _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
        _dev(out_h, "out_h", torch.bfloat16, (M, D)),
        _dev(out_hg_panels, "out_hg_panels", torch.bfloat16, (D // 32, M, 32)),
        _dev(part, "part", torch.float32, (D // 256, M)), M, K1, D, _stream(stream))
    _check(st, "coda_gemm1_residual_partial_rms_panels")


def coda_gemm2_rowscale_panels(hg_panels, W2, part, eps: float, r, epi_kind: int, out_y, stream=None):
    """Step 3 on hg in K panels [D/32, M, 32].  With part [D/256, M] the reduce is folded in and r [M] is
    written; with part None r is read (eps unused)."""
    P, M, _ = hg_panels.shape
    D = 32 * P
    N2 = W2.shape[1]
    ny = N2 if epi_kind == EPI_IDENTITY else N2 // 2
    st = load().coda_gemm2_rowscale_panels(
        _dev(hg_panels, "hg_panels", torch.bfloat16, (P, M, 32)), _dev(W2, "W2", torch.bfloat16, (D, N2)),
        None if part is None else _dev(part, "part", torch.float32, (D // 256, M)), float(eps),
        _dev(r, "r", torch.float32, (M,)), int(epi_kind), _dev(out_y, "out_y", torch.bfloat16, (M, ny)),
        M, D, N2, _stream(stream))
    _check(st, "coda_gemm2_rowscale_panels")


def workspace_r(workspace: torch.Tensor, M: int, D: int) -> torch.Tensor:
    """View of r [M] fp32 inside a workspace after coda_block_fwd / coda_block_unfused."""
    off = coda_workspace_r_offset(M, D)
    return workspace[off: off + 4 * M].view(torch.float32)


def coda_bwd_workspace_bytes(M: int, K1: int, D: int, N2: int, unfused: int = 0) -> int:
    return load().coda_bwd_workspace_bytes(M, K1, D, N2, unfused)


def alloc_bwd_workspace(M: int, K1: int, D: int, N2: int, unfused: int = 0, device="cuda"):
    n = coda_bwd_workspace_bytes(M, K1, D, N2, unfused)
    if n == 0:
        raise ValueError("no workspace size for these dimensions")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _block_bwd(name, X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, workspace,
               stream, w2_transposed=False):
    M, K1 = X.shape
    D = W1.shape[1]
    N2 = W2.shape[0] if w2_transposed else W2.shape[1]
    bf = torch.bfloat16
    args = (_dev(X, "X", bf, (M, K1)), _dev(W1, "W1", bf, (K1, D)), _dev(h, "h", bf, (M, D)),
            _dev(r, "r", torch.float32, (M,)), _dev(gamma, "gamma", torch.float32, (D,)),
            _dev(W2, "W2t", bf, (N2, D)) if w2_transposed else _dev(W2, "W2", bf, (D, N2)), _dev(dz, "dz", bf, (M, N2)),
            None if dh_out is None else _dev(dh_out, "dh_out", bf, (M, D)),
            _dev(out_dX, "out_dX", bf, (M, K1)), _dev(out_dW1, "out_dW1", torch.float32, (K1, D)),
            _dev(out_dR, "out_dR", bf, (M, D)), _dev(out_dgamma, "out_dgamma", torch.float32, (D,)),
            _dev(out_dW2, "out_dW2", torch.float32, (D, N2)))
    ws = _dev(workspace, "workspace", torch.uint8)
    st = getattr(load(), name)(*args, M, K1, D, N2, ws, workspace.numel(), _stream(stream))
    _check(st, name)


def coda_block_bwd(X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, workspace,
                   stream=None):
    """Backward of the block (fused path): dX, dW1, dR (= dh), dgamma, dW2 from dz (gradient of the second
    product's output) and dh_out (gradient arriving at h; None for none), with h and r from the forward."""
    _block_bwd("coda_block_bwd", X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2,
               workspace, stream)


def coda_block_bwd_w2t(X, W1, h, r, gamma, W2t, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, workspace,
                       stream=None):
    """coda_block_bwd with W2 given transposed (W2t [N2, D], the [out, in] layout): the same results, without
    the transpose pass over W2."""
    _block_bwd("coda_block_bwd_w2t", X, W1, h, r, gamma, W2t, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma,
               out_dW2, workspace, stream, w2_transposed=True)


def coda_block_bwd_unfused(X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2,
                           workspace, stream=None):
    """Unfused backward baseline with the same outputs."""
    _block_bwd("coda_block_bwd_unfused", X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma,
               out_dW2, workspace, stream)


def coda_ce_workspace_bytes(M: int, D: int, V: int, unfused: int = 0) -> int:
    return int(load().coda_ce_workspace_bytes(M, D, V, unfused))


def alloc_ce_workspace(M: int, D: int, V: int, unfused: int = 0, device="cuda"):
    n = coda_ce_workspace_bytes(M, D, V, unfused)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def _ce(name, H, W, labels, out_loss, out_lse, workspace, stream):
    M, D = H.shape
    V = W.shape[1]
    st = getattr(load(), name)(_dev(H, "H", torch.bfloat16, (M, D)), _dev(W, "W", torch.bfloat16, (D, V)),
                               _dev(labels, "labels", torch.int32, (M,)), _dev(out_loss, "out_loss", torch.float32, (M,)),
                               _dev(out_lse, "out_lse", torch.float32, (M,)), M, D, V,
                               _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(st, name)


def coda_ce_fwd(H, W, labels, out_loss, out_lse, workspace, stream=None):
    """Per-row cross-entropy of H W against labels (int32; negative = ignored) with the logits never stored."""
    _ce("coda_ce_fwd", H, W, labels, out_loss, out_lse, workspace, stream)


def coda_ce_unfused(H, W, labels, out_loss, out_lse, workspace, stream=None):
    """The same through stored bf16 logits (the baseline)."""
    _ce("coda_ce_unfused", H, W, labels, out_loss, out_lse, workspace, stream)


def coda_block_fwd_save_z(X, W1, R, gamma, W2, eps: float, out_h, out_y, out_z, workspace, stream=None):
    """Fused block with the SwiGLU epilogue that also stores the pre-activation z [M, N2] (gate | up)."""
    M, K1 = X.shape
    D = W1.shape[1]
    N2 = W2.shape[1]
    st = load().coda_block_fwd_save_z(
        _dev(X, "X", torch.bfloat16, (M, K1)), _dev(W1, "W1", torch.bfloat16, (K1, D)),
        _dev(R, "R", torch.bfloat16, (M, D)), _dev(gamma, "gamma", torch.float32, (D,)),
        _dev(W2, "W2", torch.bfloat16, (D, N2)), float(eps), _dev(out_h, "out_h", torch.bfloat16, (M, D)),
        _dev(out_y, "out_y", torch.bfloat16, (M, N2 // 2)), _dev(out_z, "out_z", torch.bfloat16, (M, N2)), M, K1, D, N2,
        _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))
    _check(st, "coda_block_fwd_save_z")


def coda_swiglu_bwd_workspace_bytes(M: int, F: int, unfused: int = 0) -> int:
    return int(load().coda_swiglu_bwd_workspace_bytes(M, F, unfused))


def _swiglu_bwd(name, dout, Wd, z, out_dz, workspace, stream):
    M, D = dout.shape
    F = Wd.shape[0]
    ws = _dev(workspace, "workspace", torch.uint8) if workspace is not None else None
    st = getattr(load(), name)(_dev(dout, "dout", torch.bfloat16, (M, D)), _dev(Wd, "Wd", torch.bfloat16, (F, D)),
                               _dev(z, "z", torch.bfloat16, (M, 2 * F)), _dev(out_dz, "out_dz", torch.bfloat16, (M, 2 * F)),
                               M, D, F, ws, workspace.numel() if workspace is not None else 0, _stream(stream))
    _check(st, name)


def coda_swiglu_bwd(dout, Wd, z, out_dz, workspace=None, stream=None):
    """dz of the SwiGLU epilogue from the gradient of the next product (dy never stored)."""
    _swiglu_bwd("coda_swiglu_bwd", dout, Wd, z, out_dz, workspace, stream)


def coda_swiglu_bwd_unfused(dout, Wd, z, out_dz, workspace, stream=None):
    """The same through a stored dy (workspace of coda_swiglu_bwd_workspace_bytes(M, F, 1) bytes)."""
    _swiglu_bwd("coda_swiglu_bwd_unfused", dout, Wd, z, out_dz, workspace, stream)
