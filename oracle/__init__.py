"""fp64 CPU oracle for the fused GEMM -> residual -> RMSNorm -> GEMM block.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library (``gemm_epilogue_fusion_amd``) never imports it and
shares no code with it; the two meet only in the tests, on the same seeded inputs.

The arithmetic lives in ``oracle.c`` (plain C, fp64, compiled with gcc).  This module builds it, loads it
with ctypes and wraps each entry point for numpy arrays.  Every function follows the CODA write-up
("CODA: new research optimizes Transformer training with GEMM-epilogue programming", section
"CODA: the treasure hidden in the epilogue"); the readings of what the pages leave open are listed in
``oracle.h``.

Parity pins: every function here is pinned by ``tests/test_oracle_pins.py`` against closed forms,
invariants, library routines (torch's rms_norm / silu / dtype casts) or exhaustive code tables.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

EPI_IDENTITY = 0
EPI_SWIGLU = 1

_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (-O3, no fast-math: IEEE semantics are part of the
    contract).  Returns the library path."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O3", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB)
    i64, dp, f = ctypes.c_int64, ctypes.POINTER(ctypes.c_double), ctypes.c_double
    block_sig = [i64, i64, i64, i64, dp, dp, dp, dp, dp, f, ctypes.c_int, dp, dp, dp, ctypes.c_int]
    for name in ("oracle_block_unfused_f64", "oracle_block_fused_f64", "oracle_block_roundpts_f64"):
        getattr(lib, name).argtypes = block_sig
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_gemm_residual_f64.argtypes = [i64, i64, i64, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_gemm_residual_f64.restype = ctypes.c_int
    lib.oracle_rms_scale_f64.argtypes = [i64, i64, dp, f, dp]
    lib.oracle_rms_scale_f64.restype = ctypes.c_int
    lib.oracle_rms_from_partials_f64.argtypes = [i64, i64, dp, i64, f, dp]
    lib.oracle_rms_from_partials_f64.restype = ctypes.c_int
    lib.oracle_silu.argtypes = [f]
    lib.oracle_silu.restype = f
    lib.oracle_bf16_round.argtypes = [f]
    lib.oracle_bf16_round.restype = f
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode.restype = f
    lib.oracle_e4m3_encode.argtypes = [f]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    u8p, fp = ctypes.POINTER(ctypes.c_uint8), ctypes.POINTER(ctypes.c_float)
    for name in ("oracle_dequant_rows_e4m3", "oracle_dequant_cols_e4m3"):
        getattr(lib, name).argtypes = [i64, i64, u8p, fp, dp]
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_block_bwd_f64.argtypes = [i64, i64, i64, i64, dp, dp, dp, dp, dp, f, dp, dp, dp, dp, dp, dp, dp,
                                         ctypes.c_int]
    lib.oracle_block_bwd_f64.restype = ctypes.c_int
    lib.oracle_rope_rows_f64.argtypes = [i64, i64, dp, i64, i64, i64, f]
    lib.oracle_rope_rows_f64.restype = ctypes.c_int
    lib.oracle_cross_entropy_f64.argtypes = [i64, i64, i64, dp, dp, ctypes.POINTER(ctypes.c_int64), dp, dp,
                                             ctypes.c_int]
    lib.oracle_cross_entropy_f64.restype = ctypes.c_int
    lib.oracle_mx_scale_exp.argtypes, lib.oracle_mx_scale_exp.restype = [f], ctypes.c_int
    lib.oracle_swiglu_bwd_f64.argtypes = [i64, i64, i64, dp, dp, dp, dp, ctypes.c_int]
    lib.oracle_swiglu_bwd_f64.restype = ctypes.c_int
    lib.oracle_mx_quant_rows_e4m3.argtypes = [i64, i64, i64, dp, ctypes.POINTER(ctypes.c_uint8),
                                              ctypes.POINTER(ctypes.c_int32)]
    lib.oracle_mx_quant_rows_e4m3.restype = ctypes.c_int
    for name, argt in (("oracle_bf16_round_array", [i64, dp, dp]),
                       ("oracle_e4m3_encode_array", [i64, dp, ctypes.POINTER(ctypes.c_uint8)]),
                       ("oracle_e4m3_decode_array", [i64, ctypes.POINTER(ctypes.c_uint8), dp])):
        getattr(lib, name).argtypes = argt
        getattr(lib, name).restype = ctypes.c_int
    lib.oracle_default_threads.argtypes = []
    lib.oracle_default_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray, ctype=ctypes.c_double):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def default_threads() -> int:
    return _load().oracle_default_threads()


def _block(name, X, W1, R, gamma, W2, eps, epi, nthreads):
    lib = _load()
    X, W1, R, gamma, W2 = (_f64(a) for a in (X, W1, R, gamma, W2))
    M, K1 = X.shape
    K1b, D = W1.shape
    Db, N2 = W2.shape
    if K1b != K1 or Db != D or R.shape != (M, D) or gamma.shape != (D,):
        raise ValueError("oracle: inconsistent shapes")
    ncols = N2 if epi == EPI_IDENTITY else N2 // 2
    h = np.empty((M, D), np.float64)
    r = np.empty((M,), np.float64)
    y = np.empty((M, ncols), np.float64)
    rc = getattr(lib, name)(M, K1, D, N2, _ptr(X), _ptr(W1), _ptr(R), _ptr(gamma), _ptr(W2), float(eps),
                            int(epi), _ptr(h), _ptr(r), _ptr(y), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"{name} failed with {rc}")
    return h, r, y


def block_unfused(X, W1, R, gamma, W2, eps, epi, nthreads=0):
    """h = X W1 + R; r = 1/sqrt(mean(h^2)+eps); y = epi((h * r * gamma) W2).  Returns (h, r, y) in fp64."""
    return _block("oracle_block_unfused_f64", X, W1, R, gamma, W2, eps, epi, nthreads)


def block_fused(X, W1, R, gamma, W2, eps, epi, nthreads=0):
    """Reparameterised order: y = epi(r * (h (diag(gamma) W2))).  Returns (h, r, y) in fp64."""
    return _block("oracle_block_fused_f64", X, W1, R, gamma, W2, eps, epi, nthreads)


def block_roundpts(X, W1, R, gamma, W2, eps, epi, nthreads=0):
    """Reparameterised order with bf16 storage roundings of h, diag(gamma) W2 and y (diagnostic)."""
    return _block("oracle_block_roundpts_f64", X, W1, R, gamma, W2, eps, epi, nthreads)


def block_bwd(X, W1, R, gamma, W2, eps, dz, dh_out=None, nthreads=0):
    """Backward of the block given dz [M,N2] (gradient of z = (h r gamma) W2, before the epilogue) and dh_out
    [M,D] (gradient arriving at h; None for none).  Returns (dX, dW1, dR, dgamma, dW2) in fp64."""
    lib = _load()
    X, W1, R, gamma, W2, dz = (_f64(a) for a in (X, W1, R, gamma, W2, dz))
    M, K1 = X.shape
    K1b, D = W1.shape
    Db, N2 = W2.shape
    if K1b != K1 or Db != D or R.shape != (M, D) or gamma.shape != (D,) or dz.shape != (M, N2):
        raise ValueError("oracle: inconsistent shapes")
    dhp = None
    if dh_out is not None:
        dh_out = _f64(dh_out)
        if dh_out.shape != (M, D):
            raise ValueError("oracle: inconsistent shapes")
        dhp = _ptr(dh_out)
    dX = np.empty((M, K1), np.float64)
    dW1 = np.empty((K1, D), np.float64)
    dR = np.empty((M, D), np.float64)
    dgamma = np.empty((D,), np.float64)
    dW2 = np.empty((D, N2), np.float64)
    rc = lib.oracle_block_bwd_f64(M, K1, D, N2, _ptr(X), _ptr(W1), _ptr(R), _ptr(gamma), _ptr(W2), float(eps),
                                  _ptr(dz), dhp, _ptr(dX), _ptr(dW1), _ptr(dR), _ptr(dgamma), _ptr(dW2),
                                  int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_block_bwd_f64 failed with {rc}")
    return dX, dW1, dR, dgamma, dW2


def rope_rows(y, head_dim, n_rot, seq_len, base):
    """Rotary position embedding of the rows of y [M,N] (a copy is returned): the first n_rot columns, heads of
    head_dim, pair (i, i + head_dim/2) rotated by (row mod seq_len) * base^(-2 i / head_dim)."""
    lib = _load()
    out = np.array(_f64(y), copy=True)
    M, N = out.shape
    rc = lib.oracle_rope_rows_f64(M, N, _ptr(out), int(head_dim), int(n_rot), int(seq_len), float(base))
    if rc != 0:
        raise RuntimeError(f"oracle_rope_rows_f64 failed with {rc}")
    return out


def cross_entropy(H, W, labels, nthreads=0):
    """Per-row cross-entropy of the logits H W (H [M,D], W [D,V]) against integer labels [M] (negative =
    ignored, loss 0).  Returns (loss [M], lse [M]) in fp64."""
    lib = _load()
    H, W = _f64(H), _f64(W)
    M, D = H.shape
    Db, V = W.shape
    lab = np.ascontiguousarray(np.asarray(labels, dtype=np.int64).reshape(-1))
    if Db != D or lab.shape != (M,):
        raise ValueError("oracle: inconsistent shapes")
    loss = np.empty(M, np.float64)
    lse = np.empty(M, np.float64)
    rc = lib.oracle_cross_entropy_f64(M, D, V, _ptr(H), _ptr(W), lab.ctypes.data_as(ctypes.POINTER(ctypes.c_int64)),
                                      _ptr(loss), _ptr(lse), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_cross_entropy_f64 failed with {rc}")
    return loss, lse


def gemm_residual(X, W1, R=None, nthreads=0):
    lib = _load()
    X, W1 = _f64(X), _f64(W1)
    M, K1 = X.shape
    D = W1.shape[1]
    h = np.empty((M, D), np.float64)
    Rp = None
    if R is not None:
        R = _f64(R)
        Rp = _ptr(R)
    rc = lib.oracle_gemm_residual_f64(M, K1, D, _ptr(X), _ptr(W1), Rp, _ptr(h), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_residual_f64 failed with {rc}")
    return h


def rms_scale(h, eps):
    lib = _load()
    h = _f64(h)
    M, D = h.shape
    r = np.empty((M,), np.float64)
    if lib.oracle_rms_scale_f64(M, D, _ptr(h), float(eps), _ptr(r)) != 0:
        raise RuntimeError("oracle_rms_scale_f64 failed")
    return r


def rms_from_partials(part, D, eps):
    """part [T, M] partial sums of squares -> r [M]."""
    lib = _load()
    part = _f64(part)
    T, M = part.shape
    r = np.empty((M,), np.float64)
    if lib.oracle_rms_from_partials_f64(T, M, _ptr(part), int(D), float(eps), _ptr(r)) != 0:
        raise RuntimeError("oracle_rms_from_partials_f64 failed")
    return r


def silu(x: float) -> float:
    return _load().oracle_silu(float(x))


def bf16_round(x) -> np.ndarray:
    lib = _load()
    a = _f64(x)
    out = np.empty(a.shape, np.float64)
    if lib.oracle_bf16_round_array(a.size, _ptr(a), _ptr(out)) != 0:
        raise RuntimeError("oracle_bf16_round_array failed")
    return out


def e4m3_decode(codes) -> np.ndarray:
    lib = _load()
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    out = np.empty(c.shape, np.float64)
    if lib.oracle_e4m3_decode_array(c.size, _ptr(c, ctypes.c_uint8), _ptr(out)) != 0:
        raise RuntimeError("oracle_e4m3_decode_array failed")
    return out


def e4m3_encode(x) -> np.ndarray:
    lib = _load()
    a = _f64(x)
    out = np.empty(a.shape, np.uint8)
    if lib.oracle_e4m3_encode_array(a.size, _ptr(a), _ptr(out, ctypes.c_uint8)) != 0:
        raise RuntimeError("oracle_e4m3_encode_array failed")
    return out


def dequant_rows_e4m3(q, s) -> np.ndarray:
    """Activations: out[i, k] = decode(q[i, k]) * s[i]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float64)
    if lib.oracle_dequant_rows_e4m3(rows, cols, _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float), _ptr(out)) != 0:
        raise RuntimeError("oracle_dequant_rows_e4m3 failed")
    return out


def dequant_cols_e4m3(q, s) -> np.ndarray:
    """Weights: out[k, n] = decode(q[k, n]) * s[n]."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.uint8)
    s = np.ascontiguousarray(s, dtype=np.float32)
    rows, cols = q.shape
    out = np.empty((rows, cols), np.float64)
    if lib.oracle_dequant_cols_e4m3(rows, cols, _ptr(q, ctypes.c_uint8), _ptr(s, ctypes.c_float), _ptr(out)) != 0:
        raise RuntimeError("oracle_dequant_cols_e4m3 failed")
    return out


def mx_scale_exp(amax: float) -> int:
    """Scale exponent of an MX-style e4m3 block whose largest magnitude is amax."""
    return int(_load().oracle_mx_scale_exp(float(amax)))


def mx_quant_rows_e4m3(x, block: int = 32):
    """Block-scaled e4m3 of the rows of x [rows, cols]: returns (codes uint8 [rows, cols], exps int32
    [rows, cols / block]); value = decode(code) * 2^exp of its block."""
    lib = _load()
    x = _f64(x)
    rows, cols = x.shape
    codes = np.empty((rows, cols), np.uint8)
    exps = np.empty((rows, cols // block), np.int32)
    rc = lib.oracle_mx_quant_rows_e4m3(rows, cols, int(block), _ptr(x), _ptr(codes, ctypes.c_uint8),
                                       _ptr(exps, ctypes.c_int32))
    if rc != 0:
        raise RuntimeError(f"oracle_mx_quant_rows_e4m3 failed with {rc}")
    return codes, exps


def swiglu_bwd(dout, Wd, z, nthreads=0):
    """dz [M, 2F] of y = silu(g) * u, z = [g | u], given the gradient dout [M,D] of the next product
    out = y Wd (Wd [F,D]): dy = dout Wd^T, dz = [dy u silu'(g) | dy silu(g)]."""
    lib = _load()
    dout, Wd, z = _f64(dout), _f64(Wd), _f64(z)
    M, D = dout.shape
    F, Db = Wd.shape
    if Db != D or z.shape != (M, 2 * F):
        raise ValueError("oracle: inconsistent shapes")
    dz = np.empty((M, 2 * F), np.float64)
    rc = lib.oracle_swiglu_bwd_f64(M, F, D, _ptr(dout), _ptr(Wd), _ptr(z), _ptr(dz), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_swiglu_bwd_f64 failed with {rc}")
    return dz
