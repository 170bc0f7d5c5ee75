"""Seeded synthetic inputs for the fused GEMM -> residual -> RMSNorm -> GEMM block.

This module only draws random tensors.  It holds none of the block's arithmetic, and both the GPU path and
the CPU oracle take their inputs from it (nothing else is shared between them).

Workloads (shapes of a LLaMA-3-style decoder, the model family the CODA write-up profiles in its section
on where training time goes: a 1B model trained with TorchTitan on one GPU).  Real activations are replaced
by seeded Gaussians of the stated spread; real activations may carry outlier channels that these lack.

Generation recipe: one CPU ``torch.Generator`` per tensor, seeded ``16 * seed + idx`` with idx X=0, W1=1,
R=2, gamma=3, W2=4; values are drawn in fp32 and rounded to nearest-even bf16 (gamma stays fp32).  The
fp8 workload draws the same fp32 values and quantises X per row and the weights per output column to OCP
e4m3fn with scale amax/448 (an all-zero row or column gets scale 1).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import torch

EPI_IDENTITY = 0
EPI_SWIGLU = 1
E4M3_MAX = 448.0


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    K1: int
    D: int
    N2: int
    epi: int
    eps: float
    x_std: float = 1.0
    w1_std: float = 0.02
    r_std: float = 1.0
    w2_std: float = 0.02
    gamma_lo: float = 0.5
    gamma_hi: float = 1.5
    fp8: bool = False
    seed: int = 0

    @property
    def n_out(self) -> int:
        return self.N2 if self.epi == EPI_IDENTITY else self.N2 // 2

    @property
    def flops(self) -> int:
        """Multiply-adds of the two products, counted as 2 flops each (epilogue work excluded)."""
        return 2 * self.M * self.K1 * self.D + 2 * self.M * self.D * self.N2

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The workloads.  "tiny" is the case the oracle finishes in well under a second; the others are the full-size
# shapes.
WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", M=64, K1=256, D=256, N2=512, epi=EPI_IDENTITY, eps=1e-6,
                     w1_std=(1 / 256) ** 0.5, w2_std=(1 / 256) ** 0.5),
    # attention output projection -> RMSNorm -> gate|up projection with SwiGLU, 1B-style (hidden 2048,
    # intermediate 8192), 4 sequences of 2048 tokens
    "1b_attn_out_mlp_in": Workload("1b_attn_out_mlp_in", M=8192, K1=2048, D=2048, N2=16384,
                                   epi=EPI_SWIGLU, eps=1e-5),
    # MLP down projection -> RMSNorm -> QKV projection (32 q heads + 8 k + 8 v heads of 64), 1B-style
    "1b_mlp_out_qkv": Workload("1b_mlp_out_qkv", M=8192, K1=8192, D=2048, N2=3072, epi=EPI_IDENTITY,
                               eps=1e-5, x_std=0.5),
    # attention output projection -> RMSNorm -> gate|up with SwiGLU, 8B-style (hidden 4096, inter 14336)
    "8b_attn_out_mlp_in": Workload("8b_attn_out_mlp_in", M=16384, K1=4096, D=4096, N2=28672,
                                   epi=EPI_SWIGLU, eps=1e-5),
    # attention output projection -> RMSNorm -> gate|up with SwiGLU, 70B-style (hidden 8192, inter 28672): the
    # largest hidden size the write-up's results name; D > 4096, so the partial-RMS reduce runs as its own kernel
    "70b_attn_out_mlp_in": Workload("70b_attn_out_mlp_in", M=8192, K1=8192, D=8192, N2=57344,
                                    epi=EPI_SWIGLU, eps=1e-5),
    # the 1B attention-out -> MLP-in block with e4m3 X / weights and per-row / per-column fp32 scales
    "1b_attn_out_mlp_in_fp8": Workload("1b_attn_out_mlp_in_fp8", M=8192, K1=2048, D=2048, N2=16384,
                                       epi=EPI_SWIGLU, eps=1e-5, fp8=True),
}


def _gen(seed: int, idx: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(16 * seed + idx)
    return g


def _normal(shape, std, seed, idx) -> torch.Tensor:
    return torch.randn(*shape, generator=_gen(seed, idx), dtype=torch.float32) * std


def _quantize_e4m3(t: torch.Tensor, dim: int):
    """Per-row (dim=1 reduces along columns) or per-column (dim=0) e4m3fn quantisation, scale amax/448."""
    amax = t.abs().amax(dim=dim)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    s = scale.unsqueeze(dim)
    q = (t / s).clamp(-E4M3_MAX, E4M3_MAX).to(torch.float8_e4m3fn)
    return q, scale


@dataclass
class BlockInputs:
    wl: Workload
    X: torch.Tensor        # [M, K1] bf16 (fp8 workloads: the unquantised draw, for reference only)
    W1: torch.Tensor       # [K1, D] bf16
    R: torch.Tensor        # [M, D] bf16
    gamma: torch.Tensor    # [D] fp32
    W2: torch.Tensor       # [D, N2] bf16
    Xq: Optional[torch.Tensor] = None    # [M, K1] float8_e4m3fn
    sx: Optional[torch.Tensor] = None    # [M] fp32
    W1q: Optional[torch.Tensor] = None   # [K1, D] float8_e4m3fn
    sw1: Optional[torch.Tensor] = None   # [D] fp32
    W2q: Optional[torch.Tensor] = None   # [D, N2] float8_e4m3fn
    sw2: Optional[torch.Tensor] = None   # [N2] fp32
    extras: dict = field(default_factory=dict)


def make_inputs(wl: Workload) -> BlockInputs:
    """Draw the inputs of workload ``wl`` on the CPU.  Deterministic in (wl, seed)."""
    s = wl.seed
    Xf = _normal((wl.M, wl.K1), wl.x_std, s, 0)
    W1f = _normal((wl.K1, wl.D), wl.w1_std, s, 1)
    Rf = _normal((wl.M, wl.D), wl.r_std, s, 2)
    gamma = torch.rand(wl.D, generator=_gen(s, 3), dtype=torch.float32) * (wl.gamma_hi - wl.gamma_lo) + wl.gamma_lo
    W2f = _normal((wl.D, wl.N2), wl.w2_std, s, 4)
    out = BlockInputs(wl, Xf.to(torch.bfloat16), W1f.to(torch.bfloat16), Rf.to(torch.bfloat16), gamma,
                      W2f.to(torch.bfloat16))
    if wl.fp8:
        out.Xq, out.sx = _quantize_e4m3(Xf, dim=1)
        out.W1q, out.sw1 = _quantize_e4m3(W1f, dim=0)
        out.W2q, out.sw2 = _quantize_e4m3(W2f, dim=0)
    return out


def make_grads(wl: Workload, dz_std: float = 1.0, dh_std: float = 1.0):
    """Incoming gradients for the backward of workload ``wl``: dz [M, N2] (gradient of the second product's
    output) and dh_out [M, D] (gradient arriving at the residual stream), seeded Gaussians rounded to bf16
    (idx 5 and 6 of the same seeding scheme).  The real ones come from the layers above; their scale only
    sets the scale of every output gradient."""
    s = wl.seed
    dz = _normal((wl.M, wl.N2), dz_std, s, 5).to(torch.bfloat16)
    dh = _normal((wl.M, wl.D), dh_std, s, 6).to(torch.bfloat16)
    return dz, dh


# ---- cross-entropy of a vocabulary projection ----
@dataclass(frozen=True)
class CeWorkload:
    """Per-row cross-entropy of H W against labels: H [M,D] (the final normalised hidden states), W [D,V] (the
    vocabulary projection, [in,out]), labels [M] int32."""
    name: str
    M: int
    D: int
    V: int
    h_std: float = 1.0
    w_std: float = 0.02
    ignore_every: int = 0   # every n-th row (from row 0) gets the ignored label -100 (0: none)
    seed: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.D * self.V


# LLaMA-3-style LM head at the 1B size: hidden 2048, vocabulary 128256 (= 501 x 256), 4 sequences of 2048 tokens.
# The write-up fixes no vocabulary; labels are uniform over it (a real corpus is Zipf-like, which changes
# nothing in the arithmetic).
CE_WORKLOADS: Dict[str, CeWorkload] = {
    "1b_lm_head": CeWorkload("1b_lm_head", M=8192, D=2048, V=128256, ignore_every=64),
}


def make_ce_inputs(wl: CeWorkload):
    """Draw (H bf16, W bf16, labels int32) on the CPU with idx H=8, W=9, labels=10 of the seeding scheme."""
    s = wl.seed
    H = _normal((wl.M, wl.D), wl.h_std, s, 8).to(torch.bfloat16)
    W = _normal((wl.D, wl.V), wl.w_std, s, 9).to(torch.bfloat16)
    labels = torch.randint(0, wl.V, (wl.M,), generator=_gen(s, 10), dtype=torch.int64).to(torch.int32)
    if wl.ignore_every:
        labels[::wl.ignore_every] = -100
    return H, W, labels


# ---- backward of the SwiGLU epilogue ----
@dataclass(frozen=True)
class SwigluBwdWorkload:
    """dz [M, 2F] of y = silu(g) * u from z = [g | u] [M, 2F] and the gradient dout [M, D] of the next product
    out = y Wd, Wd [F, D] (stored [in = F, out = D])."""
    name: str
    M: int
    D: int
    F: int
    z_std: float = 1.0
    dout_std: float = 1.0
    w_std: float = 0.02
    seed: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.D * self.F


# The 1B MLP (hidden 2048, intermediate 8192): the gradient comes back through the down projection.
SWIGLU_BWD_WORKLOADS: Dict[str, SwigluBwdWorkload] = {
    "1b_mlp_down_dgrad": SwigluBwdWorkload("1b_mlp_down_dgrad", M=8192, D=2048, F=8192),
}


def make_swiglu_bwd_inputs(wl: SwigluBwdWorkload):
    """Draw (dout bf16 [M,D], Wd bf16 [F,D], z bf16 [M,2F]) with idx dout=11, Wd=12, z=13 of the seeding scheme."""
    s = wl.seed
    dout = _normal((wl.M, wl.D), wl.dout_std, s, 11).to(torch.bfloat16)
    Wd = _normal((wl.F, wl.D), wl.w_std, s, 12).to(torch.bfloat16)
    z = _normal((wl.M, 2 * wl.F), wl.z_std, s, 13).to(torch.bfloat16)
    return dout, Wd, z
