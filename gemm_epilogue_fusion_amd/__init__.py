"""MI355X (gfx950) fused GEMM -> residual -> RMSNorm -> GEMM block (CODA-style GEMM-epilogue programs).

The compute path is the HIP library libcoda.so (C ABI in include/coda.h); `binding` wraps it for torch
tensors and `inputs` draws the seeded synthetic workloads.  Importing this package loads nothing: the
library is opened on first use and a missing library raises instead of falling back to anything.
"""
from . import inputs  # noqa: F401
from .binding import (  # noqa: F401
    EPI_IDENTITY, EPI_SWIGLU, CodaError, alloc_workspace, coda_abi_version, coda_block_fwd, coda_block_unfused,
    coda_block_fwd_fp8, coda_block_unfused_fp8,
    coda_gemm1_residual_partial_rms, coda_gemm2_rowscale, coda_partial_rms_reduce, coda_workspace_bytes,
    coda_workspace_r_offset, load, workspace_r)
