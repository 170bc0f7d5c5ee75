"""Builds libcoda.so (the HIP kernels and the C ABI of include/coda.h) in-tree for gfx950.

    python -m gemm_epilogue_fusion_amd.build
"""
from __future__ import annotations

import os
import re
import subprocess
import sys
from typing import Dict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libcoda.so")
SOURCES = ["kernels.hip", "bwd_kernels.hip", "ce_kernels.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: keep the compiler from forming packed fp32 (v_pk_*_f32) instructions.
# kernel-resource-usage remarks: the per-kernel register, scratch and LDS figures, checked below.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Rpass-analysis=kernel-resource-usage",
         "-I", INCLUDE, "-I", CSRC]

# The GEMM kernels keep 128 accumulator registers per lane and run two waves per SIMD (8 waves, one
# workgroup per CU); spilling to scratch would cost several times the kernel's time, so the build fails on it.
MAX_VGPRS = 256
MAX_LDS_BYTES = 160 * 1024

_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|ScratchSize \[bytes/lane\]|LDS Size \[bytes/block\]|"
                     r"Occupancy \[waves/SIMD\]):\s+(\S+)")


def resource_usage(text: str) -> Dict[str, Dict[str, str]]:
    """Per-kernel figures from the compiler's kernel-resource-usage remarks."""
    usage: Dict[str, Dict[str, str]] = {}
    cur = None
    for line in text.splitlines():
        m = _REMARK.search(line)
        if not m:
            continue
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = usage.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" ")[0]] = val
    return usage


def check_usage(usage: Dict[str, Dict[str, str]]) -> None:
    bad = []
    for name, u in usage.items():
        if int(u.get("ScratchSize", "0")) != 0:
            bad.append(f"{name}: {u['ScratchSize']} bytes of scratch per lane (register spill)")
        if int(u.get("VGPRs", "0")) > MAX_VGPRS:
            bad.append(f"{name}: {u['VGPRs']} VGPRs")
        if int(u.get("LDS", "0")) > MAX_LDS_BYTES:
            bad.append(f"{name}: {u['LDS']} bytes of LDS")
    if bad:
        raise RuntimeError("kernel resource check failed:\n  " + "\n  ".join(bad))


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *srcs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    text = r.stdout + r.stderr
    # drop the feature warning and the remarks with their echoed source lines
    out = "\n".join(l for l in text.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l and "remark:" not in l
                    and not re.match(r"^\s*\d*\s*\|", l))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{out}")
    usage = resource_usage(text)
    if not any("gemm_epilogue_kernel" in k for k in usage):
        raise RuntimeError("no kernel-resource-usage remarks for the GEMM kernels in the compiler output")
    check_usage(usage)
    if verbose:
        if out.strip():
            print(out, file=sys.stderr)
        for name, u in sorted(usage.items()):
            print(f"  {name}: VGPRs {u.get('VGPRs')}, scratch {u.get('ScratchSize')}, LDS {u.get('LDS')}",
                  file=sys.stderr)
    os.replace(tmp, LIB)
    write_build_info()
    build_mfma_ceiling()
    return LIB


CEILING_SRC = os.path.join(CSRC, "mfma_ceiling.hip")
CEILING_EXE = os.path.join(PKG, "mfma_ceiling")


def build_mfma_ceiling() -> str:
    """The MFMA-only probe bench.py runs to measure the device's matrix-core ceiling (not part of the library)."""
    tmp = CEILING_EXE + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-o", tmp, CEILING_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, CEILING_EXE)
    return CEILING_EXE


def write_build_info() -> None:
    """Records the source revision the library was built from (build_info.json, not tracked): a copy of the tree
    without its history (a benchmark machine) can still name it."""
    import json
    import time

    info = {"commit": None, "dirty": None, "built_unix": int(time.time())}
    try:
        git = lambda *a: subprocess.run(["git", *a], cwd=ROOT, capture_output=True, text=True, timeout=10).stdout
        info["commit"] = git("rev-parse", "--short=12", "HEAD").strip() or None
        info["dirty"] = bool(git("status", "--porcelain", "--untracked-files=no").strip())
    except Exception:  # noqa: BLE001 -- no git: nothing to record
        pass
    with open(os.path.join(PKG, "build_info.json"), "w") as f:
        json.dump(info, f)


if __name__ == "__main__":
    print(build(verbose=True))
