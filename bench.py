#!/usr/bin/env python3
"""Benchmark of the fused GEMM -> residual -> RMSNorm -> GEMM block on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one coda_block_fwd call (GEMM1 + residual + partial sums of squares, then GEMM2 on h * gamma whose
workgroups reduce their rows' partial sums to the row scale and apply it and SwiGLU in the epilogue) on inputs
already resident in HBM.
W untimed steps, then K timed steps between two device synchronisations.  Prints ONE JSON line.

Besides the headline the line carries:
  kernels_ms    the block's two kernels timed alone (GEMM1 writing h * gamma in K panels; GEMM2 reading them
                with the reduce folded in), the block, the row-major step entry points (GEMM1, the stand-alone
                reduce, GEMM2 with a given row scale) alone and back to back (the block before the fold and the
                panel layout), and as context GEMM2's product alone through torch.matmul (hipBLASLt, no epilogue)
  block_per_call  the block timed call by call: median, p10 and p90, warm (back to back) and cold (a 512 MiB
                write before each call pushes the operands out of the 256 MB MALL)
  roofline      the dominant kernel (GEMM2 as the block launches it) timed alone with HIP events on the stream
                it runs on, its algorithmic flops (2 M D N2) per launch divided by the average launch time,
                against the published bf16 dense MFMA peak (2.5 PFLOP/s); traffic (K3's bytes per launch at the L2's
                memory side) from the committed rocprofv3 counter summary
                (profiles/hbm_bytes_1b_attn_out_mlp_in.json) if it was taken on the current kernel sources, else null
  cpu_baseline  the fp64 CPU oracle timed on a bounded row sample of the same workload (rows are
                independent), scaled to TFLOP/s, and the GPU block's outputs on those rows compared with it
  unfused       the three-kernel baseline timed the same way, and the algorithmic HBM bytes both paths move
  fp8           the same block with e4m3 X / W1 / W2 (per-row and per-column fp32 scales), fused and unfused,
                and the block-scaled variant, timed with HIP events, against the dense fp8 MFMA peak (5 PFLOP/s)
  backward      the block's backward (dX, dW1, dR, dgamma, dW2 from dz and dh_out; four products of the
                forward's sizes, 2x its flops), fused and unfused, timed with HIP events
  rope          the 1B MLP-out -> QKV block with a rotary embedding of the q and k heads: in GEMM2's epilogue,
                against the plain block and the plain block followed by a separate rotation pass
  ce            cross-entropy of the 1B LM head (V = 128256) with the logits reduced in the GEMM's epilogue,
                against storing bf16 logits and reading them back
  tiny          the 64-row block, launch-bound: microseconds per block called eagerly and replayed from a HIP
                graph
  clock, mfma_ceiling  the shader clock under the block's load (rocm-smi), and what the matrix cores sustain on
                random bf16 operands with no memory traffic (a probe build() compiles); the roofline adds K3's
                fraction of each
  swiglu        the forward that also stores the SwiGLU pre-activation z (against the plain forward), and the
                SwiGLU backward at the 1B down-projection shape, fused into the dgrad product's epilogue and
                unfused (dy stored, then an elementwise pass)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X published dense bf16 MFMA peak
MFMA_FP8_PEAK_TFLOPS = 5000.0   # MI355X published dense fp8 MFMA peak
HBM_PEAK_GBS = 8000.0
METRIC = "fused block TFLOP/s + % bf16 MFMA peak at 1B shape M=8192; HBM bytes saved"
KERNEL_SOURCES = ["gemm_epilogue_fusion_amd/csrc/gemm_core.h", "gemm_epilogue_fusion_amd/csrc/kernels.hip"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(wl, fused: bool) -> int:
    """Compulsory HBM bytes of one block: every input read once, every output written once, plus the
    intermediates each path writes and reads back (part/r for the fused path; T and n for the unfused)."""
    M, K1, D, N2, ny = wl.M, wl.K1, wl.D, wl.N2, wl.n_out
    b = 2 * (M * K1 + K1 * D + M * D + D * N2) + 4 * D   # X, W1, R, W2, gamma
    b += 2 * M * D + 2 * M * ny                          # h, y
    if fused:
        T = D // 256
        b += 2 * 4 * T * M                                # part written + read
        # r written; read back only where the reduce is a kernel of its own (D / 256 > 16), else GEMM2 forms it
        b += 4 * M if T <= 16 else 2 * 4 * M
        b += 2 * 2 * M * D                                # h * gamma written, read back by GEMM2
    else:
        b += 2 * 2 * M * D                                # T written + read
        b += 2 * 2 * M * D + 4 * M                        # n written + read, r written
    return b


HBM_FILE = os.path.join(ROOT, "profiles", "hbm_bytes_1b_attn_out_mlp_in.json")


def kernel_algorithmic_bytes(wl) -> dict:
    """(read, write) compulsory bytes of each kernel of both paths (bf16): every operand read once, every result
    written once."""
    M, K1, D, N2, ny, T = wl.M, wl.K1, wl.D, wl.N2, wl.n_out, wl.D // 256
    return {"K1": (2 * (M * K1 + K1 * D + M * D) + 4 * D, 2 * 2 * M * D + 4 * T * M),
            "K3": (2 * M * D + 2 * D * N2 + 4 * T * M, 2 * M * ny + 4 * M),
            "U1": (2 * (M * K1 + K1 * D), 2 * M * D),
            "U2": (2 * 2 * M * D + 4 * D, 2 * 2 * M * D + 4 * M),
            "U3": (2 * M * D + 2 * D * N2, 2 * M * ny)}


def hbm_bytes_record(wl, fused_alg: int, unfused_alg: int, src_hash: str) -> dict:
    """Algorithmic bytes of both paths, and the counter-measured bytes from the committed summary when it was
    taken on the current kernel sources at this workload (else null, with the reason)."""
    M, D = wl.M, wl.D
    rec = {"fused_algorithmic": fused_alg, "unfused_algorithmic": unfused_alg,
           "saved_algorithmic": unfused_alg - fused_alg,
           # gamma folded into W2's tiles instead, GEMM2 reading h itself: the h * gamma copy is not written (its
           # read becomes a read of h), so the saving would be one [M,D] bf16 store larger; the copy is kept
           # because scaling W2's tiles costs the second GEMM 13-19% of its time
           "saved_algorithmic_if_gamma_folded_into_w2": unfused_alg - fused_alg + 2 * M * D,
           "measured": None}
    if wl.name != "1b_attn_out_mlp_in" or not os.path.exists(HBM_FILE):
        rec["measured_note"] = "no counter summary for this workload"
        return rec
    with open(HBM_FILE) as f:
        m = json.load(f)
    if m.get("kernel_source_hash") != src_hash:
        rec["measured_note"] = f"counter summary taken on other kernel sources ({m.get('kernel_source_hash')})"
        return rec
    rec["measured"] = {k: m[k] for k in ("fused", "unfused", "saved") if k in m}
    rec["measured"]["source"] = os.path.relpath(HBM_FILE, ROOT)
    rec["measured"]["what"] = m.get("what_short")
    return rec


def _bf16_gemm_kernel(name: str, mode: int) -> bool:
    """Whether a kernel name is the general bf16 instantiation of gemm_epilogue_kernel for `mode` (the template's
    FP8 and MX arguments false, and its small-row argument false where the name carries it)."""
    head = f"gemm_epilogue_kernel<{mode}, false, false"
    return head + ">" in name or head + ", false>" in name


def summarize_hbm_counters(dirs: list, out: str, wl) -> dict:
    """Writes the measured-bytes summary from rocprofv3 --pmc runs of
    `bench.py --only-fused --profile-unfused --copy-calibration-mib 1024` (one counter set per run).  Dispatches
    are attributed by kernel name and order: GEMM1 and GEMM2 of the fused block until the first plain-store GEMM,
    then U1, U2, U3 of the unfused block; the last copy kernel is the calibration copy.  Each kernel's value is
    the mean over its dispatches after the first."""
    import csv
    import glob

    vals = {}   # counter -> role -> [values]
    calib = {}
    for d in dirs:
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {d}")
        rows = sorted(csv.DictReader(open(files[0])), key=lambda r: int(r["Dispatch_Id"]))
        seen_store = False
        for r in rows:
            k, c, v = r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])
            if "gemm_epilogue_kernel<1," in k:
                seen_store = True
            role = None
            if _bf16_gemm_kernel(k, 0):
                role = "K1"
            elif _bf16_gemm_kernel(k, 3):
                role = "U3" if seen_store else "K3"
            elif _bf16_gemm_kernel(k, 1):
                role = "U1"
            elif "add_rmsnorm_kernel<false>" in k:
                role = "U2"
            elif "copy" in k.lower():
                calib[c] = v  # the last copy dispatch wins: the calibration copy comes last
            if role:
                vals.setdefault(c, {}).setdefault(role, []).append(v)
    mean = lambda xs: sum(xs[1:]) / len(xs[1:]) if len(xs) > 1 else xs[0]
    copy_bytes = 1 << 30
    fscale = copy_bytes / (calib["FETCH_SIZE"] * 1024)
    wscale = copy_bytes / (calib["WRITE_SIZE"] * 1024)
    alg = kernel_algorithmic_bytes(wl)
    kern = {}
    for role in ("K1", "K3", "U1", "U2", "U3"):
        e = {"read_bytes": round(mean(vals["FETCH_SIZE"][role]) * 1024 * fscale),
             "write_bytes": round(mean(vals["WRITE_SIZE"][role]) * 1024 * wscale),
             "algorithmic_read_bytes": alg[role][0], "algorithmic_write_bytes": alg[role][1]}
        for c in ("TCC_EA0_RDREQ_sum", "TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_WRREQ_sum", "TCC_EA0_WRREQ_DRAM_sum"):
            if c in vals and role in vals[c]:
                e[c] = round(mean(vals[c][role]))
        kern[role] = e
    paths = {"fused": ("K1", "K3"), "unfused": ("U1", "U2", "U3")}
    prof = ("rocprofv3 --pmc {c} --output-format csv -d gpurun_out/hbm/{d} -o run -- python3 bench.py --only-fused "
            "--profile-unfused --steps 10 --warmup 2 --settle-ms 0 --copy-calibration-mib 1024")
    passes = [("FETCH_SIZE", "FETCH_SIZE"), ("WRITE_SIZE", "WRITE_SIZE"),
              ("TCC_EA0_RDREQ_sum TCC_EA0_RDREQ_DRAM_sum", "TCC_EA0_RDREQ_sum"),
              ("TCC_EA0_WRREQ_sum TCC_EA0_WRREQ_DRAM_sum", "TCC_EA0_WRREQ_sum")]
    rec = {"what_short": "rocprofv3 FETCH_SIZE + WRITE_SIZE per kernel, scaled by a 1 GiB copy's readings: bytes at "
                         "the L2's memory side (Infinity Cache hits included)",
           "commands": ["cd /tmp && export TMPDIR=/tmp, then from the repository root, one counter set per run:"]
                       + [prof.format(c=c, d=d) for c, d in passes]
                       + ["python3 bench.py --summarize-hbm-counters " + " ".join(f"gpurun_out/hbm/{d}" for _, d in passes)],
           "note": "The counters sit at the L2's side towards memory: every 128-byte request that misses an XCD's L2, "
                   "served by the 256 MB Infinity Cache or by HBM (the L2 cannot tell them apart; every request is "
                   "addressed to local memory, dram_share = 1).  The copy's FETCH_SIZE reads half the copied bytes (the "
                   "derived counter prices a 128-byte request at 64 bytes) and its read-request count times 128 bytes "
                   "equals the copy, hence fetch_scale 2.  The two GEMM2s read about 8x their operands: each XCD's L2 "
                   "refills the tiles its 32 concurrent workgroups share, mostly from the Infinity Cache.",
           "kernel_source_hash": kernel_source_hash(), "workload": wl.name,
           "calibration": {"copy_bytes": copy_bytes, **{k: v for k, v in calib.items()}, "fetch_scale": round(fscale, 4),
                           "write_scale": round(wscale, 4)},
           "kernels": kern}
    for name, roles in paths.items():
        rd = sum(kern[r]["read_bytes"] for r in roles)
        wr = sum(kern[r]["write_bytes"] for r in roles)
        rec[name] = {"read_bytes": rd, "write_bytes": wr, "total_bytes": rd + wr,
                     "algorithmic_total_bytes": sum(sum(alg[r]) for r in roles)}
        if all("TCC_EA0_RDREQ_DRAM_sum" in kern[r] and "TCC_EA0_RDREQ_sum" in kern[r] for r in roles):
            rec[name]["dram_share_of_read_requests"] = round(
                sum(kern[r]["TCC_EA0_RDREQ_DRAM_sum"] for r in roles) / sum(kern[r]["TCC_EA0_RDREQ_sum"] for r in roles), 4)
        if all("TCC_EA0_WRREQ_DRAM_sum" in kern[r] and "TCC_EA0_WRREQ_sum" in kern[r] for r in roles):
            rec[name]["dram_share_of_write_requests"] = round(
                sum(kern[r]["TCC_EA0_WRREQ_DRAM_sum"] for r in roles) / sum(kern[r]["TCC_EA0_WRREQ_sum"] for r in roles), 4)
    rec["saved"] = {"total_bytes": rec["unfused"]["total_bytes"] - rec["fused"]["total_bytes"],
                    "write_bytes": rec["unfused"]["write_bytes"] - rec["fused"]["write_bytes"],
                    "algorithmic_bytes": rec["unfused"]["algorithmic_total_bytes"] - rec["fused"]["algorithmic_total_bytes"]}
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    return rec


EXTRAS_SETTLE_MS = 200.0  # untimed calls before each secondary measurement (set from --settle-ms in main)


def time_loop(fn, n: int, torch, settle_ms: float = None) -> float:
    """Average ms per call of fn over n back-to-back calls, with HIP events on the current stream, after untimed
    calls for settle_ms of wall time (default EXTRAS_SETTLE_MS; the device clock needs some milliseconds of a
    steady load to settle, and a short window right after other work would otherwise inherit its state)."""
    settle_ms = EXTRAS_SETTLE_MS if settle_ms is None else settle_ms
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(4):
                fn()
            torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(n):
        fn()
    end.record()
    end.synchronize()
    return start.elapsed_time(end) / n


def timed_steps(fn, steps: int, warmup: int, torch, settle_ms: float = 0.0):
    """The contract's timing: untimed calls for at least settle_ms of wall time (0: none), then `warmup` untimed
    calls, then exactly `steps` calls timed by the host clock between two device synchronisations.  A HIP event
    is recorded on the calls' stream before each timed call and after the last, which splits the same wall-clock
    window into per-call times without adding a synchronisation.  Returns (wall ms per call, [event ms per call],
    settle calls made)."""
    settled = 0
    if settle_ms > 0:
        t_end = time.perf_counter() + settle_ms * 1e-3
        while time.perf_counter() < t_end:
            for _ in range(10):
                fn()
            settled += 10
            torch.cuda.synchronize()
    for _ in range(warmup):
        fn()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record()
        fn()
    evs[steps].record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    return wall_ms, [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)], settled


def per_step_summary(per: list) -> dict:
    """Per-step times: mean, median, the nearest-rank 10th and 90th percentiles, first, last, max and the means of
    the first and last thirds (a trend within the window shows as a difference between the two)."""
    import statistics

    t = sorted(per)
    n = len(t)
    q = lambda p: round(t[min(n - 1, int(round(p * (n - 1))))], 4)
    return {"mean": round(sum(per) / n, 4), "first": round(per[0], 4), "last": round(per[-1], 4),
            "median": round(statistics.median(t), 4),
            "p10": q(0.1), "p90": q(0.9), "max": round(t[-1], 4), "first_third_mean": round(
                sum(per[: max(1, n // 3)]) / max(1, n // 3), 4), "last_third_mean": round(
                sum(per[n - max(1, n // 3):]) / max(1, n // 3), 4)}


def environment(torch) -> dict:
    """What ran: the source revision, the software stack and the device."""
    import subprocess

    env = {"commit": None, "csrc_hash": None, "torch": torch.__version__, "hip_runtime": torch.version.hip}
    try:
        env["commit"] = subprocess.run(["git", "rev-parse", "--short=12", "HEAD"], cwd=ROOT, capture_output=True,
                                       text=True, timeout=10).stdout.strip() or None
    except Exception:  # noqa: BLE001 -- a copy of the tree without its history
        pass
    if not env["commit"]:  # the revision recorded when the library was built (build() writes it)
        try:
            with open(os.path.join(ROOT, "gemm_epilogue_fusion_amd", "build_info.json")) as f:
                env["commit"] = json.load(f).get("commit")
            env["commit_from"] = "build_info.json"
        except (OSError, ValueError):
            pass
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "gemm_epilogue_fusion_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    env["csrc_hash"] = h.hexdigest()[:16]
    try:
        with open("/opt/rocm/.info/version") as f:
            env["rocm"] = f.read().strip()
    except OSError:
        env["rocm"] = None
    p = torch.cuda.get_device_properties(0)
    env.update({"gpu": p.name, "arch": getattr(p, "gcnArchName", None), "compute_units": p.multi_processor_count,
                "memory_gib": round(p.total_memory / 2**30, 1)})
    return env


def _find_sclk(obj):
    """The first value under a key that names the shader clock ("sclk") in rocm-smi's JSON, in MHz."""
    if isinstance(obj, dict):
        for k, v in obj.items():
            if "sclk" in str(k).lower() and not isinstance(v, (dict, list)):
                # "1 (2100Mhz)" (level and clock) or "2100Mhz"
                import re
                m = re.search(r"(\d+(?:\.\d+)?)\s*mhz", str(v).lower())
                if m:
                    return float(m.group(1))
                continue
            r = _find_sclk(v)
            if r is not None:
                return r
    elif isinstance(obj, list):
        for v in obj:
            r = _find_sclk(v)
            if r is not None:
                return r
    return None


def _read_sclk_mhz(raw: list):
    """The current shader clock of the device from rocm-smi (MHz), or None; the first raw answers are kept."""
    import subprocess

    p = subprocess.run(["rocm-smi", "--showgpuclocks", "--json"], capture_output=True, text=True, timeout=20)
    if len(raw) < 2:
        raw.append((p.returncode, p.stdout[-600:], p.stderr[-300:]))
    try:
        return _find_sclk(json.loads(p.stdout))
    except ValueError:
        return None


def mfma_ceiling() -> dict:
    """The device's MFMA-only rate on random bf16 operands (no memory traffic) and the shader clock it held, from
    the probe build() compiles (gemm_epilogue_fusion_amd/csrc/mfma_ceiling.hip), run as a child process."""
    import subprocess

    exe = os.path.join(ROOT, "gemm_epilogue_fusion_amd", "mfma_ceiling")
    if not os.path.exists(exe):
        return {"error": "probe not built (build() compiles it)"}
    p = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    rec = json.loads(p.stdout.strip().splitlines()[-1])
    rec["source"] = "gemm_epilogue_fusion_amd/csrc/mfma_ceiling.hip"
    return rec


def clock_under_load(fn, torch, seconds: float = 1.5) -> dict:
    """Shader clock read from rocm-smi a few times while fn runs back to back on the device (the clock the
    block actually runs at: MFMA-bound kernels on random data run below the 2.4 GHz peak clock)."""
    import threading

    samples, raw, stop = [], [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                v = _read_sclk_mhz(raw)
                if v:
                    samples.append(v)
            except Exception as e:  # noqa: BLE001 -- no rocm-smi: no reading
                raw.append(repr(e))
                return
            time.sleep(0.05)

    th = threading.Thread(target=poll, daemon=True)
    for _ in range(5):
        fn()
    torch.cuda.synchronize()
    th.start()
    t_end = time.perf_counter() + seconds
    while time.perf_counter() < t_end:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()
    stop.set()
    th.join(timeout=30)
    out = {"sclk_mhz_samples": samples, "sclk_mhz_median": sorted(samples)[len(samples) // 2] if samples else None,
           "how": "rocm-smi --showgpuclocks while the fused block runs back to back"}
    if not samples:
        out["rocm_smi_answers"] = raw[:2]
    return out


def step_distribution(fn, n: int, torch, scrub=None) -> dict:
    """Per-call ms of fn over n calls, each between its own pair of HIP events: median, p10 and p90.  With
    scrub, scrub() runs before each call outside its events (a write larger than the 256 MB MALL, so the
    call starts with its operands out of the cache)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in evs:
        if scrub is not None:
            scrub()
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in evs)
    q = lambda p: round(t[min(n - 1, int(round(p * (n - 1))))], 4)
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "n": n}


def cpu_baseline(wl, inp, gpu=None, y_eager=None, target_s: float = 15.0) -> dict:
    """The fp64 oracle (fused order) timed on the host on rows 0 .. n-1 of the workload, n sized to about target_s
    seconds, scaled to TFLOP/s.  gpu = (h, y, r) of the GPU's block on the same inputs: the oracle's rows are then
    also compared with the GPU's (normwise and mean errors), after the timing; y_eager (the block as PyTorch
    operators) is compared on the same rows, so that the two errors can be set side by side."""
    import numpy as np
    import torch

    import oracle

    f = lambda t: t.detach().to("cpu", torch.float64).numpy()
    W1, g, W2 = f(inp.W1), f(inp.gamma), f(inp.W2)
    per_row = 2 * (wl.K1 * wl.D + wl.D * wl.N2)
    rows = 64
    t0 = time.perf_counter()
    oracle.block_fused(f(inp.X[:rows]), W1, f(inp.R[:rows]), g, W2, wl.eps, wl.epi)
    dt = time.perf_counter() - t0
    rows2 = int(min(wl.M, max(rows, rows * target_s / max(dt, 1e-3))))
    t0 = time.perf_counter()
    oh, orr, oy = oracle.block_fused(f(inp.X[:rows2]), W1, f(inp.R[:rows2]), g, W2, wl.eps, wl.epi)
    dt2 = time.perf_counter() - t0
    rec = {"value": round(per_row * rows2 / dt2 / 1e12, 6), "unit": "TFLOP/s", "cores": oracle.default_threads(),
           "kind": "oracle",
           "sample": f"fp64 oracle (fused order) on rows 0..{rows2 - 1} of the {wl.M}-row workload, {dt2:.1f} s; "
                     f"rows are independent so the rate scales to the full block"}
    if gpu is not None:
        gh, gy, gr = (f(t[:rows2]) for t in gpu)
        scale = lambda o: max(float(np.max(np.abs(o))), 1e-30)
        rec["parity_on_these_rows"] = {
            "rows": rows2, "y_normwise": float(np.max(np.abs(gy - oy)) / scale(oy)),
            "y_mae_rel": float(np.mean(np.abs(gy - oy)) / scale(oy)),
            "h_normwise": float(np.max(np.abs(gh - oh)) / scale(oh)),
            "r_max_rel": float(np.max(np.abs(gr - orr) / np.abs(orr))),
            "bars": "y normwise <= 2e-2, y MAE/max|o| <= 1e-3, h normwise <= 1e-2"}
        if y_eager is not None:
            ey = f(y_eager[:rows2])
            rec["parity_on_these_rows"]["pytorch_eager_y_normwise"] = float(np.max(np.abs(ey - oy)) / scale(oy))
            rec["parity_on_these_rows"]["pytorch_eager_y_mae_rel"] = float(np.mean(np.abs(ey - oy)) / scale(oy))
    return rec


def eager_block(X, W1, R, gamma, W2, wl, torch):
    """The block as separate PyTorch operators on bf16 tensors, the kind of baseline the write-up measures
    against (a vendor GEMM library plus framework operators): T = X W1 and z = n W2 through torch.matmul
    (hipBLASLt on ROCm), the residual add, torch's RMSNorm and SwiGLU as operators of their own."""
    import torch.nn.functional as F

    g16 = gamma.to(torch.bfloat16)
    half = wl.N2 // 2

    def run():
        hh = torch.matmul(X, W1) + R
        n = F.rms_norm(hh, (wl.D,), g16, wl.eps)
        z = torch.matmul(n, W2)
        return F.silu(z[:, :half]) * z[:, half:] if wl.epi == 1 else z

    return run


def time_fp8(dev, n_ev: int, warmup: int, torch, cb) -> dict:
    """The e4m3 version of the headline block: fused and unfused, average ms per call by HIP events."""
    from gemm_epilogue_fusion_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["1b_attn_out_mlp_in_fp8"]
    inp = make_inputs(wl)
    a = [t.to(dev) for t in (inp.Xq, inp.sx, inp.W1q, inp.sw1, inp.R, inp.gamma, inp.W2q, inp.sw2)]
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev, fp8=1)
    wsu = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=1, device=dev, fp8=1)
    wsm = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev, fp8=2)
    fused = lambda: cb.coda_block_fwd_fp8(*a, wl.eps, wl.epi, h, y, ws)
    unfused = lambda: cb.coda_block_unfused_fp8(*a, wl.eps, wl.epi, h, y, wsu)
    mx = lambda: cb.coda_block_fwd_fp8_mx(*a, wl.eps, wl.epi, h, y, wsm)
    for _ in range(warmup):
        fused()
        unfused()
        mx()
    torch.cuda.synchronize()
    f_ms = time_loop(fused, n_ev, torch)
    u_ms = time_loop(unfused, n_ev, torch)
    m_ms = time_loop(mx, n_ev, torch)
    tf = wl.flops / (f_ms * 1e-3) / 1e12
    tm = wl.flops / (m_ms * 1e-3) / 1e12
    return {"workload": wl.name, "dtype": "e4m3 operands, fp32 accumulate, bf16 h/y",
            "fused_ms": round(f_ms, 4), "tflops": round(tf, 2),
            "pct_fp8_mfma_peak": round(100 * tf / MFMA_FP8_PEAK_TFLOPS, 2), "unfused_ms": round(u_ms, 4),
            "speedup_fused_vs_unfused": round(u_ms / f_ms, 4),
            "block_scaled": {"what": "second GEMM's A operand quantised in the first GEMM's epilogue, one "
                                     "power-of-two scale per 32 values; the reduce folded in (2 kernels)",
                             "fused_ms": round(m_ms, 4), "tflops": round(tm, 2),
                             "pct_fp8_mfma_peak": round(100 * tm / MFMA_FP8_PEAK_TFLOPS, 2),
                             "speedup_vs_unfused": round(u_ms / m_ms, 4)}}


def time_bwd(wl, X, W1, g, W2, h, ws, n_ev: int, warmup: int, torch, cb) -> dict:
    """The backward of the headline block (h and r as the forward left them), fused and unfused."""
    from gemm_epilogue_fusion_amd.inputs import make_grads

    dev = X.device
    dz, dho = (t.to(dev) for t in make_grads(wl))
    r = cb.workspace_r(ws, wl.M, wl.D)
    outs = (torch.empty(wl.M, wl.K1, dtype=torch.bfloat16, device=dev),
            torch.empty(wl.K1, wl.D, dtype=torch.float32, device=dev),
            torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev),
            torch.empty(wl.D, dtype=torch.float32, device=dev),
            torch.empty(wl.D, wl.N2, dtype=torch.float32, device=dev))
    wsf = cb.alloc_bwd_workspace(wl.M, wl.K1, wl.D, wl.N2, device=dev)
    wsu = cb.alloc_bwd_workspace(wl.M, wl.K1, wl.D, wl.N2, unfused=1, device=dev)
    W2t = W2.t().contiguous()  # the [out, in] copy a caller keeping weights that way already holds
    fused = lambda: cb.coda_block_bwd(X, W1, h, r, g, W2, dz, dho, *outs, wsf)
    fused_w2t = lambda: cb.coda_block_bwd_w2t(X, W1, h, r, g, W2t, dz, dho, *outs, wsf)
    unfused = lambda: cb.coda_block_bwd_unfused(X, W1, h, r, g, W2, dz, dho, *outs, wsu)
    # context: the same gradients as PyTorch operators (bf16 products through torch.matmul, fp32 elementwise);
    # the weights' transposes are made once outside the timing, the activations' (X^T, u^T) as copies inside it
    W1t = W1.t().contiguous()
    bf = torch.bfloat16
    rc = r[:, None]

    def eager():
        n = h.float() * rc
        u = (n * g).to(bf)
        du = torch.matmul(dz, W2t).float()
        dgamma = (du * n).sum(0)
        dug = du * g
        dh = (rc * (dug - n * (dug * n).mean(1, keepdim=True)) + dho.float()).to(bf)
        return (torch.matmul(dh, W1t), torch.matmul(X.t().contiguous(), dh), dh, dgamma,
                torch.matmul(u.t().contiguous(), dz))

    for _ in range(warmup):
        fused()
        fused_w2t()
        unfused()
        eager()
    torch.cuda.synchronize()
    f_ms = time_loop(fused, n_ev, torch)
    t_ms = time_loop(fused_w2t, n_ev, torch)
    u_ms = time_loop(unfused, n_ev, torch)
    e_ms = time_loop(eager, n_ev, torch)
    flops = 2 * wl.flops
    tf = flops / (f_ms * 1e-3) / 1e12
    return {"what": "dX, dW1, dR, dgamma, dW2 from dz and dh_out", "flops_per_call": flops, "fused_ms": round(f_ms, 4),
            "tflops": round(tf, 2), "pct_bf16_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2),
            "fused_w2t_ms": round(t_ms, 4), "unfused_ms": round(u_ms, 4),
            "speedup_fused_vs_unfused": round(u_ms / f_ms, 4),
            "pytorch_eager_ms": round(e_ms, 4), "speedup_fused_vs_pytorch_eager": round(e_ms / f_ms, 4)}


def time_tiny(dev, torch, cb) -> dict:
    """The tiny block (M=64, K1=D=256, N2=512), launch-bound: microseconds per block called eagerly (two kernel
    launches through the C ABI each) and replayed from a HIP graph holding 50 blocks, and the unfused baseline (three
    kernels) called eagerly the same way."""
    from gemm_epilogue_fusion_amd.inputs import WORKLOADS, make_inputs

    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    X, W1, R, g, W2 = (t.to(dev) for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
    call = lambda: cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    eager_ms = time_loop(call, 500, torch)
    ws_u = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=1, device=dev)
    unfused_ms = time_loop(lambda: cb.coda_block_unfused(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws_u), 500, torch)
    per_graph = 50
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(per_graph):
            call()
    graph.replay()
    torch.cuda.synchronize()
    graph_ms = time_loop(graph.replay, 20, torch) / per_graph
    return {"workload": wl.name, "M": wl.M, "K1": wl.K1, "D": wl.D, "N2": wl.N2, "kernels_per_block": 2,
            "eager_us_per_block": round(eager_ms * 1e3, 2), "graph_us_per_block": round(graph_ms * 1e3, 2),
            "graph_blocks_per_replay": per_graph, "unfused_eager_us_per_block": round(unfused_ms * 1e3, 2),
            "speedup_fused_vs_unfused_eager": round(unfused_ms / eager_ms, 4)}


def time_row_shard(dev, n_ev: int, torch, cb) -> dict:
    """One GPU's share of the two bf16 1B blocks with their rows sharded over eight GPUs (1024 of 8192 rows; no
    communication, the rows are independent): the fused block with the split of the GEMMs' last waves (the default
    workspace), the same block given a workspace without the split room (whole tiles, except that a second GEMM's
    last wave then runs as 128-row halves, which need no room), and the unfused baseline with its split;
    milliseconds per call from HIP events after EXTRAS_SETTLE_MS of untimed calls."""
    from gemm_epilogue_fusion_amd.inputs import WORKLOADS, make_inputs

    out = {}
    for name in ("1b_attn_out_mlp_in", "1b_mlp_out_qkv"):
        wl = WORKLOADS[name].with_(M=1024)
        inp = make_inputs(wl)
        X, W1, R, g, W2 = (t.to(dev) for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
        h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
        y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
        ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
        ws_whole = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev, split=False)
        wsu = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=1, device=dev)
        split = lambda: cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws)
        whole = lambda: cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws_whole)
        unf = lambda: cb.coda_block_unfused(X, W1, R, g, W2, wl.eps, wl.epi, h, y, wsu)
        ms = {k: time_loop(fn, n_ev, torch) for k, fn in (("split", split), ("no_room", whole), ("unfused", unf))}
        out[name + "_1024_rows"] = {
            "M": wl.M, "K1": wl.K1, "D": wl.D, "N2": wl.N2, "split_room_bytes": ws.numel() - ws_whole.numel(),
            "fused_ms": round(ms["split"], 4), "fused_without_split_room_ms": round(ms["no_room"], 4),
            "unfused_ms": round(ms["unfused"], 4),
            "tflops": round(wl.flops / (ms["split"] * 1e-3) / 1e12, 2),
            "speedup_split_vs_without_room": round(ms["no_room"] / ms["split"], 4)}
        del ws, ws_whole, wsu
    return out


def time_rope(dev, n_ev: int, warmup: int, torch, cb) -> dict:
    """The QKV block with RoPE on the q and k heads (32 + 8 heads of 64 of the 48), seq_len 2048, base 5e5:
    fused into GEMM2's epilogue, against the plain block alone and the plain block + a separate pass."""
    from gemm_epilogue_fusion_amd.inputs import EPI_IDENTITY, WORKLOADS, make_inputs

    wl = WORKLOADS["1b_mlp_out_qkv"]
    seq_len, n_rot, base = 2048, 2560, 500000.0
    inp = make_inputs(wl)
    X, W1, R, g, W2 = (t.to(dev) for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.N2, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_IDENTITY, device=dev)
    plain = lambda: cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, EPI_IDENTITY, h, y, ws)
    fused = lambda: cb.coda_block_fwd_rope(X, W1, R, g, W2, wl.eps, seq_len, n_rot, base, h, y, ws)

    def separate():
        plain()
        cb.coda_rope_rows(y, seq_len, n_rot, base)

    for _ in range(warmup):
        plain()
        fused()
        separate()
    torch.cuda.synchronize()
    p_ms, f_ms, s_ms = (time_loop(fn, n_ev, torch) for fn in (plain, fused, separate))
    return {"workload": wl.name, "seq_len": seq_len, "n_rope_cols": n_rot, "rope_base": base,
            "fused_ms": round(f_ms, 4), "tflops": round(wl.flops / (f_ms * 1e-3) / 1e12, 2),
            "plain_block_ms": round(p_ms, 4), "separate_pass_ms": round(s_ms, 4),
            "fused_overhead_vs_plain_pct": round(100 * (f_ms / p_ms - 1), 2),
            "speedup_fused_vs_separate": round(s_ms / f_ms, 4),
            "hbm_bytes_saved_algorithmic": 2 * 2 * wl.M * n_rot}


def time_ce(dev, n_ev: int, warmup: int, torch, cb) -> dict:
    """Cross-entropy of the 1B LM head (M=8192, D=2048, V=128256) with the logits never stored, against the
    baseline that stores bf16 logits and reads them back."""
    from gemm_epilogue_fusion_amd.inputs import CE_WORKLOADS, make_ce_inputs

    wl = CE_WORKLOADS["1b_lm_head"]
    H, W, labels = (t.to(dev) for t in make_ce_inputs(wl))
    loss = torch.empty(wl.M, dtype=torch.float32, device=dev)
    lse = torch.empty(wl.M, dtype=torch.float32, device=dev)
    ws = cb.alloc_ce_workspace(wl.M, wl.D, wl.V, device=dev)
    wsu = cb.alloc_ce_workspace(wl.M, wl.D, wl.V, unfused=1, device=dev)
    fused = lambda: cb.coda_ce_fwd(H, W, labels, loss, lse, ws)
    unfused = lambda: cb.coda_ce_unfused(H, W, labels, loss, lse, wsu)
    # context: torch.matmul for the bf16 logits, then torch's cross-entropy over them in fp32 (labels < 0 ignored)
    lab64 = labels.long()
    eager = lambda: torch.nn.functional.cross_entropy(torch.matmul(H, W).float(), lab64, reduction="none",
                                                       ignore_index=-100)
    for _ in range(warmup):
        fused()
        unfused()
        eager()
    torch.cuda.synchronize()
    n = max(5, n_ev // 4)
    f_ms = time_loop(fused, n, torch)
    u_ms = time_loop(unfused, n, torch)
    e_ms = time_loop(eager, n, torch)
    tf = wl.flops / (f_ms * 1e-3) / 1e12
    T = wl.V // 256
    saved = 2 * 2 * wl.M * wl.V - 2 * (2 * 4 * T * wl.M + 4 * wl.M)  # logits written + read, minus partials
    return {"workload": wl.name, "M": wl.M, "D": wl.D, "V": wl.V, "fused_ms": round(f_ms, 4), "tflops": round(tf, 2),
            "pct_bf16_mfma_peak": round(100 * tf / MFMA_BF16_PEAK_TFLOPS, 2), "unfused_ms": round(u_ms, 4),
            "speedup_fused_vs_unfused": round(u_ms / f_ms, 4), "pytorch_eager_ms": round(e_ms, 4),
            "speedup_fused_vs_pytorch_eager": round(e_ms / f_ms, 4), "hbm_bytes_saved_algorithmic": saved}


def time_swiglu(wl, X, W1, R, g, W2, dev, n_ev: int, warmup: int, torch, cb) -> dict:
    """The SwiGLU pieces of training: the forward that also stores z (against the plain forward), and the
    SwiGLU backward at the 1B down-projection shape, fused (dy reduced into dz in the epilogue) and unfused."""
    from gemm_epilogue_fusion_amd.inputs import EPI_SWIGLU, SWIGLU_BWD_WORKLOADS, make_swiglu_bwd_inputs

    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.N2 // 2, dtype=torch.bfloat16, device=dev)
    z = torch.empty(wl.M, wl.N2, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, EPI_SWIGLU, device=dev)
    plain = lambda: cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, EPI_SWIGLU, h, y, ws)
    savez = lambda: cb.coda_block_fwd_save_z(X, W1, R, g, W2, wl.eps, h, y, z, ws)
    bw = SWIGLU_BWD_WORKLOADS["1b_mlp_down_dgrad"]
    dout, Wd, zz = (t.to(dev) for t in make_swiglu_bwd_inputs(bw))
    dz = torch.empty(bw.M, 2 * bw.F, dtype=torch.bfloat16, device=dev)
    wsu = torch.empty(cb.coda_swiglu_bwd_workspace_bytes(bw.M, bw.F, 1), dtype=torch.uint8, device=dev)
    fused = lambda: cb.coda_swiglu_bwd(dout, Wd, zz, dz)
    unfused = lambda: cb.coda_swiglu_bwd_unfused(dout, Wd, zz, dz, wsu)
    # context: the same dz as PyTorch operators (dy through torch.matmul with Wd's transpose made once outside
    # the timing, then silu's derivative in fp32)
    WdT = Wd.t().contiguous()
    F_ = bw.F

    def eager():
        dy = torch.matmul(dout, WdT).float()
        gt, ut = zz[:, :F_].float(), zz[:, F_:].float()
        sg = torch.sigmoid(gt)
        return torch.cat(((dy * ut * sg * (1 + gt * (1 - sg))).to(torch.bfloat16), (dy * gt * sg).to(torch.bfloat16)), 1)

    for _ in range(warmup):
        plain()
        savez()
        fused()
        unfused()
        eager()
    torch.cuda.synchronize()
    p_ms, z_ms, f_ms, u_ms, e_ms = (time_loop(fn, n_ev, torch) for fn in (plain, savez, fused, unfused, eager))
    return {"forward_save_z": {"workload": wl.name, "ms": round(z_ms, 4), "plain_forward_ms": round(p_ms, 4),
                               "z_bytes_written": 2 * wl.M * wl.N2},
            "backward": {"workload": bw.name, "M": bw.M, "D": bw.D, "F": bw.F, "fused_ms": round(f_ms, 4),
                         "tflops": round(bw.flops / (f_ms * 1e-3) / 1e12, 2), "unfused_ms": round(u_ms, 4),
                         "speedup_fused_vs_unfused": round(u_ms / f_ms, 4),
                         "pytorch_eager_ms": round(e_ms, 4), "speedup_fused_vs_pytorch_eager": round(e_ms / f_ms, 4),
                         "hbm_bytes_saved_algorithmic": 2 * 2 * bw.M * bw.F}}


def traffic_record(src_hash: str, wl_name: str):
    """K3's measured bytes per launch (reads + writes at the L2's memory side) from the committed counter summary,
    if it was taken on the current kernel sources at this workload."""
    if not os.path.exists(HBM_FILE):
        return None
    with open(HBM_FILE) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != src_hash or rec.get("workload") != wl_name:
        return None
    k3 = rec["kernels"]["K3"]
    return {"bytes_per_launch": k3["read_bytes"] + k3["write_bytes"]}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="1b_attn_out_mlp_in")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-fp8", action="store_true", help="skip the e4m3 block timing")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-rope", action="store_true", help="skip the rotary-embedding block timing")
    ap.add_argument("--no-ce", action="store_true", help="skip the cross-entropy timing")
    ap.add_argument("--no-swiglu", action="store_true", help="skip the SwiGLU forward-with-z / backward timing")
    ap.add_argument("--no-tiny", action="store_true", help="skip the launch-bound tiny block (eager and graph)")
    ap.add_argument("--no-shard", action="store_true",
                    help="skip the 1024-row blocks (one GPU's share of the rows sharded over eight)")
    ap.add_argument("--settle-ms", type=float, default=500.0,
                    help="untimed calls for at least this many ms before the warm-up calls of each timed window: the "
                         "device's clock settles under sustained load only after some milliseconds (0: none)")
    ap.add_argument("--no-clock", action="store_true", help="skip the shader-clock reading under load")
    ap.add_argument("--only-fused", action="store_true", help="time the fused block only (for profiling runs)")
    ap.add_argument("--profile-unfused", action="store_true",
                    help="with --only-fused: after the fused steps run the unfused block `steps` times (counter runs "
                         "attribute dispatches to the two paths by their order)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the run, copy a buffer of this many MiB once (a plain copy of known size, the "
                         "reference that scales the HBM byte counters of a profiling run)")
    ap.add_argument("--summarize-hbm-counters", nargs="+", metavar="DIR",
                    help="write the measured-bytes summary (profiles/) from these rocprofv3 --pmc output folders and "
                         "exit (no GPU needed)")
    args = ap.parse_args()

    if args.summarize_hbm_counters:
        from gemm_epilogue_fusion_amd.inputs import WORKLOADS as _W
        rec = summarize_hbm_counters(args.summarize_hbm_counters, HBM_FILE, _W[args.workload])
        print(json.dumps({k: rec[k] for k in ("fused", "unfused", "saved")}))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this block runs on one GPU; multi-GPU runs are not part of it "
              "(the forward pass shards along rows with no communication).", file=sys.stderr)
        return 2

    import torch

    from gemm_epilogue_fusion_amd import binding as cb
    from gemm_epilogue_fusion_amd.inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py: no GPU", file=sys.stderr)
        return 2
    cb.load()
    global EXTRAS_SETTLE_MS
    EXTRAS_SETTLE_MS = min(args.settle_ms, 200.0)
    wl = WORKLOADS[args.workload]
    if wl.fp8:
        print("bench.py: fp8 workload is benchmarked with its own entry point", file=sys.stderr)
        return 2
    inp = make_inputs(wl)
    dev = torch.device("cuda:0")
    X, W1, R, g, W2 = (t.to(dev) for t in (inp.X, inp.W1, inp.R, inp.gamma, inp.W2))
    h = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    y = torch.empty(wl.M, wl.n_out, dtype=torch.bfloat16, device=dev)
    ws = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, device=dev)
    ws_u = cb.alloc_workspace(wl.M, wl.K1, wl.D, wl.N2, wl.epi, unfused=1, device=dev)

    def step():
        cb.coda_block_fwd(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws)

    def step_unfused():
        cb.coda_block_unfused(X, W1, R, g, W2, wl.eps, wl.epi, h, y, ws_u)

    # the headline: the contract's timing (host clock around exactly K calls after W warm-up calls), with a HIP
    # event before each call splitting the same window; the unfused baseline is timed the same way right after
    with torch.cuda.nvtx.range("bench:headline_fused"):
        ms, per_fused, settled = timed_steps(step, args.steps, args.warmup, torch, args.settle_ms)
    tflops = wl.flops / (ms * 1e-3) / 1e12
    if args.only_fused:
        if args.profile_unfused:
            for _ in range(args.steps):
                step_unfused()
            torch.cuda.synchronize()
        if args.copy_calibration_mib:
            n = args.copy_calibration_mib * (1 << 20)
            src = torch.ones(n, dtype=torch.uint8, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": ms}))
        return 0
    with torch.cuda.nvtx.range("bench:headline_unfused"):
        unf_ms, per_unfused, _ = timed_steps(step_unfused, args.steps, args.warmup, torch, args.settle_ms)
    # context: the same block as PyTorch operators, timed the same way in a window of its own
    eager = eager_block(X, W1, R, g, W2, wl, torch)
    with torch.cuda.nvtx.range("bench:pytorch_eager"):
        eager_ms, per_eager, _ = timed_steps(eager, args.steps, args.warmup, torch, args.settle_ms)
    step()
    y_eager = eager()
    torch.cuda.synchronize()
    eager_rec = {"what": "the block as PyTorch operators on bf16 tensors: torch.matmul (hipBLASLt) for both products, "
                         "the residual add, torch.nn.functional.rms_norm and SwiGLU as separate operators",
                 "ms_per_step_wall": round(eager_ms, 4), "per_step_events_ms": per_step_summary(per_eager),
                 "speedup_fused_vs_eager_wall": round(eager_ms / ms, 4),
                 "y_normwise_vs_fused": round(float((y_eager.float() - y.float()).abs().max()
                                                    / y.float().abs().max().clamp_min(1e-30)), 5)}
    y_eager_host = y_eager.cpu()  # for the oracle leg: the PyTorch operators' y against the oracle, same rows
    del y_eager

    # per-step kernels timed alone with HIP events (same stream as the launches: torch's current stream).
    # The block's own kernels: K1 writing h * gamma in K panels, and K3 reading them with the reduce folded in
    # (the dominant kernel).  The row-major step entry points (K1, the reduce kernel, K3) are timed too: the
    # three back to back are the block before the fold and the panel layout.
    T = wl.D // 256
    part = torch.empty(T, wl.M, dtype=torch.float32, device=dev)
    r = torch.empty(wl.M, dtype=torch.float32, device=dev)
    hg = torch.empty(wl.M, wl.D, dtype=torch.bfloat16, device=dev)
    hgp = torch.empty(wl.D // 32, wl.M, 32, dtype=torch.bfloat16, device=dev)
    n_ev = max(20, args.steps // 2)
    # the block folds the reduce into K3 where D / 256 <= 16 (D <= 4096); above that the reduce is a kernel of its
    # own and K3 reads r
    fold = wl.D // 256 <= 16
    k1p = lambda: cb.coda_gemm1_residual_partial_rms_panels(X, W1, R, g, h, hgp, part)
    if fold:
        k3p = lambda: cb.coda_gemm2_rowscale_panels(hgp, W2, part, wl.eps, r, wl.epi, y)
    else:
        cb.coda_gemm1_residual_partial_rms_panels(X, W1, R, g, h, hgp, part)
        cb.coda_partial_rms_reduce(part, wl.D, wl.eps, r)
        k3p = lambda: cb.coda_gemm2_rowscale_panels(hgp, W2, None, wl.eps, r, wl.epi, y)
    k1 = lambda: cb.coda_gemm1_residual_partial_rms(X, W1, R, g, h, hg, part)
    k2 = lambda: cb.coda_partial_rms_reduce(part, wl.D, wl.eps, r)
    k3 = lambda: cb.coda_gemm2_rowscale(hg, W2, r, wl.epi, y)
    for fn in (k1p, k3p, k1, k2, k3):
        fn()
    torch.cuda.synchronize()
    k1p_ms, k3_ms, k1_ms, k2_ms, k3r_ms = (time_loop(fn, n_ev, torch) for fn in (k1p, k3p, k1, k2, k3))
    def three_steps():  # the row-major steps, with the reduce as its own kernel between the two GEMMs
        k1()
        k2()
        k3()

    three_ms = time_loop(three_steps, n_ev, torch)
    for _ in range(args.warmup):
        step_unfused()
    unf_ev_ms = time_loop(step_unfused, n_ev, torch)
    fused_ev_ms = time_loop(step, n_ev, torch)

    # per-call spread, warm (back to back) and cold (a 512 MiB write between calls evicts the MALL)
    scrub_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    n_dist = min(100, n_ev)
    dist = {"warm_ms": step_distribution(step, n_dist, torch),
            "cold_ms": step_distribution(step, n_dist, torch, scrub=lambda: scrub_buf.fill_(1))}
    del scrub_buf
    # context: the GEMM2 product alone through torch.matmul (hipBLASLt), no epilogue
    mm_out = torch.empty(wl.M, wl.N2, dtype=torch.bfloat16, device=dev)
    mm = lambda: torch.matmul(hg, W2, out=mm_out)
    for _ in range(3):
        mm()
    torch.cuda.synchronize()
    mm_ms = time_loop(mm, n_ev, torch)
    del mm_out

    k3_flops = 2 * wl.M * wl.D * wl.N2
    k3_tflops = k3_flops / (k3_ms * 1e-3) / 1e12
    src_hash = kernel_source_hash()
    traffic = traffic_record(src_hash, wl.name)
    roofline = {"bound": "mfma", "achieved": round(k3_tflops, 2), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(k3_tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": ("gemm_epilogue_kernel<MODE_ROWSCALE_SWIGLU>" if wl.epi == 1 else
                           "gemm_epilogue_kernel<MODE_ROWSCALE>") + " as the block launches it (GEMM2 on h * gamma in K "
                          "panels, " + ("partial-RMS reduce folded in" if fold else "r from the reduce kernel") +
                          ", row scale" + (" + SwiGLU)" if wl.epi == 1 else ", identity epilogue)"),
                "kernel_ms": round(k3_ms, 4), "algorithmic_flops_per_launch": k3_flops}

    fb, ub = algorithmic_bytes(wl, True), algorithmic_bytes(wl, False)
    ev_f, ev_u = sum(per_fused) / len(per_fused), sum(per_unfused) / len(per_unfused)
    line = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded Gaussian inputs of the workload's shapes)",
        "config": {"workload": wl.name, "M": wl.M, "K1": wl.K1, "D": wl.D, "N2": wl.N2,
                   "epilogue": "swiglu" if wl.epi else "identity", "eps": wl.eps},
        "pct_bf16_mfma_peak": round(100 * tflops / MFMA_BF16_PEAK_TFLOPS, 2),
        "roofline": roofline,
        "timing": {
            "ms_per_step": "host clock around exactly `steps` calls after `warmup` warm-up calls (and settle_ms of "
                           "untimed calls before them), between two device synchronisations",
            "settle_ms": args.settle_ms, "settle_calls": settled,
            "fused_per_step_events_ms": per_step_summary(per_fused),
            "events_ms": "HIP events on the calls' stream: in the timed window one event before each call "
                         "(per_step), elsewhere one pair around n back-to-back calls (mean per call) after "
                         "extras_settle_ms of untimed calls of the same function",
            "extras_settle_ms": EXTRAS_SETTLE_MS,
        },
        "unfused": {"ms_per_step_wall": round(unf_ms, 4), "per_step_events_ms": per_step_summary(per_unfused),
                    "tflops_wall": round(wl.flops / (unf_ms * 1e-3) / 1e12, 2),
                    "speedup_fused_vs_unfused_wall": round(unf_ms / ms, 4),
                    "speedup_fused_vs_unfused_events_same_window": round(ev_u / ev_f, 4),
                    "ms_per_call_events": round(unf_ev_ms, 4), "fused_ms_per_call_events": round(fused_ev_ms, 4),
                    "speedup_fused_vs_unfused_events": round(unf_ev_ms / fused_ev_ms, 4)},
        "pytorch_eager": eager_rec,
        "kernels_ms": {"gemm1_res_prms": round(k1p_ms, 4), ("gemm2_rowscale_fold" if fold else "gemm2_rowscale"): round(k3_ms, 4),
                       "fused_block_events": round(fused_ev_ms, 4),
                       "row_major_steps": {"gemm1_res_prms": round(k1_ms, 4), "prms_reduce": round(k2_ms, 4),
                                           "gemm2_rowscale": round(k3r_ms, 4),
                                           "three_back_to_back": round(three_ms, 4)},
                       "torch_matmul_gemm2_product_only": round(mm_ms, 4)},
        "block_per_call": dist,
        "hbm_bytes": hbm_bytes_record(wl, fb, ub, src_hash),
        "kernel_source_hash": src_hash,
    }
    def extra(key, fn):
        # the further measurements: a Python-level failure in one of them (an error status from the library,
        # an allocation failure) is recorded under its key and the line is still printed with the headline.
        # Each runs inside a named marker range (roctx through torch.cuda.nvtx), which a trace taken with
        # rocprofv3 --marker-trace shows around the section's kernels.
        try:
            with torch.cuda.nvtx.range(f"bench:{key}"):
                line[key] = fn()
        except Exception as e:  # noqa: BLE001
            print(f"bench: {key} failed: {e!r}", file=sys.stderr, flush=True)
            line[key] = {"error": repr(e)}

    if not args.no_bwd:
        extra("backward", lambda: time_bwd(wl, X, W1, g, W2, h, ws, n_ev, args.warmup, torch, cb))
    if not args.no_fp8:
        extra("fp8", lambda: time_fp8(dev, n_ev, args.warmup, torch, cb))
    if not args.no_rope:
        extra("rope", lambda: time_rope(dev, n_ev, args.warmup, torch, cb))
    if not args.no_ce:
        extra("ce", lambda: time_ce(dev, n_ev, args.warmup, torch, cb))
    if not args.no_swiglu and wl.epi == 1:
        extra("swiglu", lambda: time_swiglu(wl, X, W1, R, g, W2, dev, n_ev, args.warmup, torch, cb))
    if not args.no_tiny:
        extra("tiny", lambda: time_tiny(dev, torch, cb))
    if not args.no_shard:
        extra("row_shard", lambda: time_row_shard(dev, n_ev, torch, cb))
    extra("env", lambda: environment(torch))
    if not args.no_clock:
        extra("clock", lambda: clock_under_load(step, torch))
        mhz = line.get("clock", {}).get("sclk_mhz_median")
        if mhz:
            # the same kernel against the peak at the shader clock it ran at (MFMA-bound kernels on random data run
            # below the 2.4 GHz the published peak assumes)
            peak_at_clock = MFMA_BF16_PEAK_TFLOPS * mhz / 2400.0
            roofline["frac_at_measured_clock"] = round(k3_tflops / peak_at_clock, 4)
            roofline["peak_at_measured_clock"] = round(peak_at_clock, 1)
    if not args.no_clock:
        extra("mfma_ceiling", mfma_ceiling)
        ceil = line.get("mfma_ceiling", {}).get("tflops")
        if ceil:
            # the same kernel against what the matrix cores sustain on random data with no memory traffic at all
            roofline["frac_of_mfma_ceiling"] = round(k3_tflops / ceil, 4)
        ceil8 = line.get("mfma_ceiling", {}).get("fp8", {}).get("tflops")
        f8 = line.get("fp8", {})
        if ceil8 and "tflops" in f8:
            f8["frac_of_fp8_mfma_ceiling"] = round(f8["tflops"] / ceil8, 4)
            if "tflops" in f8.get("block_scaled", {}):
                f8["block_scaled"]["frac_of_fp8_mfma_ceiling"] = round(f8["block_scaled"]["tflops"] / ceil8, 4)
    if not args.no_cpu_baseline:
        def gpu_outputs():  # the block's outputs on these inputs, for the oracle leg's comparison
            step()
            torch.cuda.synchronize()
            return h.clone(), y.clone(), cb.workspace_r(ws, wl.M, wl.D).clone()

        extra("cpu_baseline", lambda: cpu_baseline(wl, inp, gpu_outputs(), y_eager_host))
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
