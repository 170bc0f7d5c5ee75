"""Host logic of bench.py (no GPU): the byte accounting, the per-step statistics, the gating of measured bytes
on the kernel sources and the workload, the counter summary's attribution of dispatches, and the one-GPU rule."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from gemm_epilogue_fusion_amd.inputs import WORKLOADS  # noqa: E402


@pytest.mark.parametrize("name", ["1b_attn_out_mlp_in", "1b_mlp_out_qkv", "8b_attn_out_mlp_in", "tiny"])
def test_block_bytes_are_the_sum_of_their_kernels(name):
    """The two accountings are written separately: the block totals must equal the sums over their kernels (the
    fused path's K1 + K3 with the reduce folded in, the unfused U1 + U2 + U3)."""
    wl = WORKLOADS[name]
    k = bench.kernel_algorithmic_bytes(wl)
    assert wl.D // 256 <= 16
    assert bench.algorithmic_bytes(wl, True) == sum(sum(k[r]) for r in ("K1", "K3"))
    assert bench.algorithmic_bytes(wl, False) == sum(sum(k[r]) for r in ("U1", "U2", "U3"))


def test_headline_saving():
    """At the 1B shape the fused path saves T and n written and read (4 x 2MD) minus the h * gamma copy written and
    read (2 x 2MD) and the partial sums (2 x 4 (D/256) M), plus U2's r store being the one K3 makes."""
    wl = WORKLOADS["1b_attn_out_mlp_in"]
    M, D = wl.M, wl.D
    saved = bench.algorithmic_bytes(wl, False) - bench.algorithmic_bytes(wl, True)
    assert saved == 4 * 2 * M * D - 2 * 2 * M * D - 2 * 4 * (D // 256) * M
    assert saved == 66584576


def test_per_step_summary():
    s = bench.per_step_summary([5.0, 1.0, 2.0, 3.0, 4.0, 6.0, 7.0, 8.0, 9.0, 10.0])
    assert s["mean"] == 5.5 and s["first"] == 5.0 and s["last"] == 10.0 and s["max"] == 10.0
    assert s["median"] == 5.5 and s["p10"] == 2.0 and s["p90"] == 9.0
    assert s["first_third_mean"] == round((5 + 1 + 2) / 3, 4) and s["last_third_mean"] == 9.0


def test_measured_bytes_gating(tmp_path, monkeypatch):
    wl = WORKLOADS["1b_attn_out_mlp_in"]
    f = tmp_path / "hbm.json"
    rec = {"kernel_source_hash": "abc", "workload": wl.name, "fused": {"total_bytes": 1}, "unfused": {"total_bytes": 3},
           "saved": {"total_bytes": 2}, "kernels": {"K3": {"read_bytes": 5, "write_bytes": 7}}, "what_short": "x"}
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "HBM_FILE", str(f))
    assert bench.hbm_bytes_record(wl, 10, 20, "abc")["measured"]["saved"] == {"total_bytes": 2}
    assert bench.traffic_record("abc", wl.name) == {"bytes_per_launch": 12}
    off = bench.hbm_bytes_record(wl, 10, 20, "other")
    assert off["measured"] is None and "other kernel sources" in off["measured_note"]
    assert bench.traffic_record("other", wl.name) is None
    assert bench.traffic_record("abc", "8b_attn_out_mlp_in") is None
    assert bench.hbm_bytes_record(WORKLOADS["8b_attn_out_mlp_in"], 10, 20, "abc")["measured"] is None


def test_kernel_name_matching():
    """The general bf16 GEMM kernels by mode, with or without the small-row template argument; not the small-row,
    e4m3 or block-scaled instantiations."""
    f = bench._bf16_gemm_kernel
    assert f("void coda::gemm_epilogue_kernel<3, false, false, false>(void const*)", 3)
    assert f("void coda::gemm_epilogue_kernel<3, false, false>(void const*)", 3)
    assert not f("void coda::gemm_epilogue_kernel<3, false, false, true>(void const*)", 3)
    assert not f("void coda::gemm_epilogue_kernel<3, true, false, false>(void const*)", 3)
    assert not f("void coda::gemm_epilogue_kernel<3, true, true, false>(void const*)", 3)
    assert not f("void coda::gemm_epilogue_kernel<0, false, false, false>(void const*)", 3)


def _counter_dir(base, counter, value_of):
    """A counter_collection.csv as rocprofv3 writes it for one pass: two fused blocks, two unfused blocks, a copy."""
    seq = ["gemm_epilogue_kernel<0, false, false, false>", "gemm_epilogue_kernel<3, false, false, false>"] * 2 + \
          ["gemm_epilogue_kernel<1, false, false, false>", "add_rmsnorm_kernel<false>",
           "gemm_epilogue_kernel<3, false, false, false>"] * 2 + ["__amd_rocclr_copyBuffer"]
    d = base / counter
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, k in enumerate(seq):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": f"void coda::{k}(int)", "Counter_Name": counter,
                        "Counter_Value": value_of(k, i)})
    return str(d)


def test_counter_summary_attribution(tmp_path):
    """Dispatches are attributed by name and order (the GEMM2 after the first plain-store GEMM is the unfused U3),
    the first dispatch of each kernel is dropped, and the readings are scaled by the 1 GiB copy's."""
    wl = WORKLOADS["1b_attn_out_mlp_in"]
    kib = lambda x: x / 1024.0
    base = {"gemm_epilogue_kernel<0": 100, "gemm_epilogue_kernel<3": 800, "gemm_epilogue_kernel<1": 60,
            "add_rmsnorm": 50}

    def fetch(k, i):  # FETCH_SIZE reads half of the copy (128-byte requests priced at 64 bytes)
        if "copy" in k:
            return kib((1 << 30) / 2)
        v = next(b for p, b in base.items() if p in k) * 1e6
        if "<3" in k and i >= 4:
            v = 900e6  # U3 reads more than K3
        return kib(v / 2) if i not in (0, 1, 4, 5, 6) else kib(1.0)  # first dispatches carry a junk value

    def write(k, i):
        return kib(1 << 30) if "copy" in k else kib(10e6 if i not in (0, 1, 4, 5, 6) else 1.0)

    def req(k, i):
        return (1 << 30) / 128 if "copy" in k else 1.0

    dirs = [_counter_dir(tmp_path, "FETCH_SIZE", fetch), _counter_dir(tmp_path, "WRITE_SIZE", write),
            _counter_dir(tmp_path, "TCC_EA0_RDREQ_sum", req), _counter_dir(tmp_path, "TCC_EA0_WRREQ_sum", req)]
    out = tmp_path / "out.json"
    rec = bench.summarize_hbm_counters(dirs, str(out), wl)
    kern = rec["kernels"]
    assert abs(rec["calibration"]["fetch_scale"] - 2.0) < 1e-9 and abs(rec["calibration"]["write_scale"] - 1.0) < 1e-9
    assert abs(kern["K1"]["read_bytes"] - 100e6) < 2 and abs(kern["K3"]["read_bytes"] - 800e6) < 2
    assert abs(kern["U1"]["read_bytes"] - 60e6) < 2 and abs(kern["U2"]["read_bytes"] - 50e6) < 2
    assert abs(kern["U3"]["read_bytes"] - 900e6) < 2
    assert all(abs(kern[r]["write_bytes"] - 10e6) < 2 for r in kern)
    assert rec["saved"]["total_bytes"] == rec["unfused"]["total_bytes"] - rec["fused"]["total_bytes"]
    assert json.loads(out.read_text())["kernel_source_hash"] == bench.kernel_source_hash()


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2 and "one GPU" in r.stderr
