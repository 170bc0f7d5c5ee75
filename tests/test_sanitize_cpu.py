"""Address- and undefined-behaviour-sanitizer runs of the host code (CPU only, no GPU needed).

- The oracle (plain C) with tests/sanitize/oracle_driver.c, which calls every entry point on small inputs.
- The C ABI: api.hip compiled for the host only (no device code), its kernel launchers replaced by stubs generated
  here from the declarations in csrc/launch.h (each returns success and counts the call), with
  tests/sanitize/abi_driver.cpp calling every entry point with valid and invalid arguments.  The few HIP runtime
  calls the host code makes (the device number, the fixed scratch's address, error strings, the module
  registration a host-only build still emits) are stubbed as well.  Pointers are fake and never dereferenced.
Any sanitizer report aborts the driver (-fno-sanitize-recover=all), which fails the test.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
CLANG = "/opt/rocm/llvm/bin/clang++"
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout[-3000:]}\n{r.stderr[-3000:]}"
    return r


@pytest.mark.skipif(shutil.which("gcc") is None, reason="no gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-std=c11", *SAN, "-I", os.path.join(ROOT, "oracle"), "-o", exe, os.path.join(ROOT, "oracle", "oracle.c"),
          os.path.join(HERE, "oracle_driver.c"), "-lm", "-lpthread"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "all entry points ran" in r.stdout


def _stub_source(fatbin_symbol: str) -> str:
    """Definitions of every launcher declared in launch.h (returning success and counting the call), and of the HIP
    runtime entry points the host code of api.hip uses."""
    src = open(os.path.join(ROOT, "gemm_epilogue_fusion_amd", "csrc", "launch.h")).read()
    src = re.sub(r"//[^\n]*", "", src)
    out = ['#include "launch.h"', "int g_launches = 0;", "namespace coda {"]
    for ret, name, params in re.findall(r"\b(hipError_t|int|KSplit)\s+(\w+)\s*\(([^;{]*)\)\s*;", src):
        params = re.sub(r"\s*=\s*[^,]+", "", params)  # default arguments belong to the declaration only
        if name == "fold_supported":
            body = "return D / 256 <= 16;"
        elif name == "ksplit_plan":  # the split rule of a GEMM's last wave (the rules themselves are in launch.h)
            body = ("const KSplitRule& u = fp8 ? KSPLIT_E4M3 : KSPLIT_BF16; "
                    "*lg = 0; if (cus <= 0 || ntiles <= 0) return (int)ntiles; "
                    "const int64_t rem = ntiles % cus; if (rem == 0) return (int)ntiles; "
                    "if (u.tail_den * rem > cus && !(8 * rem <= 3 * cus && K >= u.long_k)) return (int)ntiles; "
                    "if (K % (2 * u.gran) || K / 2 < u.min_piece) return (int)ntiles; "
                    "int g = 1; while (g < 3 && 2 * (rem << (g + 1)) <= cus && K % ((int64_t)u.gran << (g + 1)) == 0 "
                    "&& (K >> (g + 1)) >= u.tree_piece) ++g; *lg = g; return (int)(ntiles - rem);")
        elif name == "halves_plan":  # the half-tile rule of a row-scale GEMM's last wave
            body = ("KSplit ks; if (cus <= 0 || ntiles <= 0 || M <= 64) return ks; "
                    "const int64_t rem = ntiles % cus, t = M % 256; "
                    "if (rem == 0 || 2 * rem > cus || (t != 0 && t <= 128)) return ks; "
                    "ks.full = (int)(ntiles - rem); ks.halves = 1; return ks;")
        elif name == "gemm_ksplit":  # the split rule of the weight-gradient products
            body = ("const int tiles = ((M + 255) / 256) * (N / 256); int s = 1; "
                    "while (s < 8 && tiles * s < 256 && K % (128 * s * 2) == 0) s *= 2; return s;")
        else:
            body = "++g_launches; return hipSuccess;"
        out.append(f"{ret} {name}({params}) {{ {body} }}")
    out.append("}  // namespace coda")
    out.append('extern "C" {')
    out.append("hipError_t hipGetDevice(int* d) { *d = 0; return hipSuccess; }")
    out.append("hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t, int) { *v = 256; return hipSuccess; }")
    out.append("hipError_t hipDeviceSynchronize() { return hipSuccess; }")
    out.append("hipError_t hipGetLastError() { return hipSuccess; }")
    out.append('const char* hipGetErrorString(hipError_t) { return "stub"; }')
    out.append("hipError_t hipGetSymbolAddress(void** p, const void*) { *p = (void*)((uintptr_t)3 << 44); "
               "return hipSuccess; }")
    out.append("void** __hipRegisterFatBinary(const void*) { static void* h; return &h; }")
    out.append("void __hipUnregisterFatBinary(void**) {}")
    out.append("void __hipRegisterVar(void**, void*, char*, const char*, int, size_t, int, int) {}")
    out.append(f"char {fatbin_symbol}[64];")
    out.append("}")
    return "\n".join(out) + "\n"


@pytest.mark.skipif(not os.path.exists(CLANG), reason="no ROCm clang")
def test_abi_host_code_under_sanitizers(tmp_path):
    inc = ["-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "gemm_epilogue_fusion_amd", "csrc"),
           "-I", "/opt/rocm/include"]
    host = ["-x", "hip", "--cuda-host-only", "--offload-arch=gfx950", "-std=c++17"]
    # the sanitizers apply to host code only; this build has no device code at all
    san_host = [f"-Xarch_host {f}" if f.startswith("-fsanitize") else f for f in SAN]
    san_host = [a for f in san_host for a in f.split(" ")]
    api_o = str(tmp_path / "api.o")
    _run([CLANG, *host, *san_host, *inc, "-c", "-o", api_o,
          os.path.join(ROOT, "gemm_epilogue_fusion_amd", "csrc", "api.hip")])
    syms = _run(["nm", api_o]).stdout
    fat = re.findall(r"\bU (__hip_fatbin_\w+)", syms)
    assert len(fat) == 1, syms
    stub = tmp_path / "abi_stubs.cpp"
    stub.write_text(_stub_source(fat[0]))
    exe = str(tmp_path / "abi_driver")
    _run([CLANG, "-x", "c++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", *SAN, *inc, "-c", "-o", str(tmp_path / "stubs.o"),
          str(stub)])
    _run([CLANG, "-x", "c++", "-std=c++17", *SAN, *inc, "-c", "-o", str(tmp_path / "driver.o"),
          os.path.join(HERE, "abi_driver.cpp")])
    _run([CLANG, *SAN, "-o", exe, api_o, str(tmp_path / "stubs.o"), str(tmp_path / "driver.o"), "-lpthread"])
    r = _run([exe], env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1", "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert "every status as documented" in r.stdout
