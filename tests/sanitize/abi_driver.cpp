// abi_driver.cpp -- drives the C ABI (api.hip compiled for the host only, every kernel launcher replaced by a
// stub that records the call) under the address and undefined-behaviour sanitizers (tests/test_sanitize_cpu.py).
// Test infrastructure only.  Pointers are fake, aligned and never dereferenced: the library validates them and
// hands them to the launchers.  Each call must return its documented status; a sanitizer report aborts the run.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>

#include "coda.h"

extern int g_launches;  // launcher stub calls (abi_stubs.cpp)

static int failures = 0;
#define EXPECT_EQ(a, b)                                                                              \
  do {                                                                                               \
    long long va_ = (long long)(a), vb_ = (long long)(b);                                            \
    if (va_ != vb_) {                                                                                \
      std::fprintf(stderr, "%s:%d: %s = %lld, expected %lld (%s)\n", __FILE__, __LINE__, #a, va_, vb_, \
                   coda_last_error());                                                               \
      ++failures;                                                                                    \
    }                                                                                                \
  } while (0)

static void* P(int i) { return (void*)((uintptr_t)1 << 44 | (uintptr_t)i << 36); }  // 64 GiB apart
static float* F(int i) { return (float*)P(i); }

int main() {
  const int64_t M = 300, K1 = 512, D = 512, N2 = 1024;
  size_t ws = coda_workspace_bytes(M, K1, D, N2, CODA_EPI_SWIGLU, 0, 0);
  size_t wsu = coda_workspace_bytes(M, K1, D, N2, CODA_EPI_SWIGLU, 0, 1);
  EXPECT_EQ(ws > 0 && wsu > ws, 1);
  EXPECT_EQ(coda_workspace_bytes(0, K1, D, N2, 0, 0, 0), 0);
  EXPECT_EQ(coda_workspace_bytes(M, K1, D, N2, 0, 2, 1), 0);
  EXPECT_EQ(coda_abi_version(), CODA_ABI_VERSION);
  EXPECT_EQ(coda_workspace_r_offset(M, D) < ws, 1);
  // the fused block: valid, then one bad argument at a time
  int before = g_launches;
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, P(8), ws, nullptr), 0);
  EXPECT_EQ(g_launches - before, 2);  // two kernels where D <= 4096
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), 130, 128, 4352, 256, P(8),
                           coda_workspace_bytes(130, 128, 4352, 256, 1, 0, 0), nullptr), 0);
  EXPECT_EQ(coda_block_fwd(nullptr, P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, P(8), ws, nullptr),
            CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_block_fwd((char*)P(1) + 8, P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, P(8), ws,
                           nullptr), CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), NAN, 1, P(6), P(7), M, K1, D, N2, P(8), ws, nullptr),
            CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 7, P(6), P(7), M, K1, D, N2, P(8), ws, nullptr),
            CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, 100, D, N2, P(8), ws, nullptr),
            CODA_ERR_UNSUPPORTED);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), (int64_t)1 << 40, K1, D, N2, P(8),
                           ws, nullptr), CODA_ERR_UNSUPPORTED);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, P(8), ws - 256,
                           nullptr), CODA_ERR_WORKSPACE);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(3), P(7), M, K1, D, N2, P(8), ws, nullptr), 0);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(1), M, K1, D, N2, P(8), ws, nullptr),
            CODA_ERR_ALIAS);
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), (char*)P(8) + 256, M, K1, D, N2, P(8), ws,
                           nullptr), CODA_ERR_ALIAS);
  // the unfused baseline, the e4m3 paths, RoPE
  EXPECT_EQ(coda_block_unfused(P(1), P(2), P(3), F(4), P(5), 1e-5f, 0, P(6), P(7), M, K1, D, N2, P(8), wsu, nullptr), 0);
  size_t ws8 = coda_workspace_bytes(M, K1, D, N2, 1, 1, 0), ws8u = coda_workspace_bytes(M, K1, D, N2, 1, 1, 1);
  size_t wsmx = coda_workspace_bytes(M, K1, D, N2, 1, 2, 0);
  EXPECT_EQ(coda_block_fwd_fp8(P(1), F(9), P(2), F(10), P(3), F(4), P(5), F(11), 1e-5f, 1, P(6), P(7), M, K1, D, N2,
                               P(8), ws8, nullptr), 0);
  EXPECT_EQ(coda_block_unfused_fp8(P(1), F(9), P(2), F(10), P(3), F(4), P(5), F(11), 1e-5f, 1, P(6), P(7), M, K1, D,
                                   N2, P(8), ws8u, nullptr), 0);
  EXPECT_EQ(coda_block_fwd_fp8_mx(P(1), F(9), P(2), F(10), P(3), F(4), P(5), F(11), 1e-5f, 1, P(6), P(7), M, K1, D,
                                  N2, P(8), wsmx, nullptr), 0);
  EXPECT_EQ(coda_block_fwd_fp8(P(1), nullptr, P(2), F(10), P(3), F(4), P(5), F(11), 1e-5f, 1, P(6), P(7), M, K1, D,
                               N2, P(8), ws8, nullptr), CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_block_fwd_fp8(P(1), F(9), P(2), F(10), P(3), F(4), P(5), F(11), 1e-5f, 1, P(6), P(7), M, 384, D, N2,
                               P(8), ws8, nullptr), CODA_ERR_UNSUPPORTED);
  size_t wsi = coda_workspace_bytes(M, K1, D, N2, 0, 0, 0);
  EXPECT_EQ(coda_block_fwd_rope(P(1), P(2), P(3), F(4), P(5), 1e-5f, 2048, 640, 5e5f, P(6), P(7), M, K1, D, N2, P(8),
                                wsi, nullptr), 0);
  EXPECT_EQ(coda_block_fwd_rope(P(1), P(2), P(3), F(4), P(5), 1e-5f, 2048, 600, 5e5f, P(6), P(7), M, K1, D, N2, P(8),
                                wsi, nullptr), CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_rope_rows(P(7), M, N2, 0, 64, 1e4f, nullptr), CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_rope_rows(P(7), M, N2, 16, 64, 1e4f, nullptr), 0);
  // the steps one by one
  EXPECT_EQ(coda_gemm1_residual_partial_rms(P(1), P(2), P(3), F(4), P(6), P(7), F(8), M, K1, D, nullptr), 0);
  EXPECT_EQ(coda_partial_rms_reduce(F(8), D / 256, M, D, 1e-5f, F(9), nullptr), 0);
  EXPECT_EQ(coda_partial_rms_reduce(F(8), 0, M, D, 1e-5f, F(9), nullptr), CODA_ERR_INVALID_ARG);
  EXPECT_EQ(coda_gemm2_rowscale(P(7), P(5), F(9), 1, P(10), M, D, N2, nullptr), 0);
  EXPECT_EQ(coda_gemm1_residual_partial_rms_panels(P(1), P(2), P(3), F(4), P(6), P(7), F(8), M, K1, D, nullptr), 0);
  EXPECT_EQ(coda_gemm2_rowscale_panels(P(7), P(5), F(8), 1e-5f, F(9), 1, P(10), M, D, N2, nullptr), 0);
  EXPECT_EQ(coda_gemm2_rowscale_panels(P(7), P(5), nullptr, 0.0f, F(9), 0, P(10), M, D, N2, nullptr), 0);
  // the backward
  const int64_t Mb = 1024, K1b = 256, Db = 256, N2b = 512;
  size_t wb = coda_bwd_workspace_bytes(Mb, K1b, Db, N2b, 0), wbu = coda_bwd_workspace_bytes(Mb, K1b, Db, N2b, 1);
  EXPECT_EQ(wb > 0 && wbu > wb, 1);
  EXPECT_EQ(coda_block_bwd(P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), P(9), F(10), P(11), F(12), F(13), Mb, K1b,
                           Db, N2b, P(14), wb, nullptr), 0);
  EXPECT_EQ(coda_block_bwd(P(1), P(2), P(3), F(4), F(5), P(6), P(7), nullptr, P(9), F(10), P(11), F(12), F(13), Mb,
                           K1b, Db, N2b, P(14), wb, nullptr), 0);
  EXPECT_EQ(coda_block_bwd_w2t(P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), P(9), F(10), P(11), F(12), F(13), Mb,
                               K1b, Db, N2b, P(14), wb, nullptr), 0);
  EXPECT_EQ(coda_block_bwd_unfused(P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), P(9), F(10), P(11), F(12), F(13),
                                   Mb, K1b, Db, N2b, P(14), wbu, nullptr), 0);
  EXPECT_EQ(coda_block_bwd(P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), P(9), F(10), P(11), F(12), F(13), 100,
                           K1b, Db, N2b, P(14), wb, nullptr), CODA_ERR_UNSUPPORTED);
  EXPECT_EQ(coda_block_bwd(P(1), P(2), P(3), F(4), F(5), P(6), P(7), P(8), P(1), F(10), P(11), F(12), F(13), Mb, K1b,
                           Db, N2b, P(14), wb, nullptr), CODA_ERR_ALIAS);
  // cross-entropy, the SwiGLU forward keeping z and its backward
  size_t wc = coda_ce_workspace_bytes(M, D, 2048, 0), wcu = coda_ce_workspace_bytes(M, D, 2048, 1);
  EXPECT_EQ(coda_ce_fwd(P(1), P(2), (const int32_t*)P(3), F(4), F(5), M, D, 2048, P(6), wc, nullptr), 0);
  EXPECT_EQ(coda_ce_unfused(P(1), P(2), (const int32_t*)P(3), F(4), F(5), M, D, 2048, P(6), wcu, nullptr), 0);
  EXPECT_EQ(coda_ce_fwd(P(1), P(2), (const int32_t*)P(3), F(4), F(5), M, D, 2000, P(6), wc, nullptr), CODA_ERR_UNSUPPORTED);
  EXPECT_EQ(coda_block_fwd_save_z(P(1), P(2), P(3), F(4), P(5), 1e-5f, P(6), P(7), P(9), M, K1, D, N2, P(8), ws,
                                  nullptr), 0);
  size_t wsw = coda_swiglu_bwd_workspace_bytes(M, 1024, 1);
  EXPECT_EQ(coda_swiglu_bwd(P(1), P(2), P(3), P(4), M, D, 1024, nullptr, 0, nullptr), 0);
  EXPECT_EQ(coda_swiglu_bwd_unfused(P(1), P(2), P(3), P(4), M, D, 1024, P(5), wsw, nullptr), 0);
  EXPECT_EQ(coda_swiglu_bwd_unfused(P(1), P(2), P(3), P(4), M, D, 1024, P(5), wsw - 256, nullptr), CODA_ERR_WORKSPACE);
  // the entry point on the library's fixed scratch: refused beyond it before any device call, run within it
  EXPECT_EQ(coda_block_fwd_noalloc(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), 16384, 256, 4096, 512,
                                   nullptr), CODA_ERR_WORKSPACE);
  before = g_launches;
  EXPECT_EQ(coda_block_fwd_noalloc(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, nullptr), 0);
  EXPECT_EQ(coda_block_fwd_noalloc(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), 64, 256, 256, 512, nullptr), 0);
  EXPECT_EQ(g_launches - before, 4);
  EXPECT_EQ(coda_block_fwd_noalloc(P(1), P(2), P(3), F(4), P(5), -1.0f, 1, P(6), P(7), M, K1, D, N2, nullptr),
            CODA_ERR_INVALID_ARG);
  // the debugging mode: every launch followed by a synchronisation and a check (stubbed here: it must still pass)
  setenv("CODA_SYNC_CHECK", "1", 1);
  before = g_launches;
  EXPECT_EQ(coda_block_fwd(P(1), P(2), P(3), F(4), P(5), 1e-5f, 1, P(6), P(7), M, K1, D, N2, P(8), ws, nullptr), 0);
  EXPECT_EQ(g_launches - before, 2);
  unsetenv("CODA_SYNC_CHECK");
  if (failures) std::fprintf(stderr, "%d expectation(s) failed\n", failures);
  else std::printf("abi driver: %d launcher calls, every status as documented\n", g_launches);
  return failures ? 1 : 0;
}
