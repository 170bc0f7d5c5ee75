// api.hip -- the C ABI declared in include/coda.h: argument validation, workspace layout, error reporting
// and the launch sequences of the fused block and of the unfused baseline.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstdlib>
#include <mutex>
#include <string>

#include "coda.h"
#include "launch.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return CODA_OK;
}

// CODA_SYNC_CHECK=1 in the environment (read at every launch, so a test can switch it): each launch is followed by
// a device synchronisation and an error check, so that a device-side failure is reported by the entry point and
// the launch that caused it rather than at the caller's next synchronisation.  A debugging aid: it serialises the
// caller's streams, and it cannot be used under graph capture (the synchronisation fails there).
bool sync_check() {
  const char* v = std::getenv("CODA_SYNC_CHECK");
  return v && *v && *v != '0';
}

int hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(CODA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  if (sync_check()) {
    hipError_t s = hipDeviceSynchronize();
    if (s == hipSuccess) s = hipGetLastError();
    if (s != hipSuccess) return fail(CODA_ERR_HIP, "%s (CODA_SYNC_CHECK): %s", what, hipGetErrorString(s));
  }
  return ok();
}

constexpr int64_t kMaxDim = (int64_t)1 << 30;  // keeps every row index and per-matrix element count in range

// The fused paths keep the second GEMM's A operand (h * gamma, or its e4m3 codes) in the workspace as K panels
// of the mainloop's stage width: it is private to the block, and whole-line direct loads shorten GEMM2 (see
// ALayout in gemm_core.h).  The backward keeps dh^T and n^T, the A operands of the weight-gradient products,
// the same way.  The step entry points, whose tensors the caller sees, stay row-major.
constexpr int kPanels = 1;

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

Range rng(const char* name, const void* p, size_t bytes) {
  return Range{name, (uintptr_t)p, (uintptr_t)p + bytes};
}

bool overlap(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

int check_ptr(const void* p, const char* name) {
  if (!p) return fail(CODA_ERR_INVALID_ARG, "%s is NULL", name);
  if ((uintptr_t)p & 15) return fail(CODA_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return CODA_OK;
}

// Shape rules of the GEMM tiling: row tiles are masked, column tiles and the K step are not.
int check_dims(int64_t M, int64_t K1, int64_t D, int64_t N2) {
  if (M < 1 || K1 < 1 || D < 1 || N2 < 1)
    return fail(CODA_ERR_INVALID_ARG, "dimensions must be >= 1 (M=%lld K1=%lld D=%lld N2=%lld)", (long long)M,
                (long long)K1, (long long)D, (long long)N2);
  if (M > kMaxDim || K1 > kMaxDim || D > kMaxDim || N2 > kMaxDim || M * K1 > kMaxDim * 2 ||
      M * D > kMaxDim * 2 || M * N2 > kMaxDim * 2 || D * N2 > kMaxDim * 2 || K1 * D > kMaxDim * 2)
    return fail(CODA_ERR_UNSUPPORTED, "dimensions too large");
  if (K1 % 128) return fail(CODA_ERR_UNSUPPORTED, "K1=%lld is not a multiple of 128", (long long)K1);
  if (D % 256) return fail(CODA_ERR_UNSUPPORTED, "D=%lld is not a multiple of 256", (long long)D);
  if (N2 % 256) return fail(CODA_ERR_UNSUPPORTED, "N2=%lld is not a multiple of 256", (long long)N2);
  return CODA_OK;
}

int check_epi_eps(int epi, float eps) {
  if (epi != CODA_EPI_IDENTITY && epi != CODA_EPI_SWIGLU) return fail(CODA_ERR_INVALID_ARG, "bad epi_kind %d", epi);
  if (!std::isfinite(eps) || eps < 0.0f) return fail(CODA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return CODA_OK;
}

// Outputs may not overlap inputs or each other; out_h == R (same start and size) is the one allowed alias.
int check_alias(const Range* in, int nin, const Range* out, int nout, const void* allowed_out,
                const void* allowed_in) {
  for (int o = 0; o < nout; ++o) {
    for (int i = 0; i < nin; ++i) {
      if (!overlap(out[o], in[i])) continue;
      if (out[o].lo == (uintptr_t)allowed_out && in[i].lo == (uintptr_t)allowed_in && out[o].lo == in[i].lo &&
          out[o].hi == in[i].hi)
        continue;
      return fail(CODA_ERR_ALIAS, "%s overlaps %s", out[o].name, in[i].name);
    }
    for (int p = o + 1; p < nout; ++p)
      if (overlap(out[o], out[p])) return fail(CODA_ERR_ALIAS, "%s overlaps %s", out[o].name, out[p].name);
  }
  return CODA_OK;
}

struct Workspace {
  float* part;    // [D/256][M] partial sums of squares
  float* r;       // [M] row scale
  uint16_t* hg;   // fused bf16: h * gamma [M,D] bf16, the second GEMM's A operand
  uint16_t* t;    // unfused: T = X W1 [M,D] bf16
  uint16_t* n;    // unfused bf16: normalised rows [M,D]
  uint8_t* q;     // fp8: the second GEMM's e4m3 A operand [M,D] (fused: h * gamma quantised; unfused: n quantised)
  float* qs;      // fp8: its per-row scale [M]
  float* rs2;     // fp8 fused: the second GEMM's epilogue row scale qs * r [M]
  uint8_t* mxs;   // fp8 fused, block-scaled: the block scales of q, (D/64) * ceil(M/256)*256 * 2 bytes
};

size_t ws_part_bytes(int64_t M, int64_t D) { return align256((size_t)(D / 256) * (size_t)M * 4); }
size_t ws_vec_bytes(int64_t M) { return align256((size_t)M * 4); }
size_t ws_mat_bytes(int64_t M, int64_t D, int elem) { return align256((size_t)M * (size_t)D * elem); }

// Lays the workspace out (or, with ws == nullptr, only measures it).
size_t carve(void* ws, int64_t M, int64_t D, int fp8, int unfused, Workspace* w) {
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  Workspace x{};
  x.part = (float*)take(ws_part_bytes(M, D));
  x.r = (float*)take(ws_vec_bytes(M));
  if (unfused) {
    x.t = (uint16_t*)take(ws_mat_bytes(M, D, 2));
    if (fp8) {
      x.q = (uint8_t*)take(ws_mat_bytes(M, D, 1));
      x.qs = (float*)take(ws_vec_bytes(M));
    } else {
      x.n = (uint16_t*)take(ws_mat_bytes(M, D, 2));
    }
  } else if (fp8 == 2) {  // block-scaled (MX-style) A operand of the second GEMM
    x.q = (uint8_t*)take(ws_mat_bytes(M, D, 1));
    x.mxs = (uint8_t*)take(align256((size_t)(D / 64) * (size_t)((M + 255) / 256 * 256) * 2));
  } else if (fp8) {
    x.q = (uint8_t*)take(ws_mat_bytes(M, D, 1));
    x.qs = (float*)take(ws_vec_bytes(M));
    x.rs2 = (float*)take(ws_vec_bytes(M));
  } else {
    x.hg = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  }
  if (w) *w = x;
  return off;
}

size_t ws_bytes(int64_t M, int64_t D, int fp8, int unfused) { return carve(nullptr, M, D, fp8, unfused, nullptr); }

// After those bytes the blocks keep the splits of their GEMMs' last waves of tiles (coda::KSplit): for the
// second GEMM, then for the first, the tickets (align256(tail * 4) bytes) and two accumulator slots per split tile.
// The size is planned for 256 CUs (MI355X); coda_workspace_bytes includes it, and a block splits only where the
// workspace it is given has that room (with less, from the base size on, its GEMMs run whole tiles).
constexpr int kPlanCus = 256;

int64_t gemm_tiles(int64_t M, int64_t N) { return (M + 255) / 256 * (N / 256); }

// One GEMM's split room for `ntiles` tiles over K on `cus` CUs (0: no split): per split tile S - 1 tickets and
// 2 S - 2 slots (the tree of coda::KSplit).
size_t split_bytes_one(int64_t ntiles, int64_t K, int cus, int fp8) {
  int lg = 0;
  const int64_t tail = ntiles - coda::ksplit_plan(ntiles, K, cus, fp8, &lg);
  if (tail <= 0) return 0;
  const int64_t S = (int64_t)1 << lg;
  return align256((size_t)(tail * (S - 1)) * 4) + (size_t)(tail * (2 * S - 2)) * coda::KSPLIT_SLOT_FLOATS * 4;
}

size_t ws_split_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int fp8, int cus) {
  if (M < 1 || D < 256 || N2 < 256) return 0;
  return split_bytes_one(gemm_tiles(M, N2), D, cus, fp8) + split_bytes_one(gemm_tiles(M, D), K1, cus, fp8);
}

// The split room a block validated with `workspace_bytes` may use: the planned region when it fits, else none.
size_t ws_split_room(int64_t M, int64_t K1, int64_t D, int64_t N2, int fp8, int unfused, size_t workspace_bytes) {
  const size_t base = ws_bytes(M, D, fp8, unfused);
  const size_t b = ws_split_bytes(M, K1, D, N2, fp8, kPlanCus);
  return (b && workspace_bytes >= base + b) ? b : 0;
}

// CU count of the current device (cached per device; 0 when it cannot be read).
int device_cus() {
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kDevs) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = -1;
    cache[dev].store(v, std::memory_order_relaxed);
    c = v;
  }
  return c > 0 ? c : 0;
}

// One GEMM's split laid out from `at` (which then moves past it); no split where the plan has none.
coda::KSplit split_one(char*& at, int64_t ntiles, int64_t K, int cus, int fp8, int* tickets) {
  coda::KSplit ks;
  int lg = 0;
  const int64_t full = coda::ksplit_plan(ntiles, K, cus, fp8, &lg);
  *tickets = 0;
  if (full >= ntiles) return ks;
  const int64_t tail = ntiles - full, S = (int64_t)1 << lg;
  ks.full = (int)full;
  ks.lg = lg;
  ks.cnt = (int*)at;
  ks.part = (float*)(at + align256((size_t)(tail * (S - 1)) * 4));
  at += split_bytes_one(ntiles, K, cus, fp8);
  *tickets = (int)(tail * (S - 1));
  return ks;
}

// The splits a block's GEMMs run with on this device, inside the validated room (none if they do not fit), and the
// half-tile form of the second GEMM's last wave where it is not split (bf16; needs no room): g1 for
// the first GEMM (K1 or U1, over K1), g2 for the second (K3 or U3, over D).  g1 carries g2's tickets to clear.
struct SplitPlan {
  coda::KSplit g1, g2;
  int tickets1 = 0;  // the first GEMM's tickets, cleared before it runs
};

SplitPlan split_plan(void* ws, int64_t M, int64_t K1, int64_t D, int64_t N2, int fp8, int unfused, size_t room) {
  SplitPlan p;
  const int cus = device_cus();
  const size_t need = room ? ws_split_bytes(M, K1, D, N2, fp8, cus) : 0;
  if (need && need <= room) {
    char* at = (char*)ws + ws_bytes(M, D, fp8, unfused);
    int tickets2 = 0;
    p.g2 = split_one(at, gemm_tiles(M, N2), D, cus, fp8, &tickets2);
    p.g1 = split_one(at, gemm_tiles(M, D), K1, cus, fp8, &p.tickets1);
    if (p.g2.full >= 0) {
      p.g1.clear = p.g2.cnt;
      p.g1.nclear = tickets2;
    }
  }
  // bf16: where the second GEMM's last wave is not split along K, its tiles may run as 128-row halves (no room needed)
  if (p.g2.full < 0 && !fp8) p.g2 = coda::halves_plan(gemm_tiles(M, N2), M, cus);
  return p;
}

// Validation shared by the block entry points.  fp8: X, W1, W2 are e4m3 bytes and sx, sw1, sw2 their
// scales (ignored, and may be NULL, for bf16).
int validate_block(const void* X, const float* sx, const void* W1, const float* sw1, const void* R,
                   const float* gamma, const void* W2, const float* sw2, float eps, int epi, void* out_h, void* out_y,
                   int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace, size_t workspace_bytes, int fp8,
                   int unfused) {
  int s;
  if ((s = check_ptr(X, "X")) || (s = check_ptr(W1, "W1")) || (s = check_ptr(R, "R")) ||
      (s = check_ptr(gamma, "gamma")) || (s = check_ptr(W2, "W2")) || (s = check_ptr(out_h, "out_h")) ||
      (s = check_ptr(out_y, "out_y")))
    return s;
  if (fp8 && ((s = check_ptr(sx, "sx")) || (s = check_ptr(sw1, "sw1")) || (s = check_ptr(sw2, "sw2")))) return s;
  if ((s = check_dims(M, K1, D, N2))) return s;
  if (fp8 && K1 % 256) return fail(CODA_ERR_UNSUPPORTED, "fp8: K1=%lld is not a multiple of 256", (long long)K1);
  if ((s = check_epi_eps(epi, eps))) return s;
  if (unfused && D > 8192) return fail(CODA_ERR_UNSUPPORTED, "unfused path supports D <= 8192");
  const size_t need = ws_bytes(M, D, fp8, unfused);
  if (!workspace) return fail(CODA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)workspace & 255) return fail(CODA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(CODA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const int64_t ny = epi == CODA_EPI_SWIGLU ? N2 / 2 : N2;
  const size_t el = fp8 ? 1 : 2;
  const Range in[8] = {rng("X", X, (size_t)(M * K1) * el), rng("W1", W1, (size_t)(K1 * D) * el),
                       rng("R", R, (size_t)(M * D * 2)), rng("gamma", gamma, (size_t)D * 4),
                       rng("W2", W2, (size_t)(D * N2) * el), rng("sx", sx, fp8 ? (size_t)M * 4 : 0),
                       rng("sw1", sw1, fp8 ? (size_t)D * 4 : 0), rng("sw2", sw2, fp8 ? (size_t)N2 * 4 : 0)};
  const Range out[3] = {rng("out_h", out_h, (size_t)(M * D * 2)), rng("out_y", out_y, (size_t)(M * ny * 2)),
                        rng("workspace", workspace, need + ws_split_room(M, K1, D, N2, fp8, unfused, workspace_bytes))};
  return check_alias(in, 8, out, 3, out_h, R);
}

int check_rope(int64_t N, int64_t seq_len, int64_t n_rot, float base) {
  if (seq_len < 1 || seq_len > kMaxDim) return fail(CODA_ERR_INVALID_ARG, "seq_len must be >= 1");
  if (n_rot < 0 || n_rot > N || n_rot % 64)
    return fail(CODA_ERR_INVALID_ARG, "n_rope_cols=%lld must be a multiple of 64 in [0, %lld]", (long long)n_rot,
                (long long)N);
  if (!std::isfinite(base) || !(base > 0.0f)) return fail(CODA_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  return CODA_OK;
}

// ---- backward ----
struct BwdWorkspace {
  uint16_t* G;    // r gamma P [M,D] bf16 (unfused: after P itself)
  float* part;    // row partials [D/256][M]
  float* part2;   // column partials [ceil(M/256)][D]
  float* a;       // [M]
  uint16_t* dhT;  // dh^T, M * D bf16 in K panels over M ([M/32][D][32])
  uint16_t* nT;   // n^T, same layout
  uint16_t* P;    // unfused: P = dz W2^T [M,D] bf16
  float* slabs;   // split-K partial products of dW1 and dW2 (whichever needs more)
  uint16_t* W2T;  // W2^T [N2,D] bf16 for the first product; shares its bytes with slabs (used later in the stream)
};

size_t carve_bwd(void* ws, int64_t M, int64_t K1, int64_t D, int64_t N2, int unfused, BwdWorkspace* w) {
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  BwdWorkspace x{};
  x.G = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  x.part = (float*)take(ws_part_bytes(M, D));
  x.part2 = (float*)take(align256((size_t)((M + 255) / 256) * (size_t)D * 4));
  x.a = (float*)take(ws_vec_bytes(M));
  x.dhT = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  x.nT = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  if (unfused) x.P = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  // dW1 = (dh^T X)^T: a [D,K1] product over K = M; dW2 = n^T dz: a [D,N2] product over K = M
  const int s1 = coda::gemm_ksplit((int)D, (int)K1, (int)M), s2 = coda::gemm_ksplit((int)D, (int)N2, (int)M);
  const size_t b1 = s1 > 1 ? (size_t)s1 * (size_t)D * (size_t)K1 * 4 : 0;
  const size_t b2 = s2 > 1 ? (size_t)s2 * (size_t)D * (size_t)N2 * 4 : 0;
  const size_t bt = (size_t)D * (size_t)N2 * 2;
  size_t region = b1 > b2 ? b1 : b2;
  region = region > bt ? region : bt;
  char* shared = take(align256(region));
  x.slabs = (float*)shared;
  x.W2T = (uint16_t*)shared;
  if (w) *w = x;
  return off;
}

int validate_bwd(const void* X, const void* W1, const void* h, const float* r, const float* gamma, const void* W2,
                 const void* dz, const void* dh_out, void* dX, float* dW1, void* dR, float* dgamma, float* dW2,
                 int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace, size_t workspace_bytes, int unfused) {
  int s;
  if ((s = check_ptr(X, "X")) || (s = check_ptr(W1, "W1")) || (s = check_ptr(h, "h")) || (s = check_ptr(r, "r")) ||
      (s = check_ptr(gamma, "gamma")) || (s = check_ptr(W2, "W2")) || (s = check_ptr(dz, "dz")) ||
      (s = check_ptr(dX, "out_dX")) || (s = check_ptr(dW1, "out_dW1")) || (s = check_ptr(dR, "out_dR")) ||
      (s = check_ptr(dgamma, "out_dgamma")) || (s = check_ptr(dW2, "out_dW2")))
    return s;
  if (dh_out && (s = check_ptr(dh_out, "dh_out"))) return s;
  if ((s = check_dims(M, K1, D, N2))) return s;
  if (M % 128) return fail(CODA_ERR_UNSUPPORTED, "backward: M=%lld is not a multiple of 128", (long long)M);
  if (K1 % 256) return fail(CODA_ERR_UNSUPPORTED, "backward: K1=%lld is not a multiple of 256", (long long)K1);
  const size_t need = carve_bwd(nullptr, M, K1, D, N2, unfused, nullptr);
  if (!workspace) return fail(CODA_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((uintptr_t)workspace & 255) return fail(CODA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (workspace_bytes < need)
    return fail(CODA_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  const Range in[8] = {rng("X", X, (size_t)(M * K1) * 2), rng("W1", W1, (size_t)(K1 * D) * 2),
                       rng("h", h, (size_t)(M * D) * 2),  rng("r", r, (size_t)M * 4),
                       rng("gamma", gamma, (size_t)D * 4), rng("W2", W2, (size_t)(D * N2) * 2),
                       rng("dz", dz, (size_t)(M * N2) * 2), rng("dh_out", dh_out, dh_out ? (size_t)(M * D) * 2 : 0)};
  const Range out[6] = {rng("out_dX", dX, (size_t)(M * K1) * 2),     rng("out_dW1", dW1, (size_t)(K1 * D) * 4),
                        rng("out_dR", dR, (size_t)(M * D) * 2),      rng("out_dgamma", dgamma, (size_t)D * 4),
                        rng("out_dW2", dW2, (size_t)(D * N2) * 4),   rng("workspace", workspace, need)};
  return check_alias(in, 8, out, 6, nullptr, nullptr);
}

// The fused block's launch sequence on an accepted argument set: coda_block_fwd on the caller's workspace,
// coda_block_fwd_noalloc on the library's scratch.
int launch_block_fwd(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                     int epi_kind, void* out_h, void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2,
                     void* workspace, size_t workspace_bytes, hipStream_t st, void* out_z = nullptr) {
  int s;
  Workspace w;
  carve(workspace, M, D, 0, 0, &w);
  const SplitPlan sp = split_plan(workspace, M, K1, D, N2, 0, 0, ws_split_room(M, K1, D, N2, 0, 0, workspace_bytes));
  if (sp.tickets1 && (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
    return s;
  if ((s = hip_check(coda::launch_gemm1_res_prms((const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)R, gamma,
                                                 (uint16_t*)out_h, w.hg, w.part, (int)M, (int)K1, (int)D, st, kPanels,
                                                 sp.g1),
                     "gemm1_res_prms launch")))
    return s;
  const coda::KSplit& ks = sp.g2;
  if (coda::fold_supported((int)D))  // the reduce runs inside K3's workgroups
    return hip_check(coda::launch_gemm2_rowscale_fold(w.hg, (const uint16_t*)W2, w.part, eps, w.r,
                                                      epi_kind == CODA_EPI_SWIGLU, (uint16_t*)out_y, (int)M, (int)D,
                                                      (int)N2, st, (uint16_t*)out_z, kPanels, ks),
                     "gemm2_rowscale_fold launch");
  if ((s = hip_check(coda::launch_prms_reduce(w.part, (int)(D / 256), (int)M, (int)D, eps, w.r, st),
                     "prms_reduce launch")))
    return s;
  return hip_check(coda::launch_gemm2_rowscale(w.hg, (const uint16_t*)W2, w.r, epi_kind == CODA_EPI_SWIGLU,
                                               (uint16_t*)out_y, (int)M, (int)D, (int)N2, st, (uint16_t*)out_z,
                                               kPanels, ks),
                   "gemm2_rowscale launch");
}

}  // namespace

// The fixed scratch of coda_block_fwd_noalloc: the fused block's workspace (partial sums, r, h * gamma in K panels)
// for callers that cannot allocate.  Each device the library runs on holds its own copy from the moment the
// library's code is loaded there until the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once per device (noalloc_scratch below), and
// only that address is ever passed to a kernel.
__device__ __align__(256) unsigned char scratch[CODA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of `scratch` on the current device, looked up on the first call on that device.
int noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(CODA_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(CODA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(CODA_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CODA_OK;
}

}  // namespace

extern "C" {

int coda_abi_version(void) { return CODA_ABI_VERSION; }

const char* coda_status_string(int status) {
  switch (status) {
    case CODA_OK: return "CODA_OK";
    case CODA_ERR_INVALID_ARG: return "CODA_ERR_INVALID_ARG";
    case CODA_ERR_UNSUPPORTED: return "CODA_ERR_UNSUPPORTED";
    case CODA_ERR_ALIAS: return "CODA_ERR_ALIAS";
    case CODA_ERR_WORKSPACE: return "CODA_ERR_WORKSPACE";
    case CODA_ERR_HIP: return "CODA_ERR_HIP";
    case CODA_ERR_INTERNAL: return "CODA_ERR_INTERNAL";
    default: return "CODA_ERR_UNKNOWN";
  }
}

const char* coda_last_error(void) { return g_last_error.c_str(); }

size_t coda_workspace_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int epi_kind, int fp8, int unfused) {
  (void)epi_kind;
  if (M < 1 || D < 256 || M > kMaxDim || D > kMaxDim || fp8 < 0 || fp8 > 2 || (fp8 == 2 && unfused)) return 0;
  // the split room (N2 outside the shape rules: none)
  const size_t split = (N2 >= 256 && N2 <= kMaxDim && N2 % 256 == 0 && K1 >= 1 && K1 <= kMaxDim)
                           ? ws_split_bytes(M, K1, D, N2, fp8, kPlanCus)
                           : 0;
  return ws_bytes(M, D, fp8, unfused ? 1 : 0) + split;
}

size_t coda_workspace_split_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int epi_kind, int fp8, int unfused) {
  if (coda_workspace_bytes(M, K1, D, N2, epi_kind, fp8, unfused) == 0) return 0;
  if (N2 < 256 || N2 > kMaxDim || N2 % 256 || K1 < 1 || K1 > kMaxDim) return 0;
  return ws_split_bytes(M, K1, D, N2, fp8, kPlanCus);
}

size_t coda_workspace_r_offset(int64_t M, int64_t D) { return ws_part_bytes(M, D); }

int coda_block_fwd(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                   int epi_kind, void* out_h, void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2,
                   void* workspace, size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(X, nullptr, W1, nullptr, R, gamma, W2, nullptr, eps, epi_kind, out_h, out_y, M, K1, D, N2,
                           workspace, workspace_bytes, 0, 0);
    if (s) return s;
    return launch_block_fwd(X, W1, R, gamma, W2, eps, epi_kind, out_h, out_y, M, K1, D, N2, workspace,
                            workspace_bytes, (hipStream_t)stream);
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_fwd_noalloc(const void* X, const void* W1, const void* R, const float* gamma, const void* W2,
                           float eps, int epi_kind, void* out_h, void* out_y, int64_t M, int64_t K1, int64_t D,
                           int64_t N2, void* stream) {
  try {
    // the size limit first (plain arithmetic: nothing touches the device before the arguments are accepted)
    if (M >= 1 && D >= 256 && M <= kMaxDim && D <= kMaxDim && ws_bytes(M, D, 0, 0) > (size_t)CODA_NOALLOC_SCRATCH_BYTES)
      return fail(CODA_ERR_WORKSPACE,
                  "coda_block_fwd_noalloc: M=%lld, D=%lld need %zu bytes of scratch; the library's fixed scratch holds "
                  "%zu (use coda_block_fwd with a workspace)",
                  (long long)M, (long long)D, ws_bytes(M, D, 0, 0), (size_t)CODA_NOALLOC_SCRATCH_BYTES);
    void* ws = nullptr;
    int s = noalloc_scratch(&ws);
    if (s) return s;
    s = validate_block(X, nullptr, W1, nullptr, R, gamma, W2, nullptr, eps, epi_kind, out_h, out_y, M, K1, D, N2, ws,
                       (size_t)CODA_NOALLOC_SCRATCH_BYTES, 0, 0);
    if (s) return s;
    return launch_block_fwd(X, W1, R, gamma, W2, eps, epi_kind, out_h, out_y, M, K1, D, N2, ws,
                            (size_t)CODA_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_fwd_rope(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                        int64_t seq_len, int64_t n_rope_cols, float rope_base, void* out_h, void* out_y, int64_t M,
                        int64_t K1, int64_t D, int64_t N2, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(X, nullptr, W1, nullptr, R, gamma, W2, nullptr, eps, CODA_EPI_IDENTITY, out_h, out_y, M,
                           K1, D, N2, workspace, workspace_bytes, 0, 0);
    if (s) return s;
    if ((s = check_rope(N2, seq_len, n_rope_cols, rope_base))) return s;
    hipStream_t st = (hipStream_t)stream;
    Workspace w;
    carve(workspace, M, D, 0, 0, &w);
    const SplitPlan sp =
        split_plan(workspace, M, K1, D, N2, 0, 0, ws_split_room(M, K1, D, N2, 0, 0, workspace_bytes));
    if (sp.tickets1 &&
        (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm1_res_prms((const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)R,
                                                   gamma, (uint16_t*)out_h, w.hg, w.part, (int)M, (int)K1, (int)D,
                                                   st, kPanels, sp.g1),
                       "gemm1_res_prms launch")))
      return s;
    const coda::KSplit& ks = sp.g2;
    if (coda::fold_supported((int)D))
      return hip_check(coda::launch_gemm2_rowscale_rope_fold(w.hg, (const uint16_t*)W2, w.part, eps, w.r,
                                                             (int)seq_len, (int)n_rope_cols, rope_base,
                                                             (uint16_t*)out_y, (int)M, (int)D, (int)N2, st,
                                                             kPanels, ks),
                       "gemm2_rowscale_rope_fold launch");
    if ((s = hip_check(coda::launch_prms_reduce(w.part, (int)(D / 256), (int)M, (int)D, eps, w.r, st),
                       "prms_reduce launch")))
      return s;
    return hip_check(coda::launch_gemm2_rowscale_rope(w.hg, (const uint16_t*)W2, w.r, (int)seq_len, (int)n_rope_cols,
                                                      rope_base, (uint16_t*)out_y, (int)M, (int)D, (int)N2, st,
                                                      kPanels, ks),
                     "gemm2_rowscale_rope launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_rope_rows(void* y, int64_t M, int64_t N, int64_t seq_len, int64_t n_rope_cols, float rope_base,
                   void* stream) {
  try {
    int s;
    if ((s = check_ptr(y, "y"))) return s;
    if (M < 1 || N < 1 || M > kMaxDim || N > kMaxDim || M * N > kMaxDim * 2)
      return fail(CODA_ERR_INVALID_ARG, "bad dimensions M=%lld N=%lld", (long long)M, (long long)N);
    if ((s = check_rope(N, seq_len, n_rope_cols, rope_base))) return s;
    return hip_check(coda::launch_rope_rows((uint16_t*)y, (int)M, (int)N, (int)seq_len, (int)n_rope_cols, rope_base,
                                            (hipStream_t)stream),
                     "rope_rows launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_unfused(const void* X, const void* W1, const void* R, const float* gamma, const void* W2,
                       float eps, int epi_kind, void* out_h, void* out_y, int64_t M, int64_t K1, int64_t D,
                       int64_t N2, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(X, nullptr, W1, nullptr, R, gamma, W2, nullptr, eps, epi_kind, out_h, out_y, M, K1, D, N2,
                           workspace, workspace_bytes, 0, 1);
    if (s) return s;
    hipStream_t st = (hipStream_t)stream;
    Workspace w;
    carve(workspace, M, D, 0, 1, &w);
    // the same splits of the GEMMs' last waves as the fused block (the same kernel family on the same tiles)
    const SplitPlan sp =
        split_plan(workspace, M, K1, D, N2, 0, 1, ws_split_room(M, K1, D, N2, 0, 1, workspace_bytes));
    if (sp.tickets1 &&
        (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm_store((const uint16_t*)X, (const uint16_t*)W1, w.t, (int)M, (int)K1,
                                               (int)D, st, 0, sp.g1),
                       "gemm_store launch")))
      return s;
    const coda::KSplit& ks = sp.g2;
    if ((s = hip_check(coda::launch_add_rmsnorm(w.t, (const uint16_t*)R, gamma, (uint16_t*)out_h, w.n, w.r,
                                                (int)M, (int)D, eps, st),
                       "add_rmsnorm launch")))
      return s;
    return hip_check(coda::launch_gemm2_rowscale(w.n, (const uint16_t*)W2, nullptr, epi_kind == CODA_EPI_SWIGLU,
                                                 (uint16_t*)out_y, (int)M, (int)D, (int)N2, st, nullptr, 0, ks),
                     "unfused gemm2 launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_fwd_fp8(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                       const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                       void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                       size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, M, K1, D, N2, workspace,
                           workspace_bytes, 1, 0);
    if (s) return s;
    hipStream_t st = (hipStream_t)stream;
    Workspace w;
    carve(workspace, M, D, 1, 0, &w);
    const SplitPlan sp =
        split_plan(workspace, M, K1, D, N2, 1, 0, ws_split_room(M, K1, D, N2, 1, 0, workspace_bytes));
    if (sp.tickets1 &&
        (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm1_res_prms_fp8((const uint8_t*)Xq, sx, (const uint8_t*)W1q, sw1,
                                                       (const uint16_t*)R, (uint16_t*)out_h, w.part, (int)M,
                                                       (int)K1, (int)D, st, sp.g1),
                       "fp8 gemm1_res_prms launch")))
      return s;
    if ((s = hip_check(coda::launch_prms_reduce_quant(w.part, (int)(D / 256), (int)M, (int)D, eps,
                                                      (const uint16_t*)out_h, gamma, w.q, w.r, w.qs, w.rs2, st,
                                                      kPanels),
                       "prms_reduce_quant launch")))
      return s;
    return hip_check(coda::launch_gemm2_rowscale_fp8(w.q, (const uint8_t*)W2q, w.rs2, sw2, epi_kind == CODA_EPI_SWIGLU,
                                                     (uint16_t*)out_y, (int)M, (int)D, (int)N2, st, kPanels, sp.g2),
                     "fp8 gemm2_rowscale launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_fwd_fp8_mx(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                          const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                          void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                          size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, M, K1, D, N2, workspace,
                           workspace_bytes, 2, 0);
    if (s) return s;
    hipStream_t st = (hipStream_t)stream;
    Workspace w;
    carve(workspace, M, D, 2, 0, &w);
    const SplitPlan sp =
        split_plan(workspace, M, K1, D, N2, 2, 0, ws_split_room(M, K1, D, N2, 2, 0, workspace_bytes));
    if (sp.tickets1 &&
        (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm1_res_prms_fp8_mx((const uint8_t*)Xq, sx, (const uint8_t*)W1q, sw1,
                                                          (const uint16_t*)R, gamma, (uint16_t*)out_h, w.q, w.mxs,
                                                          w.part, (int)M, (int)K1, (int)D, st, kPanels, sp.g1),
                       "fp8 block-scaled gemm1_res_prms launch")))
      return s;
    const bool fold = coda::fold_supported((int)D);
    if (!fold && (s = hip_check(coda::launch_prms_reduce(w.part, (int)(D / 256), (int)M, (int)D, eps, w.r, st),
                                "prms_reduce launch")))
      return s;
    return hip_check(coda::launch_gemm2_rowscale_fp8_mx(w.q, w.mxs, (const uint8_t*)W2q, sw2, w.r,
                                                        fold ? w.part : nullptr, eps, w.r,
                                                        epi_kind == CODA_EPI_SWIGLU, (uint16_t*)out_y, (int)M,
                                                        (int)D, (int)N2, st, kPanels, sp.g2),
                     "fp8 block-scaled gemm2_rowscale launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_unfused_fp8(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                           const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                           void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                           size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(Xq, sx, W1q, sw1, R, gamma, W2q, sw2, eps, epi_kind, out_h, out_y, M, K1, D, N2, workspace,
                           workspace_bytes, 1, 1);
    if (s) return s;
    hipStream_t st = (hipStream_t)stream;
    Workspace w;
    carve(workspace, M, D, 1, 1, &w);
    const SplitPlan sp =
        split_plan(workspace, M, K1, D, N2, 1, 1, ws_split_room(M, K1, D, N2, 1, 1, workspace_bytes));
    if (sp.tickets1 &&
        (s = hip_check(coda::launch_clear_tickets(sp.g1.cnt, sp.tickets1, st), "clear_tickets launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm_store_fp8((const uint8_t*)Xq, sx, (const uint8_t*)W1q, sw1, w.t, (int)M,
                                                   (int)K1, (int)D, st, sp.g1),
                       "fp8 gemm_store launch")))
      return s;
    if ((s = hip_check(coda::launch_add_rmsnorm_quant(w.t, (const uint16_t*)R, gamma, (uint16_t*)out_h, w.q, w.r, w.qs,
                                                      (int)M, (int)D, eps, st),
                       "add_rmsnorm_quant launch")))
      return s;
    return hip_check(coda::launch_gemm2_rowscale_fp8(w.q, (const uint8_t*)W2q, w.qs, sw2, epi_kind == CODA_EPI_SWIGLU,
                                                     (uint16_t*)out_y, (int)M, (int)D, (int)N2, st, 0, sp.g2),
                     "unfused fp8 gemm2 launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_gemm1_residual_partial_rms(const void* X, const void* W1, const void* R, const float* gamma, void* out_h,
                                    void* out_hg, float* part, int64_t M, int64_t K1, int64_t D, void* stream) {
  try {
    int s;
    if ((s = check_ptr(X, "X")) || (s = check_ptr(W1, "W1")) || (s = check_ptr(R, "R")) ||
        (s = check_ptr(gamma, "gamma")) || (s = check_ptr(out_h, "out_h")) || (s = check_ptr(out_hg, "out_hg")) ||
        (s = check_ptr(part, "part")))
      return s;
    if ((s = check_dims(M, K1, D, 256))) return s;
    const Range in[4] = {rng("X", X, (size_t)(M * K1 * 2)), rng("W1", W1, (size_t)(K1 * D * 2)),
                         rng("R", R, (size_t)(M * D * 2)), rng("gamma", gamma, (size_t)D * 4)};
    const Range out[3] = {rng("out_h", out_h, (size_t)(M * D * 2)), rng("out_hg", out_hg, (size_t)(M * D * 2)),
                          rng("part", part, (size_t)(D / 256 * M * 4))};
    if ((s = check_alias(in, 4, out, 3, out_h, R))) return s;
    return hip_check(coda::launch_gemm1_res_prms((const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)R, gamma,
                                                 (uint16_t*)out_h, (uint16_t*)out_hg, part, (int)M, (int)K1, (int)D,
                                                 (hipStream_t)stream),
                     "gemm1_res_prms launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_partial_rms_reduce(const float* part, int64_t T, int64_t M, int64_t D, float eps, float* r,
                            void* stream) {
  try {
    int s;
    if ((s = check_ptr(part, "part")) || (s = check_ptr(r, "r"))) return s;
    if (T < 1 || M < 1 || D < 1 || T > kMaxDim || M > kMaxDim || T * M > kMaxDim * 2)
      return fail(CODA_ERR_INVALID_ARG, "bad T/M/D");
    if ((s = check_epi_eps(CODA_EPI_IDENTITY, eps))) return s;
    const Range in[1] = {rng("part", part, (size_t)(T * M * 4))};
    const Range out[1] = {rng("r", r, (size_t)M * 4)};
    if ((s = check_alias(in, 1, out, 1, nullptr, nullptr))) return s;
    return hip_check(coda::launch_prms_reduce(part, (int)T, (int)M, (int)D, eps, r, (hipStream_t)stream),
                     "prms_reduce launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_gemm2_rowscale(const void* hg, const void* W2, const float* r, int epi_kind, void* out_y, int64_t M,
                        int64_t D, int64_t N2, void* stream) {
  try {
    int s;
    if ((s = check_ptr(hg, "hg")) || (s = check_ptr(W2, "W2")) || (s = check_ptr(r, "r")) ||
        (s = check_ptr(out_y, "out_y")))
      return s;
    if ((s = check_dims(M, 128, D, N2))) return s;
    if ((s = check_epi_eps(epi_kind, 0.0f))) return s;
    const int64_t ny = epi_kind == CODA_EPI_SWIGLU ? N2 / 2 : N2;
    const Range in[3] = {rng("hg", hg, (size_t)(M * D * 2)), rng("W2", W2, (size_t)(D * N2 * 2)),
                         rng("r", r, (size_t)M * 4)};
    const Range out[1] = {rng("out_y", out_y, (size_t)(M * ny * 2))};
    if ((s = check_alias(in, 3, out, 1, nullptr, nullptr))) return s;
    return hip_check(coda::launch_gemm2_rowscale((const uint16_t*)hg, (const uint16_t*)W2, r,
                                                 epi_kind == CODA_EPI_SWIGLU, (uint16_t*)out_y, (int)M, (int)D,
                                                 (int)N2, (hipStream_t)stream),
                     "gemm2_rowscale launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_gemm1_residual_partial_rms_panels(const void* X, const void* W1, const void* R, const float* gamma,
                                           void* out_h, void* out_hg, float* part, int64_t M, int64_t K1, int64_t D,
                                           void* stream) {
  try {
    int s;
    if ((s = check_ptr(X, "X")) || (s = check_ptr(W1, "W1")) || (s = check_ptr(R, "R")) ||
        (s = check_ptr(gamma, "gamma")) || (s = check_ptr(out_h, "out_h")) || (s = check_ptr(out_hg, "out_hg")) ||
        (s = check_ptr(part, "part")))
      return s;
    if ((s = check_dims(M, K1, D, 256))) return s;
    const Range in[4] = {rng("X", X, (size_t)(M * K1 * 2)), rng("W1", W1, (size_t)(K1 * D * 2)),
                         rng("R", R, (size_t)(M * D * 2)), rng("gamma", gamma, (size_t)D * 4)};
    const Range out[3] = {rng("out_h", out_h, (size_t)(M * D * 2)), rng("out_hg", out_hg, (size_t)(M * D * 2)),
                          rng("part", part, (size_t)(D / 256 * M * 4))};
    if ((s = check_alias(in, 4, out, 3, out_h, R))) return s;
    return hip_check(coda::launch_gemm1_res_prms((const uint16_t*)X, (const uint16_t*)W1, (const uint16_t*)R, gamma,
                                                 (uint16_t*)out_h, (uint16_t*)out_hg, part, (int)M, (int)K1, (int)D,
                                                 (hipStream_t)stream, kPanels),
                     "gemm1_res_prms launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_gemm2_rowscale_panels(const void* hg, const void* W2, const float* part, float eps, float* r, int epi_kind,
                               void* out_y, int64_t M, int64_t D, int64_t N2, void* stream) {
  try {
    int s;
    if ((s = check_ptr(hg, "hg")) || (s = check_ptr(W2, "W2")) || (s = check_ptr(r, "r")) ||
        (s = check_ptr(out_y, "out_y")))
      return s;
    if (part && (s = check_ptr(part, "part"))) return s;
    if ((s = check_dims(M, 128, D, N2))) return s;
    if ((s = check_epi_eps(epi_kind, part ? eps : 0.0f))) return s;
    if (part && !coda::fold_supported((int)D))
      return fail(CODA_ERR_UNSUPPORTED, "the folded reduce takes D <= 4096 (D = %lld)", (long long)D);
    const int64_t ny = epi_kind == CODA_EPI_SWIGLU ? N2 / 2 : N2;
    const bool sw = epi_kind == CODA_EPI_SWIGLU;
    const hipStream_t st = (hipStream_t)stream;
    if (part) {
      const Range in[3] = {rng("hg", hg, (size_t)(M * D * 2)), rng("W2", W2, (size_t)(D * N2 * 2)),
                           rng("part", part, (size_t)(D / 256 * M * 4))};
      const Range out[2] = {rng("out_y", out_y, (size_t)(M * ny * 2)), rng("r", r, (size_t)M * 4)};
      if ((s = check_alias(in, 3, out, 2, nullptr, nullptr))) return s;
      return hip_check(coda::launch_gemm2_rowscale_fold((const uint16_t*)hg, (const uint16_t*)W2, part, eps, r, sw,
                                                        (uint16_t*)out_y, (int)M, (int)D, (int)N2, st, nullptr,
                                                        kPanels),
                       "gemm2_rowscale_fold launch");
    }
    const Range in[3] = {rng("hg", hg, (size_t)(M * D * 2)), rng("W2", W2, (size_t)(D * N2 * 2)),
                         rng("r", r, (size_t)M * 4)};
    const Range out[1] = {rng("out_y", out_y, (size_t)(M * ny * 2))};
    if ((s = check_alias(in, 3, out, 1, nullptr, nullptr))) return s;
    return hip_check(coda::launch_gemm2_rowscale((const uint16_t*)hg, (const uint16_t*)W2, r, sw, (uint16_t*)out_y,
                                                 (int)M, (int)D, (int)N2, st, nullptr, kPanels),
                     "gemm2_rowscale launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

}  // extern "C"

extern "C" {

size_t coda_bwd_workspace_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int unfused) {
  if (M < 1 || K1 < 1 || D < 1 || N2 < 1 || M > kMaxDim || K1 > kMaxDim || D > kMaxDim || N2 > kMaxDim) return 0;
  return carve_bwd(nullptr, M, K1, D, N2, unfused ? 1 : 0, nullptr);
}

static int block_bwd(const void* X, const void* W1, const void* h, const float* r, const float* gamma, const void* W2,
                     const void* dz, const void* dh_out, void* out_dX, float* out_dW1, void* out_dR,
                     float* out_dgamma, float* out_dW2, int64_t M, int64_t K1, int64_t D, int64_t N2,
                     void* workspace, size_t workspace_bytes, void* stream, int unfused, int w2_transposed = 0) {
  try {
    // w2_transposed: the caller passes W2^T [N2,D] in W2's place (same size, same checks) and B0 is skipped
    int s = validate_bwd(X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, M, K1, D,
                         N2, workspace, workspace_bytes, unfused);
    if (s) return s;
    hipStream_t st = (hipStream_t)stream;
    BwdWorkspace w;
    carve_bwd(workspace, M, K1, D, N2, unfused, &w);
    const uint16_t* hh = (const uint16_t*)h;
    // the first product reads W2 K-major: transpose it once (a [D,N2] -> [N2,D] pass, HBM-bound) so that the
    // product runs on the NN mainloop, which fetches whole 512-byte weight rows per stage; a caller that holds
    // W2^T already (weights kept [out,in]) passes it instead
    const uint16_t* W2T = w2_transposed ? (const uint16_t*)W2 : w.W2T;
    if (!w2_transposed &&
        (s = hip_check(coda::launch_transpose_bf16((const uint16_t*)W2, (int)D, (int)N2, w.W2T, st),
                       "bwd W2 transpose launch")))
      return s;
    if (unfused) {
      // P = dz W2^T stored, then its row and column statistics in a separate pass
      if ((s = hip_check(coda::launch_gemm_nn_store((const uint16_t*)dz, W2T, w.P, (int)M, (int)N2, (int)D, st),
                         "bwd P launch")))
        return s;
      if ((s = hip_check(coda::launch_bwd_p_from_mem(w.P, hh, r, gamma, w.G, w.part, w.part2, (int)M, (int)D, st),
                         "bwd P statistics launch")))
        return s;
    } else {
      if ((s = hip_check(coda::launch_bwd_p_nn((const uint16_t*)dz, W2T, hh, r, gamma, w.G, w.part, w.part2,
                                               (int)M, (int)D, (int)N2, st),
                         "bwd P launch")))
        return s;
    }
    if ((s = hip_check(coda::launch_bwd_reduce(w.part, (int)(D / 256), w.part2, (int)((M + 255) / 256), r, (int)M,
                                               (int)D, w.a, out_dgamma, st),
                       "bwd reduce launch")))
      return s;
    if ((s = hip_check(coda::launch_bwd_dh(w.G, hh, (const uint16_t*)dh_out, r, w.a, (int)M, (int)D,
                                           (uint16_t*)out_dR, w.dhT, w.nT, st, kPanels),
                       "bwd dh launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm_nt_store((const uint16_t*)out_dR, (const uint16_t*)W1, (uint16_t*)out_dX,
                                                  (int)M, (int)D, (int)K1, st),
                       "bwd dX launch")))
      return s;
    if ((s = hip_check(coda::launch_gemm_f32_trans(w.dhT, (const uint16_t*)X, out_dW1, (int)D, (int)M, (int)K1,
                                                   w.slabs, st, kPanels),
                       "bwd dW1 launch")))
      return s;
    return hip_check(coda::launch_gemm_f32_rowscale(w.nT, (const uint16_t*)dz, gamma, out_dW2, (int)D, (int)M,
                                                    (int)N2, w.slabs, st, kPanels),
                     "bwd dW2 launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

int coda_block_bwd(const void* X, const void* W1, const void* h, const float* r, const float* gamma, const void* W2,
                   const void* dz, const void* dh_out, void* out_dX, float* out_dW1, void* out_dR, float* out_dgamma,
                   float* out_dW2, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return block_bwd(X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, M, K1, D, N2,
                   workspace, workspace_bytes, stream, 0);
}

int coda_block_bwd_w2t(const void* X, const void* W1, const void* h, const float* r, const float* gamma,
                       const void* W2t, const void* dz, const void* dh_out, void* out_dX, float* out_dW1, void* out_dR,
                       float* out_dgamma, float* out_dW2, int64_t M, int64_t K1, int64_t D, int64_t N2,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return block_bwd(X, W1, h, r, gamma, W2t, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, M, K1, D, N2,
                   workspace, workspace_bytes, stream, 0, 1);
}

int coda_block_bwd_unfused(const void* X, const void* W1, const void* h, const float* r, const float* gamma,
                           const void* W2, const void* dz, const void* dh_out, void* out_dX, float* out_dW1,
                           void* out_dR, float* out_dgamma, float* out_dW2, int64_t M, int64_t K1, int64_t D,
                           int64_t N2, void* workspace, size_t workspace_bytes, void* stream) {
  return block_bwd(X, W1, h, r, gamma, W2, dz, dh_out, out_dX, out_dW1, out_dR, out_dgamma, out_dW2, M, K1, D, N2,
                   workspace, workspace_bytes, stream, 1);
}

}  // extern "C"

// ---- cross-entropy of a vocabulary projection ----
namespace {

struct CeWorkspace {
  float* part_m;  // [V/256][M] per-tile row maxima
  float* part_s;  // [V/256][M] per-tile row sums of exp(z - max)
  float* zlab;    // [M] the label's logit
  uint16_t* z;    // unfused: the bf16 logits [M,V]
  uint16_t* hp;   // H in K panels of 32 columns ([D/32][M][32]), the product's A operand on both paths
};

size_t carve_ce(void* ws, int64_t M, int64_t D, int64_t V, int unfused, CeWorkspace* w) {
  char* base = (char*)ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  };
  CeWorkspace x{};
  x.hp = (uint16_t*)take(ws_mat_bytes(M, D, 2));
  if (unfused) {
    x.z = (uint16_t*)take(ws_mat_bytes(M, V, 2));
  } else {
    x.part_m = (float*)take(ws_part_bytes(M, V));
    x.part_s = (float*)take(ws_part_bytes(M, V));
    x.zlab = (float*)take(ws_vec_bytes(M));
  }
  if (w) *w = x;
  return off;
}

int ce(const void* H, const void* W, const int* labels, float* out_loss, float* out_lse, int64_t M, int64_t D,
       int64_t V, void* workspace, size_t workspace_bytes, void* stream, int unfused) {
  try {
    int s;
    if ((s = check_ptr(H, "H")) || (s = check_ptr(W, "W")) || (s = check_ptr(labels, "labels")) ||
        (s = check_ptr(out_loss, "out_loss")) || (s = check_ptr(out_lse, "out_lse")))
      return s;
    if (M < 1 || D < 1 || V < 1)
      return fail(CODA_ERR_INVALID_ARG, "dimensions must be >= 1 (M=%lld D=%lld V=%lld)", (long long)M,
                  (long long)D, (long long)V);
    if (M > kMaxDim || D > kMaxDim || V > kMaxDim || M * D > kMaxDim * 2 || D * V > kMaxDim * 2 ||
        M * V > kMaxDim * 8)
      return fail(CODA_ERR_UNSUPPORTED, "dimensions too large");
    if (D % 128) return fail(CODA_ERR_UNSUPPORTED, "D=%lld is not a multiple of 128", (long long)D);
    if (V % 256) return fail(CODA_ERR_UNSUPPORTED, "V=%lld is not a multiple of 256", (long long)V);
    const size_t need = carve_ce(nullptr, M, D, V, unfused, nullptr);
    if (!workspace) return fail(CODA_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace & 255) return fail(CODA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (workspace_bytes < need)
      return fail(CODA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    const Range in[3] = {rng("H", H, (size_t)M * D * 2), rng("W", W, (size_t)D * V * 2),
                         rng("labels", labels, (size_t)M * 4)};
    const Range out[3] = {rng("out_loss", out_loss, (size_t)M * 4), rng("out_lse", out_lse, (size_t)M * 4),
                          rng("workspace", workspace, need)};
    if ((s = check_alias(in, 3, out, 3, nullptr, nullptr))) return s;
    hipStream_t st = (hipStream_t)stream;
    CeWorkspace w;
    carve_ce(workspace, M, D, V, unfused, &w);
    if ((s = hip_check(coda::launch_panelize_bf16((const uint16_t*)H, (int)M, (int)D, w.hp, st), "ce panel launch")))
      return s;
    if (unfused) {
      if ((s = hip_check(coda::launch_gemm_store(w.hp, (const uint16_t*)W, w.z, (int)M, (int)D, (int)V, st, kPanels),
                         "ce logits launch")))
        return s;
      return hip_check(coda::launch_ce_rows(w.z, labels, (int)M, (int)V, out_loss, out_lse, st), "ce rows launch");
    }
    if ((s = hip_check(coda::launch_ce_gemm(w.hp, (const uint16_t*)W, labels, w.part_m, w.part_s, w.zlab, (int)M,
                                            (int)D, (int)V, st, kPanels),
                       "ce gemm launch")))
      return s;
    return hip_check(coda::launch_ce_reduce(w.part_m, w.part_s, w.zlab, labels, (int)(V / 256), (int)M, (int)V,
                                            out_loss, out_lse, st),
                     "ce reduce launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

}  // namespace

extern "C" {

size_t coda_ce_workspace_bytes(int64_t M, int64_t D, int64_t V, int unfused) {
  if (M < 1 || D < 1 || V < 256 || M > kMaxDim || D > kMaxDim || V > kMaxDim) return 0;
  return carve_ce(nullptr, M, D, V, unfused, nullptr);
}

int coda_ce_fwd(const void* H, const void* W, const int32_t* labels, float* out_loss, float* out_lse, int64_t M,
                int64_t D, int64_t V, void* workspace, size_t workspace_bytes, void* stream) {
  return ce(H, W, labels, out_loss, out_lse, M, D, V, workspace, workspace_bytes, stream, 0);
}

int coda_ce_unfused(const void* H, const void* W, const int32_t* labels, float* out_loss, float* out_lse, int64_t M,
                    int64_t D, int64_t V, void* workspace, size_t workspace_bytes, void* stream) {
  return ce(H, W, labels, out_loss, out_lse, M, D, V, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"

// ---- SwiGLU: the forward that keeps z, and the backward of the SwiGLU epilogue ----
extern "C" {

int coda_block_fwd_save_z(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                          void* out_h, void* out_y, void* out_z, int64_t M, int64_t K1, int64_t D, int64_t N2,
                          void* workspace, size_t workspace_bytes, void* stream) {
  try {
    int s = validate_block(X, nullptr, W1, nullptr, R, gamma, W2, nullptr, eps, CODA_EPI_SWIGLU, out_h, out_y, M, K1,
                           D, N2, workspace, workspace_bytes, 0, 0);
    if (s) return s;
    if ((s = check_ptr(out_z, "out_z"))) return s;
    const Range zr = rng("out_z", out_z, (size_t)(M * N2) * 2);
    const Range others[8] = {rng("X", X, (size_t)(M * K1) * 2), rng("W1", W1, (size_t)(K1 * D) * 2),
                             rng("R", R, (size_t)(M * D) * 2),  rng("gamma", gamma, (size_t)D * 4),
                             rng("W2", W2, (size_t)(D * N2) * 2), rng("out_h", out_h, (size_t)(M * D) * 2),
                             rng("out_y", out_y, (size_t)(M * (N2 / 2)) * 2),
                             rng("workspace", workspace,
                                 ws_bytes(M, D, 0, 0) + ws_split_room(M, K1, D, N2, 0, 0, workspace_bytes))};
    for (int i = 0; i < 8; ++i)
      if (overlap(zr, others[i])) return fail(CODA_ERR_ALIAS, "out_z overlaps %s", others[i].name);
    return launch_block_fwd(X, W1, R, gamma, W2, eps, CODA_EPI_SWIGLU, out_h, out_y, M, K1, D, N2, workspace,
                            workspace_bytes, (hipStream_t)stream, out_z);
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

size_t coda_swiglu_bwd_workspace_bytes(int64_t M, int64_t F, int unfused) {
  if (M < 1 || F < 1 || M > kMaxDim || F > kMaxDim) return 0;
  return unfused ? align256((size_t)M * (size_t)F * 2) : 0;
}

}  // extern "C"

namespace {

int swiglu_bwd(const void* dout, const void* Wd, const void* z, void* out_dz, int64_t M, int64_t D, int64_t F,
               void* workspace, size_t workspace_bytes, void* stream, int unfused) {
  try {
    int s;
    if ((s = check_ptr(dout, "dout")) || (s = check_ptr(Wd, "Wd")) || (s = check_ptr(z, "z")) ||
        (s = check_ptr(out_dz, "out_dz")))
      return s;
    if (M < 1 || D < 1 || F < 1)
      return fail(CODA_ERR_INVALID_ARG, "dimensions must be >= 1 (M=%lld D=%lld F=%lld)", (long long)M, (long long)D,
                  (long long)F);
    if (M > kMaxDim || D > kMaxDim || F > kMaxDim || M * D > kMaxDim * 2 || F * D > kMaxDim * 2 ||
        M * F > kMaxDim)
      return fail(CODA_ERR_UNSUPPORTED, "dimensions too large");
    if (D % 128) return fail(CODA_ERR_UNSUPPORTED, "D=%lld is not a multiple of 128", (long long)D);
    if (F % 256) return fail(CODA_ERR_UNSUPPORTED, "F=%lld is not a multiple of 256", (long long)F);
    const size_t need = coda_swiglu_bwd_workspace_bytes(M, F, unfused);
    if (need) {
      if (!workspace) return fail(CODA_ERR_WORKSPACE, "workspace is NULL");
      if ((uintptr_t)workspace & 255) return fail(CODA_ERR_WORKSPACE, "workspace is not 256-byte aligned");
      if (workspace_bytes < need)
        return fail(CODA_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
    }
    const Range in[3] = {rng("dout", dout, (size_t)(M * D) * 2), rng("Wd", Wd, (size_t)(F * D) * 2),
                         rng("z", z, (size_t)(M * 2 * F) * 2)};
    const Range out[2] = {rng("out_dz", out_dz, (size_t)(M * 2 * F) * 2), rng("workspace", workspace, need)};
    if ((s = check_alias(in, 3, out, need ? 2 : 1, nullptr, nullptr))) return s;
    hipStream_t st = (hipStream_t)stream;
    if (!unfused)
      return hip_check(coda::launch_swiglu_bwd((const uint16_t*)dout, (const uint16_t*)Wd, (const uint16_t*)z,
                                               (uint16_t*)out_dz, (int)M, (int)D, (int)F, st),
                       "swiglu_bwd launch");
    uint16_t* dy = (uint16_t*)workspace;
    if ((s = hip_check(coda::launch_gemm_nt_store((const uint16_t*)dout, (const uint16_t*)Wd, dy, (int)M, (int)D,
                                                  (int)F, st),
                       "swiglu_bwd dy launch")))
      return s;
    return hip_check(coda::launch_swiglu_bwd_rows(dy, (const uint16_t*)z, (uint16_t*)out_dz, (int)M, (int)F, st),
                     "swiglu_bwd rows launch");
  } catch (...) {
    return fail(CODA_ERR_INTERNAL, "unexpected exception");
  }
}

}  // namespace

extern "C" {

int coda_swiglu_bwd(const void* dout, const void* Wd, const void* z, void* out_dz, int64_t M, int64_t D, int64_t F,
                    void* workspace, size_t workspace_bytes, void* stream) {
  return swiglu_bwd(dout, Wd, z, out_dz, M, D, F, workspace, workspace_bytes, stream, 0);
}

int coda_swiglu_bwd_unfused(const void* dout, const void* Wd, const void* z, void* out_dz, int64_t M, int64_t D,
                            int64_t F, void* workspace, size_t workspace_bytes, void* stream) {
  return swiglu_bwd(dout, Wd, z, out_dz, M, D, F, workspace, workspace_bytes, stream, 1);
}

}  // extern "C"
