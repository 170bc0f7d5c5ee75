// ce_kernels.hip -- cross-entropy of a vocabulary projection with the logits never stored.
//
// The CODA write-up ("CODA: new research optimizes Transformer training with GEMM-epilogue programming") names
// cross-entropy among the operations its epilogue programming covers (section "CODA: the treasure hidden in
// the epilogue") and builds reductions from per-tile partial results merged by a light kernel (section "Five
// blocks and a Lego language").  Here:
//   C1 ce_gemm_kernel   : z = H W tile by tile (the bf16 mainloop of gemm_core.h); the epilogue reduces each row
//                         of the 256-column tile to a log-sum-exp pair (m, s), m = max z, s = sum exp(z - m),
//                         stored as part_m[t][i], part_s[t][i]; the tile holding a row's label stores that
//                         logit in zlab[i]
//   C2 ce_reduce_kernel : merges the pairs of each row in tile order: lse = m + log s, loss = lse - zlab (0 for a
//                         negative label, NaN for a label >= V)
// The unfused baseline stores the logits in bf16 (the first GEMM kernel's plain store) and reads them back:
//   CU ce_rows_kernel   : one workgroup per row of the stored logits.
// Both paths first copy H into K panels of 32 columns (panelize_bf16_kernel; ALayout in gemm_core.h): the
// product re-reads each H row tile once per 256 vocabulary columns, and whole-line loads of it shorten the
// product by more than the copy costs.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "gemm_core.h"
#include "launch.h"

namespace coda {

constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// (m, s) <- the log-sum-exp pair of the union of two sets of values, s = sum exp(v - m).  An empty set is
// (-inf, 0).  Symmetric in its two arguments, so two lanes merging each other's pairs get the same bits.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  if (s2 == 0.0f) return;
  if (s == 0.0f) {
    m = m2;
    s = s2;
    return;
  }
  const float mm = fmaxf(m, m2);
  s = s * exp2_hw((m - mm) * LOG2E) + s2 * exp2_hw((m2 - mm) * LOG2E);
  m = mm;
}

__global__ __launch_bounds__(NTHREADS, 1) void ce_gemm_kernel(const uint16_t* __restrict__ H,
                                                             const uint16_t* __restrict__ W,
                                                             const int* __restrict__ labels, float* __restrict__ part_m,
                                                             float* __restrict__ part_s, float* __restrict__ zlab,
                                                             int M, int K, int V, int group_m, int a_panels) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = V / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5;

  // the labels of this lane's four rows, fetched before the mainloop (rows past M read row M-1)
  int lab[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
    lab[mb] = labels[m < M ? m : M - 1];
  }

  f32x16 acc[4][NB];
  gemm_mainloop(H, a_panels ? ALayout{BK, (int64_t)M * BK} : ALayout{K, BK}, M, m0, W, V,
                ContiguousCols<8>{(int64_t)n0}, K, smem, acc);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(acc[mb][nb]));

  // acc[mb][nb][r] is row m0 + 128 wm + 32 mb + lane%32, column n0 + 64 wn + 32 nb + 8 (r/4) + 4 half + r%4:
  // a lane holds 32 of its row's 256 tile columns, the lane 32 apart the next 32, and the four waves of the
  // same wm the rest.
  float pm[4], ps[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float mx = acc[mb][0][0];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[mb][nb][r]);
    float s = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s += exp2_hw((acc[mb][nb][r] - mx) * LOG2E);
    lse_merge(mx, s, __shfl_xor(mx, 32), __shfl_xor(s, 32));
    pm[mb] = mx;
    ps[mb] = s;
    // the label's logit, if this lane holds its column
    const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
    const int c = lab[mb] - n0 - wn * 64 - 4 * half;  // column offset within this lane's pieces
    float zl = 0.0f;
    bool hit = false;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (c == 32 * nb + 8 * (r >> 2) + (r & 3)) {
          zl = acc[mb][nb][r];
          hit = true;
        }
    if (hit && m < M) zlab[m] = zl;
  }

  // the four waves of a row range merge their pairs through LDS (the mainloop's ring is free once every wave
  // has passed this barrier), in wave order
  __syncthreads();
  float* red_m = (float*)smem;             // [4 waves wn][256 rows]
  float* red_s = (float*)smem + 4 * BM;
  if (half == 0) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = wm * 128 + mb * 32 + lane;
      red_m[wn * BM + r] = pm[mb];
      red_s[wn * BM + r] = ps[mb];
    }
  }
  __syncthreads();
  if (t < BM && m0 + t < M) {
    float mx = red_m[t], s = red_s[t];
#pragma unroll
    for (int w = 1; w < 4; ++w) lse_merge(mx, s, red_m[w * BM + t], red_s[w * BM + t]);
    part_m[(int64_t)tn * M + m0 + t] = mx;
    part_s[(int64_t)tn * M + m0 + t] = s;
  }
}

// C2: 32 rows per workgroup, eight lanes groups per row each merging every eighth tile, then the eight merged
// in group order.
__global__ __launch_bounds__(256) void ce_reduce_kernel(const float* __restrict__ part_m,
                                                        const float* __restrict__ part_s,
                                                        const float* __restrict__ zlab, const int* __restrict__ labels,
                                                        int T, int M, int V, float* __restrict__ loss,
                                                        float* __restrict__ lse) {
  __shared__ float sm[8][32], ss[8][32];
  const int r = threadIdx.x & 31, g = threadIdx.x >> 5;
  const int i = blockIdx.x * 32 + r;
  float mx = -INFINITY, s = 0.0f;
  if (i < M)
    for (int tt = g; tt < T; tt += 8) lse_merge(mx, s, part_m[(int64_t)tt * M + i], part_s[(int64_t)tt * M + i]);
  sm[g][r] = mx;
  ss[g][r] = s;
  __syncthreads();
  if (g == 0 && i < M) {
#pragma unroll
    for (int q = 1; q < 8; ++q) lse_merge(mx, s, sm[q][r], ss[q][r]);
    const float l = mx + logf(s);
    const int lb = labels[i];
    lse[i] = l;
    loss[i] = lb < 0 ? 0.0f : (lb < V ? l - zlab[i] : __builtin_nanf(""));
  }
}

// CU: cross-entropy of stored bf16 logits Z [M,V], one workgroup of 256 lanes per row; each lane keeps a
// running (m, s) over 8-value chunks, then the lanes merge in a fixed tree.
__global__ __launch_bounds__(256) void ce_rows_kernel(const uint16_t* __restrict__ Z, const int* __restrict__ labels,
                                                      int M, int V, float* __restrict__ loss, float* __restrict__ lse) {
  __shared__ float sm[256], ss[256];
  const int i = blockIdx.x;
  const int t = threadIdx.x;
  const uint16_t* row = Z + (int64_t)i * V;
  float mx = -INFINITY, s = 0.0f;
  for (int c = t; c < V / 8; c += 256) {
    const u32x4 w = *(const u32x4*)(row + 8 * c);
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_lo(w[e]);
      v[2 * e + 1] = bf16_hi(w[e]);
    }
    float cm = v[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) cm = fmaxf(cm, v[e]);
    float cs = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) cs += exp2_hw((v[e] - cm) * LOG2E);
    lse_merge(mx, s, cm, cs);
  }
  sm[t] = mx;
  ss[t] = s;
  __syncthreads();
  for (int w = 128; w >= 1; w >>= 1) {
    if (t < w) {
      float a = sm[t], b = ss[t];
      lse_merge(a, b, sm[t + w], ss[t + w]);
      sm[t] = a;
      ss[t] = b;
    }
    __syncthreads();
  }
  if (t == 0) {
    const float l = sm[0] + logf(ss[0]);
    const int lb = labels[i];
    lse[i] = l;
    loss[i] = lb < 0 ? 0.0f : (lb < V ? l - bf16_lo(row[lb]) : __builtin_nanf(""));
  }
}

static int ce_group_m(int tiles_m) { return tiles_m < 4 ? tiles_m : 4; }

hipError_t launch_ce_gemm(const uint16_t* H, const uint16_t* W, const int* labels, float* part_m, float* part_s,
                          float* zlab, int M, int D, int V, hipStream_t stream, int a_panels) {
  const int tiles_m = (M + BM - 1) / BM;
  hipLaunchKernelGGL(ce_gemm_kernel, dim3(tiles_m * (V / BN)), dim3(NTHREADS), 0, stream, H, W, labels, part_m,
                     part_s, zlab, M, D, V, ce_group_m(tiles_m), a_panels);
  return hipGetLastError();
}

// dst = src [M, D] bf16 in K panels of 32 columns: src[m][32 p + j] -> dst[(p M + m) 32 + j].  A workgroup moves
// 64 rows of one panel: each lane one 16-byte piece, so a workgroup writes 4 KiB of the panel contiguously.
__global__ __launch_bounds__(256) void panelize_bf16_kernel(const uint16_t* __restrict__ src,
                                                            uint16_t* __restrict__ dst, int M, int D) {
  const int p = blockIdx.x;
  const int r = blockIdx.y * 64 + (threadIdx.x >> 2);
  const int c4 = threadIdx.x & 3;
  if (r >= M) return;
  const u32x4 v = *(const u32x4*)(src + (int64_t)r * D + 32 * p + 8 * c4);
  store_nt(dst + ((int64_t)p * M + r) * 32 + 8 * c4, v);
}

hipError_t launch_panelize_bf16(const uint16_t* src, int M, int D, uint16_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(panelize_bf16_kernel, dim3(D / 32, (M + 63) / 64), dim3(256), 0, stream, src, dst, M, D);
  return hipGetLastError();
}

hipError_t launch_ce_reduce(const float* part_m, const float* part_s, const float* zlab, const int* labels, int T,
                            int M, int V, float* loss, float* lse, hipStream_t stream) {
  hipLaunchKernelGGL(ce_reduce_kernel, dim3((M + 31) / 32), dim3(256), 0, stream, part_m, part_s, zlab, labels, T, M,
                     V, loss, lse);
  return hipGetLastError();
}

hipError_t launch_ce_rows(const uint16_t* Z, const int* labels, int M, int V, float* loss, float* lse,
                          hipStream_t stream) {
  hipLaunchKernelGGL(ce_rows_kernel, dim3(M), dim3(256), 0, stream, Z, labels, M, V, loss, lse);
  return hipGetLastError();
}

}  // namespace coda
