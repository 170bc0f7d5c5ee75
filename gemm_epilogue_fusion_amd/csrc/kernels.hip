// kernels.hip -- the block's kernels for gfx950 and their host-side launchers.
//
// Fused path (CODA write-up, "CODA: new research optimizes Transformer training with GEMM-epilogue
// programming", section "CODA: the treasure hidden in the epilogue"):
//   K1 gemm1_res_prms : h = X W1 + R in the epilogue, store bf16 h and bf16(h * gamma) (gamma broadcast
//                       along the rows, the write-up's vector-load primitive), per-row per-tile sums of
//                       squares of h
//   K2 prms_reduce    : the light reduction, r = 1 / sqrt(sum_t part / D + eps)
//   K3 gemm2_rowscale : mainloop on h * gamma against W2, i.e. h (diag(gamma) W2); the epilogue applies r
//                       (a per-row scalar commutes with the product) and SwiGLU
// Unfused baseline (three operators whose intermediates round-trip HBM, the pattern the same section
// describes as the conventional one):
//   U1 gemm_store     : T = bf16(X W1)
//   U2 add_rmsnorm    : h = bf16(T + R), n = bf16((T + R) r gamma)
//   U3 gemm2_rowscale : y = epi(n W2) (no gamma, no row scale)
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.h"
#include "launch.h"

namespace coda {

enum EpiMode { MODE_RES_PRMS = 0, MODE_STORE = 1, MODE_ROWSCALE = 2, MODE_ROWSCALE_SWIGLU = 3 };

// silu(x) = x / (1 + exp(-x)) in fp32 with the hardware exp2 and reciprocal (each about 1 ulp; the result
// is rounded to bf16 afterwards).
__device__ __forceinline__ float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Global column of a tile's 8-column chunk c (0..31) when the tile's 256 accumulator columns are one
// contiguous range starting at n0.
struct ContiguousCols {
  int64_t n0;
  __device__ int64_t operator()(int c) const { return n0 + 8 * c; }
};
// SwiGLU tiles: wave column group w (64 accumulator columns) holds 32 gate columns c0 + 32 w .. +32 followed
// by the matching 32 up columns half + c0 + 32 w .. +32, so gate and up of one output share a lane.
struct GateUpCols {
  int64_t c0, half;
  __device__ int64_t operator()(int c) const {
    const int nl = 8 * c, w = nl >> 6, within = nl & 63;
    return within < 32 ? c0 + 32 * w + within : half + c0 + 32 * w + (within - 32);
  }
};

// One GEMM with a programmable epilogue.
//   A [M,K] bf16 (row stride K), B [K,Nb] bf16 (row stride Nb); the accumulator tile covers 256 columns.
//   MODE_RES_PRMS:  out [M,Nb] = bf16(acc + R); out2 [M,Nb] = bf16((acc + R) * gamma[n]);
//                   part[tn][m] = sum over the tile's columns of (acc + R)^2
//   MODE_STORE:     out [M,Nb] = bf16(acc)
//   MODE_ROWSCALE:  out [M,Nb] = bf16(rs[m] * acc)            (rs == nullptr: scale 1)
//   MODE_ROWSCALE_SWIGLU: the tile's columns are 128 gate columns [tn*128, +128) and the matching 128 up
//                   columns [Nb/2 + tn*128, +128); out [M,Nb/2] = bf16(silu(rs*gate) * (rs*up))
template <int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_epilogue_kernel(
    const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, const float* __restrict__ gamma,
    const uint16_t* R, const float* __restrict__ rs, uint16_t* out, uint16_t* __restrict__ out2,
    float* __restrict__ part, int M, int K, int Nb, int group_m) {
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = Nb / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, group_m, tm, tn);
  const int m0 = tm * BM;

  f32x16 acc[4][NB];
  if (MODE == MODE_ROWSCALE_SWIGLU)
    gemm_mainloop(A, K, M, m0, B, Nb, GateUpCols{(int64_t)tn * 128, Nb / 2}, K, smem, acc);
  else
    gemm_mainloop(A, K, M, m0, B, Nb, ContiguousCols{(int64_t)tn * BN}, K, smem, acc);

  // ---- epilogue: the accumulator tile is still in registers ----
  // acc[mb][nb][r] is row m0 + 128 wm + 32 mb + lane%32, column 64 wn + 32 nb + 8 (r/4) + 4 (lane/32) + r%4
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5;

  if (MODE == MODE_RES_PRMS || MODE == MODE_STORE) {
    const int n_base = tn * BN + wn * 64 + 4 * half;
    // the tile's residual values first, as one batch of loads (rows past M read row M-1, never stored)
    u32x2 rr[4][NB][4];
    if (MODE == MODE_RES_PRMS) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
        const int mr = m < M ? m : M - 1;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) rr[mb][nb][gq] = *(const u32x2*)(R + (int64_t)mr * Nb + n_base + nb * 32 + 8 * gq);
      }
    }
    // gamma of this lane's columns: the same 4-column groups for every row
    f32x4 gv[NB][4];
    if (MODE == MODE_RES_PRMS) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) gv[nb][gq] = *(const f32x4*)(gamma + n_base + nb * 32 + 8 * gq);
    }
    float ss[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      float s = 0.0f;
      u32x2 hv[NB][4], gvv[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          float v0 = acc[mb][nb][4 * gq + 0], v1 = acc[mb][nb][4 * gq + 1];
          float v2 = acc[mb][nb][4 * gq + 2], v3 = acc[mb][nb][4 * gq + 3];
          if (MODE == MODE_RES_PRMS) {
            const u32x2 r2 = rr[mb][nb][gq];
            v0 += bf16_lo(r2[0]);
            v1 += bf16_hi(r2[0]);
            v2 += bf16_lo(r2[1]);
            v3 += bf16_hi(r2[1]);
            s += v0 * v0;
            s += v1 * v1;
            s += v2 * v2;
            s += v3 * v3;
            const f32x4 g = gv[nb][gq];
            gvv[nb][gq] = (u32x2){pack_bf16(v0 * g[0], v1 * g[1]), pack_bf16(v2 * g[2], v3 * g[3])};
          }
          hv[nb][gq] = (u32x2){pack_bf16(v0, v1), pack_bf16(v2, v3)};
        }
      ss[mb] = s;
      if (m < M) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            const int64_t o = (int64_t)m * Nb + n_base + nb * 32 + 8 * gq;
            *(u32x2*)(out + o) = hv[nb][gq];
            if (MODE == MODE_RES_PRMS) *(u32x2*)(out2 + o) = gvv[nb][gq];
          }
      }
    }
    if (MODE == MODE_RES_PRMS) {
      // lanes l and l+32 hold the same row: add their halves, then the four waves sharing the rows, in a
      // fixed order (no atomics: the partial sums are reproducible bit for bit)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) ss[mb] += __shfl_xor(ss[mb], 32);
      __syncthreads();  // every wave is done with the mainloop's LDS stages
      float* red = (float*)smem;  // [4 wn][256 rows]
      if (lane < 32) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) red[wn * 256 + wm * 128 + mb * 32 + lane] = ss[mb];
      }
      __syncthreads();
      if (wn == 0 && lane < 32) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int row = wm * 128 + mb * 32 + lane;
          const int m = m0 + row;
          if (m < M) part[(int64_t)tn * M + m] = ((red[row] + red[256 + row]) + red[512 + row]) + red[768 + row];
        }
      }
    }
  } else if (MODE == MODE_ROWSCALE) {
    const int n_base = tn * BN + wn * 64 + 4 * half;
    float scs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      scs[mb] = rs ? rs[m < M ? m : M - 1] : 1.0f;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      if (m >= M) continue;
      const float sc = scs[mb];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n_base + nb * 32 + 8 * gq;
          const f32x16& a = acc[mb][nb];
          *(u32x2*)(out + (int64_t)m * Nb + n) =
              (u32x2){pack_bf16(sc * a[4 * gq + 0], sc * a[4 * gq + 1]), pack_bf16(sc * a[4 * gq + 2], sc * a[4 * gq + 3])};
        }
    }
  } else {  // MODE_ROWSCALE_SWIGLU: accumulator block 0 holds gate columns, block 1 the matching up columns
    const int ny = Nb / 2;
    const int c_base = tn * 128 + wn * 32 + 4 * half;
    float scs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      scs[mb] = rs ? rs[m < M ? m : M - 1] : 1.0f;
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      if (m >= M) continue;
      const float sc = scs[mb];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const int c = c_base + 8 * gq;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gate = sc * acc[mb][0][4 * gq + e];
          const float up = sc * acc[mb][1][4 * gq + e];
          y[e] = silu_f32(gate) * up;
        }
        *(u32x2*)(out + (int64_t)m * ny + c) = (u32x2){pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
      }
    }
  }
}

// K2: r[i] = 1 / sqrt((sum_t part[t][i]) / D + eps), t summed in order 0..T-1.
__global__ __launch_bounds__(256) void prms_reduce_kernel(const float* __restrict__ part, int T, int M, float D,
                                                          float eps, float* __restrict__ r) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= M) return;
  float s = 0.0f;
  for (int t = 0; t < T; ++t) s += part[(int64_t)t * M + i];
  r[i] = 1.0f / sqrtf(s / D + eps);
}

// U2: one workgroup per row.  hf = T + R (fp32); h = bf16(hf); r = 1/sqrt(mean(hf^2) + eps);
// n = bf16(hf * r * gamma).  Each thread keeps up to 4 chunks of 8 columns in registers (D <= 8192).
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(const uint16_t* __restrict__ Tm, const uint16_t* R,
                                                          const float* __restrict__ gamma, uint16_t* H,
                                                          uint16_t* __restrict__ Nout, float* __restrict__ rout,
                                                          int D, float eps) {
  constexpr int MAXC = 4;
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x;
  const int nchunks = D / 8;
  float hv[MAXC][8];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + 256 * i;
    if (c < nchunks) {
      const u32x4 a = *(const u32x4*)(Tm + row * D + 8 * c);
      const u32x4 b = *(const u32x4*)(R + row * D + 8 * c);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hv[i][2 * q] = bf16_lo(a[q]) + bf16_lo(b[q]);
        hv[i][2 * q + 1] = bf16_hi(a[q]) + bf16_hi(b[q]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) s += hv[i][e] * hv[i][e];
    }
  }
  // wave reduction (fixed butterfly order), then across the 4 waves
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off);
  if ((t & 63) == 0) red[t >> 6] = s;
  __syncthreads();
  const float tot = ((red[0] + red[1]) + red[2]) + red[3];
  const float r = 1.0f / sqrtf(tot / (float)D + eps);
  if (t == 0 && rout) rout[row] = r;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + 256 * i;
    if (c < nchunks) {
      u32x4 ho, no;
      const float4 g0 = *(const float4*)(gamma + 8 * c);
      const float4 g1 = *(const float4*)(gamma + 8 * c + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ho[q] = pack_bf16(hv[i][2 * q], hv[i][2 * q + 1]);
        no[q] = pack_bf16(hv[i][2 * q] * r * gg[2 * q], hv[i][2 * q + 1] * r * gg[2 * q + 1]);
      }
      *(u32x4*)(H + row * D + 8 * c) = ho;
      *(u32x4*)(Nout + row * D + 8 * c) = no;
    }
  }
}

// ------------------------------------------------------------------------------------------------------
// launchers (host)

static int group_m_for(int tiles_m) { return tiles_m < 4 ? tiles_m : 4; }

template <int MODE>
static hipError_t launch_gemm(const uint16_t* A, const uint16_t* B, const float* gamma, const uint16_t* R,
                              const float* rs, uint16_t* out, uint16_t* out2, float* part, int M, int K, int Nb,
                              hipStream_t stream) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = Nb / BN;
  dim3 grid(tiles_m * tiles_n), block(NTHREADS);
  hipLaunchKernelGGL((gemm_epilogue_kernel<MODE>), grid, block, 0, stream, A, B, gamma, R, rs, out, out2, part, M,
                     K, Nb, group_m_for(tiles_m));
  return hipGetLastError();
}

hipError_t launch_gemm1_res_prms(const uint16_t* X, const uint16_t* W1, const uint16_t* R, const float* gamma,
                                 uint16_t* H, uint16_t* HG, float* part, int M, int K1, int D, hipStream_t stream) {
  return launch_gemm<MODE_RES_PRMS>(X, W1, gamma, R, nullptr, H, HG, part, M, K1, D, stream);
}

hipError_t launch_prms_reduce(const float* part, int T, int M, int D, float eps, float* r, hipStream_t stream) {
  dim3 grid((M + 255) / 256), block(256);
  hipLaunchKernelGGL(prms_reduce_kernel, grid, block, 0, stream, part, T, M, (float)D, eps, r);
  return hipGetLastError();
}

hipError_t launch_gemm2_rowscale(const uint16_t* A, const uint16_t* W2, const float* r, int swiglu, uint16_t* Y,
                                 int M, int D, int N2, hipStream_t stream) {
  if (swiglu) return launch_gemm<MODE_ROWSCALE_SWIGLU>(A, W2, nullptr, nullptr, r, Y, nullptr, nullptr, M, D, N2, stream);
  return launch_gemm<MODE_ROWSCALE>(A, W2, nullptr, nullptr, r, Y, nullptr, nullptr, M, D, N2, stream);
}

hipError_t launch_gemm_store(const uint16_t* X, const uint16_t* W, uint16_t* T, int M, int K, int N,
                             hipStream_t stream) {
  return launch_gemm<MODE_STORE>(X, W, nullptr, nullptr, nullptr, T, nullptr, nullptr, M, K, N, stream);
}

hipError_t launch_add_rmsnorm(const uint16_t* T, const uint16_t* R, const float* gamma, uint16_t* H, uint16_t* N,
                              float* r, int M, int D, float eps, hipStream_t stream) {
  dim3 grid(M), block(256);
  hipLaunchKernelGGL(add_rmsnorm_kernel, grid, block, 0, stream, T, R, gamma, H, N, r, D, eps);
  return hipGetLastError();
}

}  // namespace coda
