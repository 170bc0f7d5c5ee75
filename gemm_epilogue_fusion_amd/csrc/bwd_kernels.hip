// bwd_kernels.hip -- backward of the GEMM -> residual -> RMSNorm -> GEMM block for gfx950.
//
// The CODA write-up ("CODA: new research optimizes Transformer training with GEMM-epilogue programming",
// sections "CODA: the treasure hidden in the epilogue" and "Experimental results") applies the epilogue
// rewrite to back-propagation as well.  Forward: h = X W1 + R, r_i = 1/sqrt(mean_j h_ij^2 + eps), n = r h,
// u = n * gamma, z = u W2.  Given dz (the gradient of z) and dh_out (the gradient arriving at the residual
// stream h), the textbook backward is
//   du = dz W2^T;  dgamma_j = sum_i du_ij n_ij;  dh = r (du gamma - n mean_j(du_ij gamma_j n_ij)) + dh_out
//   dR = dh;  dX = dh W1^T;  dW1 = X^T dh;  dW2 = u^T dz.
// With P = dz W2^T the per-row pieces become
//   dh_ij = r_i gamma_j P_ij - a_i h_ij + dh_out_ij,   a_i = r_i^3 S_i / D,   S_i = sum_j gamma_j P_ij h_ij
//   dgamma_j = sum_i P_ij r_i h_ij,                    dW2 = diag(gamma) (n^T dz)
// so the kernels are
//   B1 bwd_p      : P = dz W2^T (W2 read as its own [D,N2] rows, K = N2); the epilogue, with the tile's h, r
//                   and gamma, stores G = r gamma P (bf16), per-row partial sums of gamma P h (one slot per
//                   column tile) and per-column partial sums of P r h (one slot per row tile)
//   B2 bwd_reduce : a_i from the row partials (summed in tile order), dgamma from the column partials
//   B3 bwd_dh     : dh = G - a h + dh_out -> dR (bf16), and the transposes dh^T, n^T [D,M] (bf16)
//   B4 dX  = dh W1^T        (W1 read as its own [K1,D] rows)
//   B5 dW1 = (dh^T X)^T     (fp32, the tile stored transposed)
//   B6 dW2 = diag(gamma) (n^T dz)   (fp32, gamma as the output row scale)
// The unfused baseline replaces B1 by a GEMM that stores du = P (bf16) and a separate pass over du and h
// that computes what B1's epilogue computes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_core.h"
#include "launch.h"

namespace coda {

enum BwdMode { BWD_P = 0, BWD_P_FROM_MEM = 1, BWD_STORE_BF16 = 2, BWD_F32_ROWSCALE = 3, BWD_F32_TRANS = 4,
               BWD_SWIGLU = 5 };

struct BwdArgs {
  const uint16_t* A;   // [M, K] row-major
  const uint16_t* B;   // [K, Nb] row-major, or (BT) [Nb, K] row-major
  const uint16_t* h;   // BWD_P*: h [M, Nb]
  const float* r;      // BWD_P*: r [M]
  const float* gamma;  // BWD_P*: gamma [Nb];  BWD_F32_ROWSCALE: the output row scale [M]
  uint16_t* out;       // bf16 output [M, Nb] (G or the plain product)
  float* outf;         // fp32 output: [M, Nb], or [Nb, M] (BWD_F32_TRANS)
  float* part;         // BWD_P*: row partials [Nb/256][M]
  float* part2;        // BWD_P*: column partials [ceil(M/256)][Nb]
  int M, K, Nb, group_m;
  int64_t slab;        // BWD_F32_*: split-K partial products go to outf + blockIdx.y * slab (K per split = K)
                       // BWD_SWIGLU: h = z [M, 2 Nb] (gate | up), out = dz [M, 2 Nb]
  int a_panels;        // non-transposed B: A in K panels [K_total / 32][M][32] (ALayout in gemm_core.h)
};

// silu(x) = x s(x) and its derivative s(x) (1 + x (1 - s(x))), s the logistic function, in fp32 with the
// hardware exp2 and reciprocal (each about 1 ulp)
__device__ __forceinline__ float logistic_f32(float x) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * 1.4426950408889634f));
}

// SwiGLU backward of four values: dg = dy u silu'(g), du = dy silu(g)
__device__ __forceinline__ void swiglu_bwd4(const float (&dy)[4], const float (&g)[4], const float (&u)[4],
                                            float (&dg)[4], float (&du)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float sg = logistic_f32(g[e]);
    dg[e] = dy[e] * u[e] * (sg * (1.0f + g[e] * (1.0f - sg)));
    du[e] = dy[e] * (g[e] * sg);
  }
}

// rows r0 .. r0+127 of a bf16 tile of 256 columns between global memory (row stride ld) and LDS (tile_off<32>
// layout relative to row r0); rows past M read row M-1 and are not written
__device__ __forceinline__ void load_half_tile(const uint16_t* src, int ld, int m0, int n0, int M, char* dst) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int r0 = wave * 16 + 2 * j;  // 2 rows of 512 bytes per wave instruction
    const int r = r0 + lane / 32;
    const int slot = lane % 32;
    int m = m0 + r;
    m = m < M ? m : M - 1;
    g2lds16(src + (int64_t)m * ld + n0 + 8 * (slot ^ (r & 31)), dst + r0 * 512);
  }
}
__device__ __forceinline__ void store_half_tile(const char* srcl, uint16_t* dst, int ld, int m0, int n0, int M) {
  const int t = threadIdx.x;
  const int c = t % 32;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = p * 16 + t / 32;
    const u32x4 v = *(const u32x4*)(srcl + tile_off<32>(r, c));
    const int m = m0 + r;
    if (m < M) store_nt(dst + (int64_t)m * ld + n0 + 8 * c, v);
  }
}

// The SwiGLU backward's first half tile of z (rows m0 .. m0+127): gate rows 0..63 and 64..127, then up rows
// 0..63, into ring stages 0, 1, 2 as the mainloop drains (NoDrain in gemm_core.h); the staging layout is
// load_half_tile's, gate at smem and up at smem + 64 KiB.
struct SwigluDrain {
  static constexpr int LOADS = 4;
  const uint16_t* z;
  int ldz, m0, n0, nb, M;
  char* smem;
  __device__ void operator()(int s) const {
    if (s < 2)
      load_tile_rows64<32>(z, ldz, m0, n0, M, smem, 64 * s);
    else
      load_tile_rows64<32>(z, ldz, m0, nb + n0, M, smem + 65536, 0);
  }
};

struct RowsFrom {
  int64_t n0;
  __device__ int64_t operator()(int r) const { return n0 + r; }
};

// fp32 tile staging: 128 rows x 256 columns, row pitch 1 KiB, 16-byte chunk c of row r at c ^ (r % 64)
__device__ __forceinline__ int f32_off(int r, int c) { return r * 1024 + ((c ^ (r & 63)) << 4); }
// transposed fp32 staging: 256 rows (the tile's columns) x 128 columns (the tile's rows), pitch 512 B,
// 4-byte word w of row q at word (w ^ 32 (q % 2)) so that the two lane halves use different banks
__device__ __forceinline__ int f32t_off(int q, int w) { return q * 512 + ((w ^ ((q & 1) << 5)) << 2); }

template <int MODE, bool BT>
__global__ __launch_bounds__(NTHREADS, 1) void bwd_gemm_kernel(BwdArgs args) {
  constexpr bool PMODE = MODE == BWD_P || MODE == BWD_P_FROM_MEM;
  // the mainloop ring (reused as the staging area), plus the row / column partial-sum exchanges
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES + (PMODE ? 6144 : 0)];
  const int M = args.M, Nb = args.Nb;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = Nb / BN;
  int tm, tn;
  tile_coords(tiles_m, tiles_n, args.group_m, tm, tn);
  const int m0 = tm * BM, n0 = tn * BN;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int half = lane >> 5;

  f32x16 acc[4][NB];
  if (MODE == BWD_P_FROM_MEM) {
    // the product was stored by an earlier kernel (bf16 [M, Nb]): bring the tile into the accumulator layout
    load_tile_rows<32>(args.A, Nb, m0, n0, M, smem);
    wait_barrier<0>();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int rr = wm * 128 + mb * 32 + (lane & 31);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const u32x2 v = *(const u32x2*)(smem + tile_off<32>(rr, wn * 8 + nb * 4 + gq) + 8 * half);
          acc[mb][nb][4 * gq + 0] = bf16_lo(v[0]);
          acc[mb][nb][4 * gq + 1] = bf16_hi(v[0]);
          acc[mb][nb][4 * gq + 2] = bf16_lo(v[1]);
          acc[mb][nb][4 * gq + 3] = bf16_hi(v[1]);
        }
    }
  } else if (BT) {
    if (MODE == BWD_SWIGLU)  // the first half tile of z arrives as the ring drains (SwigluDrain)
      gemm_mainloop_nt(args.A, args.K, M, m0, args.B, args.K, RowsFrom{n0}, args.K, smem, acc,
                       SwigluDrain{args.h, 2 * Nb, m0, n0, Nb, M, smem});
    else
      gemm_mainloop_nt(args.A, args.K, M, m0, args.B, args.K, RowsFrom{n0}, args.K, smem, acc);
  } else {
    // split K: workgroup row blockIdx.y multiplies K range [y K, (y + 1) K) of the gridDim.y K ranges
    const int64_t k0 = (int64_t)blockIdx.y * args.K;
    const int64_t lda = (int64_t)args.K * gridDim.y;
    const int64_t pstep = (int64_t)M * BK;  // one K panel of A
    const uint16_t* a0 = args.a_panels ? args.A + (k0 / BK) * pstep : args.A + k0;
    const ALayout al = args.a_panels ? ALayout{BK, pstep} : ALayout{lda, BK};
    if (MODE == BWD_P)  // the h tile's first 192 rows arrive as the ring drains
      gemm_mainloop(a0, al, M, m0, args.B + k0 * Nb, Nb, ContiguousCols<8>{n0}, args.K, smem, acc, NoHook{},
                    TileRowsDrain{args.h, Nb, m0, n0, M, smem});
    else
      gemm_mainloop(a0, al, M, m0, args.B + k0 * Nb, Nb, ContiguousCols<8>{n0}, args.K, smem, acc);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(acc[mb][nb]));
  __syncthreads();  // every wave is done with the LDS (ring or tile)

  // acc[mb][nb][e] is row m0 + 128 wm + 32 mb + lane%32, column n0 + 64 wn + 32 nb + 8 (e/4) + 4 half + e%4
  if (PMODE) {
    if (MODE == BWD_P && !BT)
      load_tile_rows64<32>(args.h, Nb, m0, n0, M, smem, 192);  // rows 0 .. 191 came with the mainloop's drain
    else
      load_tile_rows<32>(args.h, Nb, m0, n0, M, smem);
    float rv[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      rv[mb] = args.r[m < M ? m : M - 1];
    }
    const int c_base = n0 + wn * 64 + 4 * half;
    f32x4 gv[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) gv[nb][gq] = *(const f32x4*)(args.gamma + c_base + nb * 32 + 8 * gq);
    wait_barrier<0>();
    float srow[4];
    float tcol[NB][4][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int e = 0; e < 4; ++e) tcol[nb][gq][e] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int rr = wm * 128 + mb * 32 + (lane & 31);
      const bool live = m0 + rr < M;
      const float ri = rv[mb];
      float s = 0.0f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          char* slot = smem + tile_off<32>(rr, wn * 8 + nb * 4 + gq) + 8 * half;
          const u32x2 hv = *(const u32x2*)slot;
          const float hf[4] = {bf16_lo(hv[0]), bf16_hi(hv[0]), bf16_lo(hv[1]), bf16_hi(hv[1])};
          float g[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p = acc[mb][nb][4 * gq + e];
            const float gp = gv[nb][gq][e] * p;
            s += gp * hf[e];
            if (live) tcol[nb][gq][e] += p * ri * hf[e];
            g[e] = ri * gp;
          }
          *(u32x2*)slot = (u32x2){pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3])};
        }
      srow[mb] = s;
    }
    // column partials: the 32 lanes of each half hold the same columns for different rows
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float v = tcol[nb][gq][e];
#pragma unroll
          for (int off = 1; off < 32; off <<= 1) v += __shfl_xor(v, off);
          tcol[nb][gq][e] = v;
        }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) srow[mb] += __shfl_xor(srow[mb], 32);
    float* red = (float*)(smem + LDS_BYTES);          // [4 wn][256 rows]
    float* red2 = (float*)(smem + LDS_BYTES + 4096);  // [2 wm][256 columns]
    if (lane < 32) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) red[wn * 256 + wm * 128 + mb * 32 + lane] = srow[mb];
    }
    if ((lane & 31) == 0) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq)
#pragma unroll
          for (int e = 0; e < 4; ++e) red2[wm * 256 + wn * 64 + nb * 32 + 8 * gq + 4 * half + e] = tcol[nb][gq][e];
    }
    __syncthreads();
    store_tile_rows<32>(smem, args.out, Nb, m0, n0, M);
    if (wn == 0 && lane < 32) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int row = wm * 128 + mb * 32 + lane;
        const int m = m0 + row;
        if (m < M) args.part[(int64_t)tn * M + m] = ((red[row] + red[256 + row]) + red[512 + row]) + red[768 + row];
      }
    }
    if (t < 256) args.part2[(int64_t)tm * Nb + n0 + t] = red2[t] + red2[256 + t];
  } else if (MODE == BWD_STORE_BF16) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int rr = wm * 128 + mb * 32 + (lane & 31);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x16& a = acc[mb][nb];
          *(u32x2*)(smem + tile_off<32>(rr, wn * 8 + nb * 4 + gq) + 8 * half) =
              (u32x2){pack_bf16(a[4 * gq], a[4 * gq + 1]), pack_bf16(a[4 * gq + 2], a[4 * gq + 3])};
        }
    }
    __syncthreads();
    store_tile_rows<32>(smem, args.out, Nb, m0, n0, M);
  } else if (MODE == BWD_F32_ROWSCALE) {
    // fp32 [M, Nb] with a row scale, staged 128 rows at a time
    float rs[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + wm * 128 + mb * 32 + (lane & 31);
      rs[mb] = args.gamma ? args.gamma[m < M ? m : M - 1] : 1.0f;
    }
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (wm == hh) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int rr = mb * 32 + (lane & 31);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const f32x16& a = acc[mb][nb];
              const float sc = rs[mb];
              *(f32x4*)(smem + f32_off(rr, (wn * 64 + nb * 32 + 8 * gq + 4 * half) >> 2)) =
                  (f32x4){a[4 * gq] * sc, a[4 * gq + 1] * sc, a[4 * gq + 2] * sc, a[4 * gq + 3] * sc};
            }
        }
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int rr = p * 8 + (t >> 6);
        const int c = t & 63;
        const f32x4 v = *(const f32x4*)(smem + f32_off(rr, c));
        const int m = m0 + hh * 128 + rr;
        if (m < M) store_nt(args.outf + blockIdx.y * args.slab + (int64_t)m * Nb + n0 + 4 * c, v);
      }
      __syncthreads();
    }
  } else if (MODE == BWD_SWIGLU) {
    // the tile is dy for columns n0 .. n0+255 of F = Nb; the gate and up tiles of z come into LDS 128 rows at a
    // time (gate in the first 64 KiB, up in the second), the waves owning those rows replace them in place by
    // dg and du, and both go out as whole rows
    const int ldz = 2 * Nb;
#pragma unroll 1
    for (int hh = 0; hh < 2; ++hh) {
      if (hh == 0) {  // the mainloop's drain has fetched gate rows 0 .. 127 and up rows 0 .. 63
        load_tile_rows64<32>(args.h, ldz, m0, Nb + n0, M, smem + 65536, 64);
      } else {
        load_half_tile(args.h, ldz, m0 + 128 * hh, n0, M, smem);
        load_half_tile(args.h, ldz, m0 + 128 * hh, Nb + n0, M, smem + 65536);
      }
      wait_barrier<0>();
      if (wm == hh) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int rr = mb * 32 + (lane & 31);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              char* sg = smem + tile_off<32>(rr, wn * 8 + nb * 4 + gq) + 8 * half;
              char* su = sg + 65536;
              const u32x2 gv = *(const u32x2*)sg, uv = *(const u32x2*)su;
              const float g[4] = {bf16_lo(gv[0]), bf16_hi(gv[0]), bf16_lo(gv[1]), bf16_hi(gv[1])};
              const float u[4] = {bf16_lo(uv[0]), bf16_hi(uv[0]), bf16_lo(uv[1]), bf16_hi(uv[1])};
              const float dy[4] = {acc[mb][nb][4 * gq], acc[mb][nb][4 * gq + 1], acc[mb][nb][4 * gq + 2],
                                   acc[mb][nb][4 * gq + 3]};
              float dg[4], du[4];
              swiglu_bwd4(dy, g, u, dg, du);
              *(u32x2*)sg = (u32x2){pack_bf16(dg[0], dg[1]), pack_bf16(dg[2], dg[3])};
              *(u32x2*)su = (u32x2){pack_bf16(du[0], du[1]), pack_bf16(du[2], du[3])};
            }
        }
      }
      __syncthreads();
      store_half_tile(smem, args.out, ldz, m0 + 128 * hh, n0, M);
      store_half_tile(smem + 65536, args.out, ldz, m0 + 128 * hh, Nb + n0, M);
      __syncthreads();
    }
  } else {  // BWD_F32_TRANS: outf [Nb, M] = the tile transposed, fp32, staged 128 tile rows at a time
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      if (wm == hh) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int w = mb * 32 + (lane & 31);  // tile row within the half = output column
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int q = wn * 64 + nb * 32 + 8 * gq + 4 * half + e;  // tile column = output row
                *(float*)(smem + f32t_off(q, w)) = acc[mb][nb][4 * gq + e];
              }
        }
      }
      __syncthreads();
#pragma unroll
      for (int p = 0; p < 16; ++p) {
        const int q = p * 16 + (t >> 5);
        const int c = t & 31;  // 4 words = 4 output columns
        const float* src = (const float*)(smem + q * 512);
        const int sw = (q & 1) << 5;
        const f32x4 v = {src[(4 * c) ^ sw], src[(4 * c + 1) ^ sw], src[(4 * c + 2) ^ sw], src[(4 * c + 3) ^ sw]};
        const int col = m0 + hh * 128 + 4 * c;
        if (col < M) store_nt(args.outf + blockIdx.y * args.slab + (int64_t)(n0 + q) * M + col, v);
      }
      __syncthreads();
    }
  }
}

// B2: a_i = r_i^3 / D * sum_t part[t][i] (t in order), one thread per row; dgamma_j = sum_q part2[q][j], 32
// lanes per column (each lane sums q = lane, lane + 32, ... in order, then a fixed butterfly).
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const float* __restrict__ part, int T,
                                                         const float* __restrict__ part2, int Q,
                                                         const float* __restrict__ r, int M, int D,
                                                         float* __restrict__ a, float* __restrict__ dgamma) {
  const int row_blocks = (M + 255) / 256;
  if ((int)blockIdx.x < row_blocks) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < M) {
      float s = 0.0f;
#pragma unroll 8
      for (int t = 0; t < T; ++t) s += part[(int64_t)t * M + i];
      const float ri = r[i];
      a[i] = ri * ri * ri * s / (float)D;
    }
    return;
  }
  const int j = ((int)blockIdx.x - row_blocks) * 8 + (threadIdx.x >> 5);
  const int lane = threadIdx.x & 31;
  float g = 0.0f;
  if (j < D)
    for (int q = lane; q < Q; q += 32) g += part2[(int64_t)q * D + j];
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) g += __shfl_xor(g, off, 32);
  if (j < D && lane == 0) dgamma[j] = g;
}

// Sum of S split-K slabs of n floats (slab s at src + s * n), in slab order, times an optional row scale
// (rows of `cols` floats).  n and cols multiples of 4.
__global__ __launch_bounds__(256) void slab_sum_kernel(const float* __restrict__ src, int S, int64_t n, int cols,
                                                       const float* __restrict__ rowsc, float* __restrict__ dst) {
  const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e >= n) return;
  f32x4 v = *(const f32x4*)(src + e);
  for (int s = 1; s < S; ++s) v += *(const f32x4*)(src + (int64_t)s * n + e);
  if (rowsc) v *= rowsc[e / cols];
  store_nt(dst + e, v);
}

// B3: one 64 x 64 tile of [M, D] per workgroup.  dh = G - a_i h + dh_out (fp32, then bf16) -> dR; the same
// dh and n = bf16(r_i h) are written transposed, [D, M], through LDS.
__global__ __launch_bounds__(256) void bwd_dh_kernel(const uint16_t* __restrict__ G, const uint16_t* __restrict__ h,
                                                     const uint16_t* __restrict__ dh_out, const float* __restrict__ r,
                                                     const float* __restrict__ a, int M, int D,
                                                     uint16_t* __restrict__ dR, uint16_t* __restrict__ dhT,
                                                     uint16_t* __restrict__ nT, int panels) {
  __shared__ uint16_t tdh[64][64 + 2];
  __shared__ uint16_t tn[64][64 + 2];
  const int t = threadIdx.x;
  const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;
  const int ri_ = t >> 2;          // tile row
  const int cj = (t & 3) * 16;     // 16 columns
  const int64_t i = i0 + ri_;
  const float rr = r[i], ai = a[i];
#pragma unroll
  for (int hlf = 0; hlf < 2; ++hlf) {
    const int j = j0 + cj + 8 * hlf;
    const u32x4 gv = *(const u32x4*)(G + i * D + j);
    const u32x4 hv = *(const u32x4*)(h + i * D + j);
    const u32x4 ov = dh_out ? *(const u32x4*)(dh_out + i * D + j) : (u32x4){0u, 0u, 0u, 0u};
    u32x4 dv, nv;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float h0 = bf16_lo(hv[q]), h1 = bf16_hi(hv[q]);
      const float d0 = bf16_lo(gv[q]) - ai * h0 + bf16_lo(ov[q]);
      const float d1 = bf16_hi(gv[q]) - ai * h1 + bf16_hi(ov[q]);
      dv[q] = pack_bf16(d0, d1);
      nv[q] = pack_bf16(rr * h0, rr * h1);
      const int c = cj + 8 * hlf + 2 * q;
      tdh[c][ri_] = (uint16_t)(dv[q] & 0xffff);
      tdh[c + 1][ri_] = (uint16_t)(dv[q] >> 16);
      tn[c][ri_] = (uint16_t)(nv[q] & 0xffff);
      tn[c + 1][ri_] = (uint16_t)(nv[q] >> 16);
    }
    store_nt(dR + i * D + j, dv);
  }
  __syncthreads();
  // transposed rows: row j of the tile holds 64 values of i; 8 per thread-chunk, 512 chunks per tensor
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int ch = t + 256 * p;
    const int jr = ch >> 3, ic = (ch & 7) * 8;
    u32x4 o1, o2;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o1[q] = (uint32_t)tdh[jr][ic + 2 * q] | ((uint32_t)tdh[jr][ic + 2 * q + 1] << 16);
      o2[q] = (uint32_t)tn[jr][ic + 2 * q] | ((uint32_t)tn[jr][ic + 2 * q + 1] << 16);
    }
    // [D, M] rows, or (panels) K panels over M of the weight-gradient products: ((m / 32) D + d) 32 + m % 32
    const int64_t off = panels ? ((int64_t)((i0 + ic) >> 5) * D + j0 + jr) * 32 + ((i0 + ic) & 31)
                               : (int64_t)(j0 + jr) * M + i0 + ic;
    store_nt(dhT + off, o1);
    store_nt(nT + off, o2);
  }
}

// ------------------------------------------------------------------------------------------------------
// launchers (host)

template <int MODE, bool BT>
static hipError_t launch_bwd(const BwdArgs& a0, hipStream_t stream, int ksplit = 1) {
  BwdArgs a = a0;
  const int tiles_m = (a.M + BM - 1) / BM;
  const int tiles_n = a.Nb / BN;
  a.group_m = tiles_m < 4 ? tiles_m : 4;
  a.K /= ksplit;
  hipLaunchKernelGGL((bwd_gemm_kernel<MODE, BT>), dim3(tiles_m * tiles_n, ksplit), dim3(NTHREADS), 0, stream, a);
  return hipGetLastError();
}

int gemm_ksplit(int M, int N, int K) {
  const int tiles = ((M + BM - 1) / BM) * (N / BN);
  int s = 1;
  while (s < 8 && tiles * s < 256 && K % (K_MULTIPLE * s * 2) == 0) s *= 2;
  return s;
}

hipError_t launch_swiglu_bwd(const uint16_t* dout, const uint16_t* Wd, const uint16_t* z, uint16_t* dz, int M, int D,
                             int F, hipStream_t stream) {
  BwdArgs a{};
  a.A = dout;
  a.B = Wd;
  a.h = z;
  a.out = dz;
  a.M = M;
  a.K = D;
  a.Nb = F;
  return launch_bwd<BWD_SWIGLU, true>(a, stream);
}

hipError_t launch_bwd_p(const uint16_t* dz, const uint16_t* W2, const uint16_t* h, const float* r, const float* gamma,
                        uint16_t* G, float* part, float* part2, int M, int D, int N2, hipStream_t stream) {
  BwdArgs a{dz, W2, h, r, gamma, G, nullptr, part, part2, M, N2, D, 0, 0};
  return launch_bwd<BWD_P, true>(a, stream);
}

// B1 on the NN mainloop: W2T = W2^T [N2, D] is read K-major like any [in,out] weight.
hipError_t launch_bwd_p_nn(const uint16_t* dz, const uint16_t* W2T, const uint16_t* h, const float* r,
                           const float* gamma, uint16_t* G, float* part, float* part2, int M, int D, int N2,
                           hipStream_t stream) {
  BwdArgs a{dz, W2T, h, r, gamma, G, nullptr, part, part2, M, N2, D, 0, 0};
  return launch_bwd<BWD_P, false>(a, stream);
}

hipError_t launch_gemm_nn_store(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int K, int N,
                                hipStream_t stream) {
  BwdArgs a{A, B, nullptr, nullptr, nullptr, C, nullptr, nullptr, nullptr, M, K, N, 0, 0};
  return launch_bwd<BWD_STORE_BF16, false>(a, stream);
}

// dst [C, R] = src [R, C]^T (bf16), 64 x 64 tiles through LDS (rows of 66 elements: the column reads of the
// second phase fall in different banks); R and C multiples of 64.
__global__ __launch_bounds__(256) void transpose_bf16_kernel(const uint16_t* __restrict__ src, int R, int C,
                                                             uint16_t* __restrict__ dst) {
  __shared__ uint16_t tile[64][66];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = ty + 4 * j;
    tile[i][tx] = src[(int64_t)(r0 + i) * C + c0 + tx];
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = ty + 4 * j;
    dst[(int64_t)(c0 + i) * R + r0 + tx] = tile[tx][i];
  }
}

hipError_t launch_transpose_bf16(const uint16_t* src, int R, int C, uint16_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(transpose_bf16_kernel, dim3(C / 64, R / 64), dim3(256), 0, stream, src, R, C, dst);
  return hipGetLastError();
}

hipError_t launch_bwd_p_from_mem(const uint16_t* P, const uint16_t* h, const float* r, const float* gamma, uint16_t* G,
                                 float* part, float* part2, int M, int D, hipStream_t stream) {
  BwdArgs a{P, nullptr, h, r, gamma, G, nullptr, part, part2, M, 0, D, 0, 0};
  return launch_bwd<BWD_P_FROM_MEM, false>(a, stream);
}

// The unfused counterpart of S1's epilogue: one thread per 4 consecutive columns of dy [M,F].
__global__ __launch_bounds__(256) void swiglu_bwd_rows_kernel(const uint16_t* __restrict__ dy,
                                                              const uint16_t* __restrict__ z, uint16_t* __restrict__ dz,
                                                              int M, int F) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // 4-column group
  const int64_t groups = (int64_t)M * (F / 4);
  if (q >= groups) return;
  const int64_t m = q / (F / 4), f = 4 * (q % (F / 4));
  const u32x2 dv = *(const u32x2*)(dy + m * F + f);
  const u32x2 gv = *(const u32x2*)(z + m * 2 * F + f);
  const u32x2 uv = *(const u32x2*)(z + m * 2 * F + F + f);
  const float d[4] = {bf16_lo(dv[0]), bf16_hi(dv[0]), bf16_lo(dv[1]), bf16_hi(dv[1])};
  const float g[4] = {bf16_lo(gv[0]), bf16_hi(gv[0]), bf16_lo(gv[1]), bf16_hi(gv[1])};
  const float u[4] = {bf16_lo(uv[0]), bf16_hi(uv[0]), bf16_lo(uv[1]), bf16_hi(uv[1])};
  float dg[4], du[4];
  swiglu_bwd4(d, g, u, dg, du);
  store_nt(dz + m * 2 * F + f, (u32x2){pack_bf16(dg[0], dg[1]), pack_bf16(dg[2], dg[3])});
  store_nt(dz + m * 2 * F + F + f, (u32x2){pack_bf16(du[0], du[1]), pack_bf16(du[2], du[3])});
}

hipError_t launch_swiglu_bwd_rows(const uint16_t* dy, const uint16_t* z, uint16_t* dz, int M, int F,
                                  hipStream_t stream) {
  const int64_t groups = (int64_t)M * (F / 4);
  hipLaunchKernelGGL(swiglu_bwd_rows_kernel, dim3((unsigned)((groups + 255) / 256)), dim3(256), 0, stream, dy, z, dz,
                     M, F);
  return hipGetLastError();
}

hipError_t launch_gemm_nt_store(const uint16_t* A, const uint16_t* Bt, uint16_t* C, int M, int K, int N,
                                hipStream_t stream) {
  BwdArgs a{A, Bt, nullptr, nullptr, nullptr, C, nullptr, nullptr, nullptr, M, K, N, 0, 0};
  return launch_bwd<BWD_STORE_BF16, true>(a, stream);
}

static hipError_t slab_sum(const float* slabs, int S, int64_t n, int cols, const float* rowsc, float* dst,
                           hipStream_t stream) {
  hipLaunchKernelGGL(slab_sum_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, stream, slabs, S, n, cols,
                     rowsc, dst);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_rowscale(const uint16_t* A, const uint16_t* B, const float* rowsc, float* C, int M, int K,
                                    int N, float* slabs, hipStream_t stream, int a_panels) {
  const int S = gemm_ksplit(M, N, K);
  const int64_t n = (int64_t)M * N;
  BwdArgs a{A, B, nullptr, nullptr, S > 1 ? nullptr : rowsc, nullptr, S > 1 ? slabs : C, nullptr, nullptr, M, K, N,
            0, n, a_panels};
  hipError_t e = launch_bwd<BWD_F32_ROWSCALE, false>(a, stream, S);
  if (e != hipSuccess || S == 1) return e;
  return slab_sum(slabs, S, n, N, rowsc, C, stream);
}

hipError_t launch_gemm_f32_trans(const uint16_t* A, const uint16_t* B, float* Ct, int M, int K, int N, float* slabs,
                                 hipStream_t stream, int a_panels) {
  const int S = gemm_ksplit(M, N, K);
  const int64_t n = (int64_t)M * N;
  BwdArgs a{A, B, nullptr, nullptr, nullptr, nullptr, S > 1 ? slabs : Ct, nullptr, nullptr, M, K, N, 0, n, a_panels};
  hipError_t e = launch_bwd<BWD_F32_TRANS, false>(a, stream, S);
  if (e != hipSuccess || S == 1) return e;
  return slab_sum(slabs, S, n, M, nullptr, Ct, stream);
}

hipError_t launch_bwd_reduce(const float* part, int T, const float* part2, int Q, const float* r, int M, int D,
                             float* a, float* dgamma, hipStream_t stream) {
  const int blocks = (M + 255) / 256 + (D + 7) / 8;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(blocks), dim3(256), 0, stream, part, T, part2, Q, r, M, D, a, dgamma);
  return hipGetLastError();
}

hipError_t launch_bwd_dh(const uint16_t* G, const uint16_t* h, const uint16_t* dh_out, const float* r, const float* a,
                         int M, int D, uint16_t* dR, uint16_t* dhT, uint16_t* nT, hipStream_t stream, int panels) {
  hipLaunchKernelGGL(bwd_dh_kernel, dim3(D / 64, M / 64), dim3(256), 0, stream, G, h, dh_out, r, a, M, D, dR, dhT, nT,
                     panels);
  return hipGetLastError();
}

}  // namespace coda
