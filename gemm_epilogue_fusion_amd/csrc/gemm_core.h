// gemm_core.h -- bf16 MFMA GEMM mainloop for gfx950 (CDNA4) shared by the block's two GEMMs.
//
// The CODA write-up ("CODA: new research optimizes Transformer training with GEMM-epilogue programming",
// section "CODA: the treasure hidden in the epilogue") splits a GEMM into a mainloop (tiled
// multiply-accumulate) and an epilogue (finishing work done while the output tile is still in registers).
// This file is the mainloop; the epilogues live with the kernels.
//
// Tiling (one workgroup = 4 waves of 64 lanes):
//   macro tile 256 (M) x 256 (N), K step 64, each wave owns a 128 x 128 sub-tile held as 4 x 4 blocks of
//   32 x 32 fp32 accumulators (256 accumulator registers per lane).
//   Operands: A [M,K] row-major (K contiguous); B [K,N] row-major (N contiguous), as weights are stored.
//   Both tiles are staged global -> VGPR -> LDS with 16-byte loads, double-buffered in LDS (128 KiB of the
//   160 KiB a CU has).  B stays N-contiguous in LDS and is read K-contiguous with ds_read_b64_tr_b16, the
//   gfx950 transposing LDS read, so no transpose pass over the weights is needed.
//   The MFMA is v_mfma_f32_32x32x16_bf16 with the B fragment as its first operand and the A fragment as
//   its second, which computes the transposed tile: every lane then owns one output row (4 groups of 4
//   consecutive columns per 32 x 32 block), so row-wise epilogue work (sums of squares, the row scale)
//   stays inside a lane.
//
// Lane layouts (verified on the device):
//   v_mfma_f32_32x32x16_bf16(a, b, c): a lane l holds a[row l%32][k 8(l/32)+e], b lane l holds
//   b[k 8(l/32)+e][col l%32]; result register r of lane l is c[row 8(r/4)+4(l/32)+r%4][col l%32].
//   ds_read_b64_tr_b16: inside each group of 16 lanes, element e of lane i is element i%4 of the 8 bytes
//   addressed by lane 4e + i/4 of the group.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 64;
constexpr int NTHREADS = 256;
constexpr int A_TILE_BYTES = BM * BK * 2;  // 32 KiB
constexpr int B_TILE_BYTES = BK * BN * 2;  // 32 KiB
constexpr int STAGE_BYTES = A_TILE_BYTES + B_TILE_BYTES;
constexpr int LDS_BYTES = 2 * STAGE_BYTES;  // 128 KiB

// ---- small conversions --------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- LDS layouts ------------------------------------------------------------------------------------
// A tile: 256 rows of 128 bytes (8 chunks of 16 B); chunk c of row m sits at slot c ^ (m % 8), so the 8
// rows a 16-byte fragment read touches at once fall in 8 different bank groups.
__device__ __forceinline__ int a_off(int m, int c) { return m * 128 + ((c ^ (m & 7)) << 4); }
// B tile: 64 rows of 512 bytes (32 chunks of 16 B); chunk c of row k sits at slot c ^ (2 (k % 4)), so the
// 4 rows x 32 bytes one transposing read of 16 lanes touches fall in 8 different bank groups.  Rows k and
// k + 4 share a swizzle, which lets the second half of a fragment reuse the first half's address + 2 KiB.
__device__ __forceinline__ int b_off(int k, int c) { return k * 512 + ((c ^ ((k & 3) << 1)) << 4); }

__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

// One K step of 64 from the LDS stage (sA, sB) into the wave's 4 x 4 accumulator blocks.
// wm, wn: the wave's position (0/1) in the 2 x 2 wave grid; lane: 0..63.
__device__ __forceinline__ void mma_stage(const char* sA, const char* sB, int wm, int wn, int lane,
                                          f32x16 (&acc)[4][4]) {
  const int q = lane >> 4;  // 16-lane group
  const int j = lane & 15;
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    s16x8 bfr[4], afr[4];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      // lane j of group q points at row k0 + j/4, columns n0 + 4 (j%4) .. +3 of the tile, so that after the
      // transposing read lane i of the group holds rows k0..k0+3 of column n0 + i.
      const int n0 = wn * 128 + nb * 32 + 16 * (q & 1);
      const int krow = 16 * s + 8 * (q >> 1) + (j >> 2);
      const int piece = (n0 >> 2) + (j & 3);  // 8-byte piece within the 512-byte row
      const char* p = sB + b_off(krow, piece >> 1) + ((piece & 1) << 3);
      s16x4 lo = lds_read_tr16(p);
      s16x4 hi = lds_read_tr16(p + 4 * 512);  // rows k0+4..k0+7, same swizzle
      bfr[nb] = (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = wm * 128 + mb * 32 + (lane & 31);
      afr[mb] = *(const s16x8*)(sA + a_off(m, 2 * s + (lane >> 5)));
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, bfr[nb]),
                                                             __builtin_bit_cast(bf16x8, afr[mb]),
                                                             acc[mb][nb], 0, 0, 0);
  }
}

// 8 bf16 scaled by one fp32 factor and rounded back to bf16 (round to nearest even).
__device__ __forceinline__ u32x4 scale_bf16x8(u32x4 v, float g) {
  u32x4 o;
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = pack_bf16(bf16_lo(v[i]) * g, bf16_hi(v[i]) * g);
  return o;
}

// The mainloop.  acc += A[m0:m0+256, :] * B[:, tile columns] over the full K.
//   A: [M,K] bf16 with row stride lda; rows >= M are read as row M-1 (their results are never stored).
//   B: [K,*] bf16 with row stride ldb; bcol = global column of the 8 tile columns this thread stages
//      (tile column chunk t % 32), which lets a tile gather column segments (gate | up halves).
//   gamma: if non-null, B row k is multiplied by gamma[k] while staged (W2' = diag(gamma) W2).
__device__ __forceinline__ void gemm_mainloop(const uint16_t* __restrict__ A, int64_t lda, int M, int m0,
                                              const uint16_t* __restrict__ B, int64_t ldb, int64_t bcol,
                                              const float* __restrict__ gamma, int K, char* smem,
                                              f32x16 (&acc)[4][4]) {
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave & 1, wn = wave >> 1;

#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = (f32x16){};

  // per-thread global pointers: A row t/8 + 32p (chunk t%8), B row t/32 + 8p (chunk t%32)
  const uint16_t* aptr[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    int row = m0 + (t >> 3) + 32 * p;
    row = row < M ? row : M - 1;
    aptr[p] = A + (int64_t)row * lda + (t & 7) * 8;
  }
  const uint16_t* bptr = B + (int64_t)(t >> 5) * ldb + bcol;
  const int64_t bstep = 8 * ldb;

  u32x4 ra[8], rb[8];
  float g[8];
  const int nk = K / BK;

  auto load = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int p = 0; p < 8; ++p) ra[p] = *(const u32x4*)(aptr[p] + k0);
#pragma unroll
    for (int p = 0; p < 8; ++p) rb[p] = *(const u32x4*)(bptr + (int64_t)k0 * ldb + p * bstep);
    if (gamma) {
#pragma unroll
      for (int p = 0; p < 8; ++p) g[p] = gamma[k0 + (t >> 5) + 8 * p];
    }
  };
  auto store = [&](char* stage) {
    char* sA = stage;
    char* sB = stage + A_TILE_BYTES;
#pragma unroll
    for (int p = 0; p < 8; ++p) *(u32x4*)(sA + a_off((t >> 3) + 32 * p, t & 7)) = ra[p];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      u32x4 v = gamma ? scale_bf16x8(rb[p], g[p]) : rb[p];
      *(u32x4*)(sB + b_off((t >> 5) + 8 * p, t & 31)) = v;
    }
  };

  load(0);
  store(smem);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    char* cur = smem + (kt & 1) * STAGE_BYTES;
    if (kt + 1 < nk) load(kt + 1);
    mma_stage(cur, cur + A_TILE_BYTES, wm, wn, lane, acc);
    if (kt + 1 < nk) store(smem + ((kt + 1) & 1) * STAGE_BYTES);
    __syncthreads();
  }
}

// Maps the linear workgroup id to a (row tile, column tile) pair.
// Workgroups are dealt to the 8 XCDs round-robin (id % 8), each XCD with its own L2.  The id is first
// remapped so that XCD x receives a contiguous range of the tile order, then tiles are ordered in groups of
// `group_m` row tiles (row tile fastest inside a group), so the tiles one XCD runs together share A row
// tiles and B column tiles in its L2.
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  int b = blockIdx.x;
  const int ntiles = tiles_m * tiles_n;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  const int group_size = group_m * tiles_n;
  const int group = b / group_size;
  const int first_m = group * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in_group = b - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

}  // namespace coda
