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
// With e4m3 operands K1 stores h only, and K2 (prms_reduce_quant) forms h * gamma from the stored h and
// quantises it per row for K3.  Inside the block, h * gamma (or its codes) is written in K panels of K3's
// stage width (ALayout in gemm_core.h) and K2 is folded into K3 where D <= 4096 (RowFold).
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

enum EpiMode { MODE_RES_PRMS = 0, MODE_STORE = 1, MODE_ROWSCALE = 2, MODE_ROWSCALE_SWIGLU = 3, MODE_ROWSCALE_ROPE = 4 };

// Rotary position embedding applied in MODE_ROWSCALE_ROPE's epilogue: the first n_rot output columns form
// heads of 64; in each, the pair (i, i + 32) is rotated by pos * base^(-2 i / 64), pos = row mod seq_len.
// rev[i] = base^(-2 i / 64) / (2 pi) is built on the host in double: the angle is taken in revolutions, reduced
// to [0, 1) and fed to the hardware sine and cosine, whose input is in revolutions over a limited range.
struct RopeParams {
  int seq_len;
  int n_rot;
  float rev[32];
};

// The partial-RMS reduce folded into the second GEMM (T > 0): the workgroup forms the row scales of its own
// rows from the first GEMM's partial sums, r = 1 / sqrt((sum_t part[t][m]) / D + eps) with t summed in order
// 0..T-1 (the expression of prms_reduce_kernel, so the values are the same), and the tiles of column 0 write
// r out for the backward.
constexpr int FOLD_MAX_T = 16;  // D <= 4096
struct RowFold {
  int T;
  float D;
  float eps;
  float* r;
};

__device__ __forceinline__ void rope_sincos(float pos, float rev, float& c, float& s) {
  const float t = __builtin_amdgcn_fractf(pos * rev);
  c = __builtin_amdgcn_cosf(t);
  s = __builtin_amdgcn_sinf(t);
}

// ---- e4m3 quantisation ----------------------------------------------------------------------------------
constexpr float E4M3_MAX = 448.0f;

// Four fp32 values -> four OCP e4m3fn bytes, round to nearest even (v_cvt_pk_fp8_f32; gfx950 uses the OCP
// encoding).  Values are clamped to +-448 first, so the conversion never sees an out-of-range input.
__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -E4M3_MAX), E4M3_MAX);
  b = fminf(fmaxf(b, -E4M3_MAX), E4M3_MAX);
  c = fminf(fmaxf(c, -E4M3_MAX), E4M3_MAX);
  d = fminf(fmaxf(d, -E4M3_MAX), E4M3_MAX);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// Power-of-two scale of a block of 32 values (MX-style e4m3): the smallest e with amax <= 448 * 2^e, 0 for
// amax = 0 (or NaN), limited to [-127, 127].  Exact: with amax = m 2^e2 (0.5 <= m < 1), the test
// 2m <= 1.75 on the mantissa bits decides between e2 - 9 and e2 - 8.
__device__ __forceinline__ int mx_scale_exp(float amax) {
  if (!(amax > 0.0f)) return 0;
  const uint32_t u = __float_as_uint(amax);
  const int ef = (int)((u >> 23) & 0xff);
  if (ef == 0) return -127;  // below 2^-126: under every scale the 8-bit exponent can hold
  if (ef == 255) return 127;
  const int e2 = ef - 126;
  const int e = (u & 0x7fffffu) <= 0x600000u ? e2 - 9 : e2 - 8;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// silu(x) = x / (1 + exp(-x)) in fp32 with the hardware exp2 and reciprocal (each about 1 ulp; the result
// is rounded to bf16 afterwards).
__device__ __forceinline__ float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(-x * 1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// SwiGLU tiles: wave column group w (64 accumulator columns) holds 32 gate columns c0 + 32 w .. +32 followed
// by the matching 32 up columns half + c0 + 32 w .. +32, so gate and up of one output share a lane.
template <int W>
struct GateUpCols {
  int64_t c0, half;
  __device__ int64_t operator()(int c) const {
    const int nl = W * c, w = nl >> 6, within = nl & 63;
    return within < 32 ? c0 + 32 * w + within : half + c0 + 32 * w + (within - 32);
  }
};

// One GEMM with a programmable epilogue.  The accumulator tile covers 256 columns of B; A [M,K] and B
// [K,Nb] are bf16 (FP8 = false) or e4m3 bytes (FP8 = true), row-major.  In the epilogue the accumulator is
// first multiplied by rowsc[m] * colsc[n] where those are given (dequantisation scales and / or the row
// scale r; column scales exist for e4m3 operands only, so the bf16 kernels compile without them), giving v:
//   MODE_RES_PRMS:  out [M,Nb] = bf16(v + R); out2 [M,Nb] = bf16((v + R) * gamma[n]) (bf16 operands only);
//                   part[tn][m] = sum over the tile's columns of (v + R)^2
//   MODE_STORE:     out [M,Nb] = bf16(v)
//   MODE_ROWSCALE:  out [M,Nb] = bf16(v)
//   MODE_ROWSCALE_ROPE: out [M,Nb] = bf16(rope(v)) (bf16 operands; see RopeParams)
//   MODE_ROWSCALE_SWIGLU: the tile's columns are 128 gate columns [tn*128, +128) and the matching 128 up
//                   columns [Nb/2 + tn*128, +128); out [M,Nb/2] = bf16(silu(v_gate) * v_up)
// panels != 0: MODE_RES_PRMS writes out2 (h * gamma, or the MX codes) in K panels of the second GEMM's stage
// width ([Nb / 32][M][32] bf16, [Nb / 64][M][64] bytes), and the row-scale modes and MODE_STORE read A from such
// panels (ALayout in gemm_core.h); A of MODE_RES_PRMS is always row-major.
// SMALL (bf16, M <= SMALL_MAX_ROWS): the mainloop's small-row form (wave_pos in gemm_core.h).
// HALF (bf16, row-scale modes): the half-tile form of the mainloop.  The workgroups take the tiles from ks.full on (in
// tile order) as two 128-row halves each, both halves of a tile on one XCD (KSplit::halves).
// The kernels are gemm_epilogue_kernel (whole tiles, the K split) and gemm_epilogue_half_kernel (HALF) below.
template <int MODE, bool FP8, bool MX, bool SMALL, bool HALF>
__device__ __forceinline__ void gemm_epilogue_body(
    const void* __restrict__ A, const void* __restrict__ B, const float* __restrict__ gamma, const uint16_t* R,
    const float* __restrict__ rowsc, const float* __restrict__ colsc, uint16_t* out, uint16_t* __restrict__ out2,
    float* __restrict__ part, int M, int K, int Nb, int group_m, RopeParams rope, RowFold fold, uint8_t* mxs,
    int panels, KSplit ks) {
  constexpr bool ROWSCALE_MODE = MODE == MODE_ROWSCALE || MODE == MODE_ROWSCALE_SWIGLU || MODE == MODE_ROWSCALE_ROPE;
  static_assert(!SMALL || !FP8, "the small-row form is bf16 only");
  static_assert(!HALF || (!FP8 && !SMALL && ROWSCALE_MODE), "the half-tile form is for the bf16 row-scale modes");
  // MX (e4m3 only): K1 (MODE_RES_PRMS) also quantises h * gamma in blocks of 32 columns with power-of-two
  // scales (codes to out2, scales to mxs); K3 (row-scale modes) reads its A operand's block scales from mxs
  constexpr bool MX_A = FP8 && MX && ROWSCALE_MODE;
  // row-scale modes of the second GEMM can fold the partial-RMS reduce in (see RowFold), except the e4m3 path
  // with per-row A scales, whose reduce kernel also quantises
  constexpr bool CAN_FOLD = (!FP8 || MX) && ROWSCALE_MODE;
  // the mainloop ring (reused as the output staging area), plus the row-sum exchange of MODE_RES_PRMS (and the bf16
  // K1's gamma) or the folded row scales, plus the MX scale stages
  constexpr int FOLD_LDS = CAN_FOLD ? 1024 + FOLD_MAX_T * BM * 4 : 0;  // row scales, then the partial sums
  constexpr int GAMMA_LDS = MODE == MODE_RES_PRMS && !FP8 ? BN * 4 : 0;
  __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES + (MODE == MODE_RES_PRMS ? 4096 + GAMMA_LDS : FOLD_LDS) +
                                                    (MX_A ? NSTAGE * MX_STAGE_BYTES : 0)];
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = Nb / BN;
  // the split of the last wave (KSplit); the first GEMMs also clear the second GEMM's tickets
  constexpr bool FIRST_GEMM = MODE == MODE_RES_PRMS || MODE == MODE_STORE;
  constexpr bool CAN_SPLIT = ROWSCALE_MODE || FIRST_GEMM;
  if (FIRST_GEMM && ks.clear && blockIdx.x == 0)
    for (int i = threadIdx.x; i < ks.nclear; i += NTHREADS) ks.clear[i] = 0;
  int tm, tn, piece = -1, tile_ord = 0, hrow = 0;
  if (HALF) {
    // workgroup p takes half p % 2 of tile ks.full + p / 2, with p remapped (as tile_coords_split remaps its pieces)
    // so that each XCD receives a contiguous range: the two halves of a tile run on one XCD
    int p = blockIdx.x;
    const int np = gridDim.x;
    if ((np & 15) == 0) p = (p & 7) * (np >> 3) + (p >> 3);
    hrow = 128 * (p & 1);
    tile_of_order(ks.full + (p >> 1), tiles_m, tiles_n, group_m, tm, tn);
  } else if (CAN_SPLIT && ks.full >= 0) {
    piece = tile_coords_split(tiles_m, tiles_n, group_m, ks.full, ks.lg, tm, tn, tile_ord);
  } else {
    tile_coords(tiles_m, tiles_n, group_m, tm, tn);
  }
  const int m0 = tm * BM + hrow;
  // the rows this workgroup may store: a half-tile's 128, or the tile's up to M
  const int Mh = HALF ? (M < m0 + 128 ? M : m0 + 128) : M;
  // a piece multiplies over its share of K
  const int kpart = piece >= 0 ? K >> ks.lg : K;
  const int kbeg = piece > 0 ? piece * kpart : 0;

  // folded reduce: before the mainloop the partial sums of the tile's rows go global -> LDS (4 bytes per lane,
  // 64 rows per load, rows past M read row M-1), older than every stage load, so the mainloop's first wait
  // covers them; once the first stage has landed thread t < 256 sums row t's T values in order and forms r
  // bf16 K1: gamma of the tile's 256 columns goes global -> LDS in one direct load of wave 0 before the mainloop,
  // older than every stage load, so the mainloop's first wait covers it; the epilogue reads it from there (at 64
  // rows, waiting for it after the mainloop cost 1.1 us of the block's 18 us)
  const float* gamma_lds = (const float*)(smem + LDS_BYTES + 4096);
  if (GAMMA_LDS > 0 && threadIdx.x < 64)
    __builtin_amdgcn_global_load_lds(gamma + tn * BN + 4 * threadIdx.x, (lds_void*)gamma_lds, 16, 0, 0);
  const bool folding = CAN_FOLD && fold.T > 0;
  float* fold_r = (float*)(smem + LDS_BYTES);                 // [256] the row scales
  float* fold_part = (float*)(smem + LDS_BYTES + 1024);       // [T][256] the partial sums
  float rfold = 1.0f;
  if (CAN_FOLD && folding) {
    const int wv = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int ln = (int)threadIdx.x & 63;
    for (int u = wv; u < fold.T * 4; u += NWAVES) {
      const int tt = u >> 2, r = (u & 3) * 64 + ln;
      const int row = m0 + r < M ? m0 + r : M - 1;
      __builtin_amdgcn_global_load_lds(part + (int64_t)tt * M + row, (lds_void*)(fold_part + tt * BM + (u & 3) * 64),
                                       4, 0, 0);
    }
  }
  auto fold_hook = [&]() {
    if (CAN_FOLD && folding && threadIdx.x < BM) {
      float s = 0.0f;
      for (int i = 0; i < fold.T; ++i) s += fold_part[i * BM + threadIdx.x];
      rfold = 1.0f / sqrtf(s / fold.D + fold.eps);
    }
  };

  constexpr int KS = FP8 ? BK8 : BK;  // K per stage: the panel width
  const ALayout al = ((ROWSCALE_MODE || MODE == MODE_STORE) && panels) ? ALayout{KS, (int64_t)M * KS}
                                                                        : ALayout{K, KS};
  f32x16 acc[4][NB];
  if (FP8) {
    // a piece's share of K starts kbeg / KS stages in: A and B by that offset, and the block scales (MX) by
    // that many K steps of their layout (mx_scale_index: tiles_m * 512 bytes per step)
    const uint8_t* A8 = (const uint8_t*)A + (int64_t)(kbeg / KS) * al.step;
    const uint8_t* B8 = (const uint8_t*)B + (int64_t)kbeg * Nb;
    const uint8_t* asc = MX_A ? mxs + (int64_t)(kbeg / KS) * tiles_m * 512 : mxs;
    char* mx_smem = smem + LDS_BYTES + FOLD_LDS;
    if (MODE == MODE_ROWSCALE_SWIGLU)
      gemm_mainloop_fp8<MX_A>(A8, al, M, m0, B8, Nb, GateUpCols<16>{(int64_t)tn * 128, Nb / 2}, kpart, smem, acc,
                              fold_hook, asc, mx_smem);
    else if (MODE == MODE_RES_PRMS)  // the residual tile's first 192 rows arrive as the ring drains
      gemm_mainloop_fp8<MX_A>(A8, al, M, m0, B8, Nb, ContiguousCols<16>{(int64_t)tn * BN}, kpart, smem, acc,
                              fold_hook, asc, mx_smem, TileRowsDrain{R, Nb, m0, tn * BN, M, smem});
    else
      gemm_mainloop_fp8<MX_A>(A8, al, M, m0, B8, Nb, ContiguousCols<16>{(int64_t)tn * BN}, kpart, smem, acc,
                              fold_hook, asc, mx_smem);
  } else {
    const uint16_t* A16 = (const uint16_t*)A + (int64_t)(kbeg / KS) * al.step;
    const uint16_t* B16 = (const uint16_t*)B + (int64_t)kbeg * Nb;
    constexpr std::integral_constant<bool, SMALL> small{};
    constexpr std::integral_constant<bool, HALF> half_tile{};
    // (a half tile's A rows past its 128 read its last row, never used)
    if (MODE == MODE_ROWSCALE_SWIGLU)
      gemm_mainloop(A16, al, Mh, m0, B16, Nb, GateUpCols<8>{(int64_t)tn * 128, Nb / 2}, kpart, smem, acc, fold_hook,
                    NoDrain{}, small, half_tile);
    else if (MODE == MODE_RES_PRMS)  // the residual tile's first 192 rows arrive as the ring drains
      gemm_mainloop(A16, al, M, m0, B16, Nb, ContiguousCols<8>{(int64_t)tn * BN}, kpart, smem, acc, fold_hook,
                    TileRowsDrain{R, Nb, m0, tn * BN, M, smem}, small);
    else
      gemm_mainloop(A16, al, Mh, m0, B16, Nb, ContiguousCols<8>{(int64_t)tn * BN}, kpart, smem, acc, fold_hook,
                    NoDrain{}, small, half_tile);
  }

  // Materialise the accumulators here: otherwise the compiler may sink the last MFMAs into the epilogue's
  // row-masked store blocks, which keeps every operand fragment alive into the epilogue.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(acc[mb][nb]));

  if (CAN_SPLIT && piece >= 0) {
    // A piece of a split tile (KSplit): the pieces meet in a binary tree.  At level l the piece stores its
    // accumulators in its slot, lane-major (wave w's register group j at w * 8192 + j * 256 floats, lane l at 4 l:
    // each store instruction writes 1 KiB), then takes a ticket from its node's counter; the workgroup that draws
    // ticket 1 adds the sibling's slot, written in the same layout, to its accumulators and goes up a level.
    // Ordering: every wave waits for its own slot stores to complete (vmcnt(0); a workgroup barrier alone does not
    // wait for other waves' global stores), then after the barrier one wave makes them visible on every XCD
    // (agent-scope release: the L2 writes its dirty lines back, whichever wave wrote them) and takes the ticket.  On
    // the other side each wave discards stale cached lines (agent-scope acquire) before its own slot loads.  The
    // release runs in one wave only: it acts on the whole L2, and in all eight waves (as seq_cst fences) it made the
    // 1B MLP-out -> QKV GEMM2 2.4x slower; the acquire in every wave cost 0.2-3 us per block against one wave's.
    // The ticket is broadcast through a word of the kernel's LDS array that nothing reads or writes at this point:
    // the first word of the row sums' exchange area (used later in the epilogue), of the folded-reduce area (its
    // partial sums were consumed by the hook long before), or of ring stage 0 (free after the mainloop where no
    // drain refills it).  A __shared__ variable of its own would make the compiler wait for every in-flight direct
    // load (vmcnt(0)) before each LDS read of the mainloop, unable to tell that the two objects do not overlap
    // (measured: 40% on the product's time, whole tiles included).
    int& ticket = *(int*)(MODE == MODE_RES_PRMS ? smem + LDS_BYTES : FOLD_LDS > 0 ? smem + LDS_BYTES + 1024 : smem);
    const int S = 1 << ks.lg;
    const int64_t st = tile_ord - ks.full;  // the split tile's index
    float* slots = ks.part + st * (2 * S - 2) * KSPLIT_SLOT_FLOATS;
    int* tickets = ks.cnt + st * (S - 1);
    const int lane_off = (int)(threadIdx.x >> 6) * 8192 + (int)(threadIdx.x & 63) * 4;
    int idx = piece;  // this workgroup's node at the current level
#pragma unroll 1
    for (int l = 0; l < ks.lg; ++l) {
      const int slot0 = 2 * S - 2 * (S >> l);  // level l's first slot
      float* mine = slots + (int64_t)(slot0 + idx) * KSPLIT_SLOT_FLOATS + lane_off;
      const float* other = slots + (int64_t)(slot0 + (idx ^ 1)) * KSPLIT_SLOT_FLOATS + lane_off;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x16& a = acc[mb][nb];
            *(f32x4*)(mine + ((mb * NB + nb) * 4 + q) * 256) =
                (f32x4){a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]};
          }
      wait_barrier<0>();  // every wave's slot stores have completed (a workgroup barrier alone does not wait for them)
      if (threadIdx.x < 64) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      if (threadIdx.x == 0)
        ticket = __hip_atomic_fetch_add(tickets + (S - (S >> l)) + (idx >> 1), 1, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      if (ticket == 0) return;  // the sibling goes on
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // each wave, before its own slot loads
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 o = *(const f32x4*)(other + ((mb * NB + nb) * 4 + q) * 256);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[mb][nb][4 * q + e] += o[e];
          }
      idx >>= 1;
    }
  }

  // ---- epilogue: the accumulator tile is still in registers ----
  // acc[mb][nb][r] is row m0 + 128 wm + 32 mb + lane%32, column 64 wn + 32 nb + 8 (r/4) + 4 (lane/32) + r%4.
  // Each lane owns 4-column pieces of its rows, so the results are first staged as a bf16 tile in LDS
  // (the mainloop's ring is free by then) and written out as whole rows: stores of 8 scattered bytes per
  // lane would cost the memory system a request per 16 bytes.
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  int wm, wn;
  wave_pos<SMALL>(wave, wm, wn);
  const int half = lane >> 5;
  // the tile row of accumulator block mb's lane 0: in the half-tile form blocks 0 and 1 hold rows 64 wm .. +64 and
  // blocks 2 and 3 (zero) map to rows 128 .. 255, which are never stored
  auto rowof = [&](int mb) { return HALF ? (mb >> 1) * 128 + wm * 64 + (mb & 1) * 32 : wm * 128 + mb * 32; };

  // per-row scales of this lane's four rows (rows past M read row M-1; they are never stored)
  float rsv[4];
  if (CAN_FOLD && folding) {
    if (t < BM) {
      fold_r[t] = rfold;
      if (tn == 0 && m0 + t < Mh) fold.r[m0 + t] = rfold;
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int m = m0 + rowof(mb) + (lane & 31);
      // row scales: the e4m3 dequantisation scales, or r in the row-scale modes (bf16 GEMM1 and plain stores
      // have none, so their kernels compile without the load)
      rsv[mb] = ((FP8 || ROWSCALE_MODE) && rowsc) ? rowsc[m < M ? m : M - 1] : 1.0f;
    }
  }
  // e4m3: this lane's column dequantisation scales, loaded once per tile (32 registers; the mainloop's fragments
  // are dead by now) and before the barrier, so their latency overlaps it.  SwiGLU: csv[0..3] gate, csv[4..7] up
  // columns; otherwise csv[4 nb + gq] for accumulator block nb, column group gq.
  f32x4 csv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t col = MODE == MODE_ROWSCALE_SWIGLU
                            ? (j < 4 ? 0 : Nb / 2) + tn * 128 + wn * 32 + 4 * half + 8 * (j & 3)
                            : tn * BN + wn * 64 + 4 * half + (j >> 2) * 32 + 8 * (j & 3);
    csv[j] = (FP8 && colsc) ? *(const f32x4*)(colsc + col) : (f32x4){1.f, 1.f, 1.f, 1.f};
  }
  __syncthreads();  // every wave is done with the mainloop's LDS stages (and the folded row scales are in)
  if (CAN_FOLD && folding) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) rsv[mb] = fold_r[rowof(mb) + (lane & 31)];
  }

  if (MODE == MODE_RES_PRMS || MODE == MODE_STORE || MODE == MODE_ROWSCALE) {
    // h * gamma is written by the bf16 K1 only (the e4m3 path forms it in K2 from the stored h)
    constexpr bool WRITE_HG = MODE == MODE_RES_PRMS && !FP8;
    // gamma of this lane's 4-column groups (the same for every row), from the copy in LDS
    f32x4 gv[NB][4];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
        gv[nb][gq] = WRITE_HG ? *(const f32x4*)(gamma_lds + wn * 64 + 4 * half + nb * 32 + 8 * gq)
                              : (f32x4){1.f, 1.f, 1.f, 1.f};
    if (MODE == MODE_RES_PRMS) {
      // the residual tile R[m0.., tn*256..] into the staging area with direct loads (whole rows); the mainloop has
      // fetched rows 0 .. 191 as its ring drained.  A tile whose rows end before row 192 has nothing left to fetch
      // (rows past M are never stored).
      if (m0 + 192 < M) load_tile_rows64<32>(R, Nb, m0, tn * BN, M, smem, 192);
      wait_barrier<0>();
    }
    float ss[4];
    u32x2 hgv[4][NB][4];  // bf16(h * gamma), staged after h has been written out
    // The small-row form stores rows 0 .. 63 only, so it leaves the other rows' slots alone and stages h * gamma in
    // rows 64 .. 127 of the staging area beside h: both tiles go out after one barrier instead of three.
    constexpr bool ONE_PASS = SMALL && WRITE_HG;
    constexpr int STAGED = SMALL ? SMALL_MAX_ROWS : BM;  // the staged rows that may be stored
    char* const hg_stage = smem + SMALL_MAX_ROWS * 512;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = rowof(mb) + (lane & 31);
      float s = 0.0f;
      const bool live = !SMALL || (wm == 0 && mb < 2);
      if (live) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            char* slot = smem + tile_off<32>(r, wn * 8 + nb * 4 + gq) + 8 * half;
            const f32x4 c = csv[nb * 4 + gq];
            const float sc = rsv[mb];
            float v0 = acc[mb][nb][4 * gq + 0] * sc * c[0], v1 = acc[mb][nb][4 * gq + 1] * sc * c[1];
            float v2 = acc[mb][nb][4 * gq + 2] * sc * c[2], v3 = acc[mb][nb][4 * gq + 3] * sc * c[3];
            if (MODE == MODE_RES_PRMS) {
              // the slot holds this lane's residual values; h replaces them in place
              const u32x2 r2 = *(const u32x2*)slot;
              v0 += bf16_lo(r2[0]);
              v1 += bf16_hi(r2[0]);
              v2 += bf16_lo(r2[1]);
              v3 += bf16_hi(r2[1]);
              s += v0 * v0;
              s += v1 * v1;
              s += v2 * v2;
              s += v3 * v3;
              if (WRITE_HG) {
                const f32x4 g = gv[nb][gq];
                const u32x2 hgw = {pack_bf16(v0 * g[0], v1 * g[1]), pack_bf16(v2 * g[2], v3 * g[3])};
                if (ONE_PASS)
                  *(u32x2*)(hg_stage + tile_off<32>(r, wn * 8 + nb * 4 + gq) + 8 * half) = hgw;
                else
                  hgv[mb][nb][gq] = hgw;
              }
            }
            *(u32x2*)slot = (u32x2){pack_bf16(v0, v1), pack_bf16(v2, v3)};
          }
      }
      ss[mb] = s;
    }
    if (!ONE_PASS) {
      __syncthreads();
      store_tile_rows<32, STAGED>(smem, out, Nb, m0, tn * BN, Mh);
    }
    if (MODE == MODE_RES_PRMS) {
      if (WRITE_HG && !ONE_PASS) {
        __syncthreads();
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int r = rowof(mb) + (lane & 31);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq)
              *(u32x2*)(smem + tile_off<32>(r, wn * 8 + nb * 4 + gq) + 8 * half) = hgv[mb][nb][gq];
        }
      }
      // lanes l and l+32 hold the same row: add their halves, then the four waves sharing the rows, in a
      // fixed order (no atomics: the partial sums are reproducible bit for bit)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) ss[mb] += __shfl_xor(ss[mb], 32);
      float* red = (float*)(smem + LDS_BYTES);  // [4 wn][256 rows], outside the staging area
      if (lane < 32) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) red[wn * 256 + rowof(mb) + lane] = ss[mb];
      }
      __syncthreads();
      if (ONE_PASS) store_tile_rows<32, STAGED>(smem, out, Nb, m0, tn * BN, Mh);
      if (WRITE_HG) {
        const char* hs = ONE_PASS ? hg_stage : smem;
        if (panels)
          store_tile_panels<32, STAGED>(hs, out2, (int64_t)M * 32, m0, tn * BN, M);
        else
          store_tile_rows<32, STAGED>(hs, out2, Nb, m0, tn * BN, M);
      }
      if (wn == 0 && lane < 32) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
          const int row = rowof(mb) + lane;
          const int m = m0 + row;
          if (m < M) part[(int64_t)tn * M + m] = ((red[row] + red[256 + row]) + red[512 + row]) + red[768 + row];
        }
      }
      if (FP8 && MX) {
        // a = bf16(h) * gamma in fp32 from the h tile still staged in LDS, quantised per 32-column block:
        // thread t takes block t % 8 of rows t / 8 + 64 p; codes (32 bytes) to out2 = hq [M, Nb], the block's
        // scale byte e + 127 to mxs (mx_scale_index layout)
        const int b = t & 7;
        const int col0 = tn * BN + 32 * b;
        float g[32];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const f32x4 v = *(const f32x4*)(gamma + col0 + 4 * i);
          g[4 * i] = v[0];
          g[4 * i + 1] = v[1];
          g[4 * i + 2] = v[2];
          g[4 * i + 3] = v[3];
        }
        uint8_t* hq = (uint8_t*)out2;
        const int tiles_m_k3 = (M + BM - 1) / BM;
#pragma unroll 1
        for (int p = 0; p < 4; ++p) {
          const int r = p * 64 + (t >> 3);
          const int m = m0 + r;
          float a[32];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4 w = *(const u32x4*)(smem + tile_off<32>(r, 4 * b + c));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a[8 * c + 2 * e] = bf16_lo(w[e]) * g[8 * c + 2 * e];
              a[8 * c + 2 * e + 1] = bf16_hi(w[e]) * g[8 * c + 2 * e + 1];
            }
          }
          float amax = 0.0f;
#pragma unroll
          for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(a[i]));
          const int e = mx_scale_exp(amax);
          const float inv = ldexpf(1.0f, -e);
          if (m < M) {
            u32x4 q[2];
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
              for (int w = 0; w < 4; ++w) {
                const float* v = a + 16 * h2 + 4 * w;
                q[h2][w] = pack_e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
              }
            uint8_t* dq = panels ? hq + (int64_t)(col0 >> 6) * M * 64 + (int64_t)m * 64 + (col0 & 63)
                                 : hq + (int64_t)m * Nb + col0;
            store_nt(dq, q[0]);
            store_nt(dq + 16, q[1]);
            mxs[mx_scale_index(col0 >> 6, tiles_m_k3, m, (col0 >> 5) & 1)] = (uint8_t)(e + 127);
          }
        }
      }
    }
  } else if (MODE == MODE_ROWSCALE_ROPE) {
    // a wave's 64 accumulator columns are one head: block 0 holds head columns 0..31, block 1 columns 32..63,
    // so the rotated pairs (i, i + 32) share a lane and a register index
    const int head0 = tn * BN + wn * 64;
    const bool rotate = head0 < rope.n_rot;
    float rev[4][4];
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int e = 0; e < 4; ++e) rev[gq][e] = half ? rope.rev[8 * gq + 4 + e] : rope.rev[8 * gq + e];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = rowof(mb) + (lane & 31);
      const int m = m0 + r;
      const float pos = (float)((m < M ? m : M - 1) % rope.seq_len);
      const float sc = rsv[mb];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = acc[mb][0][4 * gq + e] * sc, b = acc[mb][1][4 * gq + e] * sc;
          if (rotate) {
            float c, sn;
            rope_sincos(pos, rev[gq][e], c, sn);
            lo[e] = a * c - b * sn;
            hi[e] = b * c + a * sn;
          } else {
            lo[e] = a;
            hi[e] = b;
          }
        }
        *(u32x2*)(smem + tile_off<32>(r, wn * 8 + gq) + 8 * half) =
            (u32x2){pack_bf16(lo[0], lo[1]), pack_bf16(lo[2], lo[3])};
        *(u32x2*)(smem + tile_off<32>(r, wn * 8 + 4 + gq) + 8 * half) =
            (u32x2){pack_bf16(hi[0], hi[1]), pack_bf16(hi[2], hi[3])};
      }
    }
    __syncthreads();
    store_tile_rows<32>(smem, out, Nb, m0, tn * BN, Mh);
  } else {  // MODE_ROWSCALE_SWIGLU: accumulator block 0 holds gate columns, block 1 the matching up columns
    const int ny = Nb / 2;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int r = rowof(mb) + (lane & 31);
      const float sc = rsv[mb];
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float gate = acc[mb][0][4 * gq + e] * sc * csv[gq][e];
          const float up = acc[mb][1][4 * gq + e] * sc * csv[4 + gq][e];
          y[e] = silu_f32(gate) * up;
        }
        *(u32x2*)(smem + tile_off<16>(r, wn * 4 + gq) + 8 * half) =
            (u32x2){pack_bf16(y[0], y[1]), pack_bf16(y[2], y[3])};
      }
    }
    __syncthreads();
    store_tile_rows<16>(smem, out, ny, m0, tn * 128, Mh);
    if (out2) {
      // the pre-activation z = [gate | up] (bf16 [M, Nb]) for the backward: the tile's gate columns, then its up
      // columns, staged side by side once the y tile has left the staging area
      __syncthreads();
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const int r = rowof(mb) + (lane & 31);
        const float sc = rsv[mb];
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const f32x4 cg = csv[gq], cu = csv[4 + gq];
          float g[4], u[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            g[e] = acc[mb][0][4 * gq + e] * sc * cg[e];
            u[e] = acc[mb][1][4 * gq + e] * sc * cu[e];
          }
          *(u32x2*)(smem + tile_off<16>(r, wn * 4 + gq) + 8 * half) =
              (u32x2){pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3])};
          *(u32x2*)(smem + 65536 + tile_off<16>(r, wn * 4 + gq) + 8 * half) =
              (u32x2){pack_bf16(u[0], u[1]), pack_bf16(u[2], u[3])};
        }
      }
      __syncthreads();
      store_tile_rows<16>(smem, out2, Nb, m0, tn * 128, Mh);
      store_tile_rows<16>(smem + 65536, out2, Nb, m0, ny + tn * 128, Mh);
    }
  }
}

template <int MODE, bool FP8, bool MX = false, bool SMALL = false>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_epilogue_kernel(
    const void* __restrict__ A, const void* __restrict__ B, const float* __restrict__ gamma, const uint16_t* R,
    const float* __restrict__ rowsc, const float* __restrict__ colsc, uint16_t* out, uint16_t* __restrict__ out2,
    float* __restrict__ part, int M, int K, int Nb, int group_m, RopeParams rope, RowFold fold, uint8_t* mxs,
    int panels, KSplit ks) {
  gemm_epilogue_body<MODE, FP8, MX, SMALL, false>(A, B, gamma, R, rowsc, colsc, out, out2, part, M, K, Nb, group_m, rope, fold, mxs, panels, ks);
}

// The half-tile form of the bf16 row-scale modes: grid 2 (ntiles - ks.full), the tiles from ks.full on.
template <int MODE>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_epilogue_half_kernel(
    const void* __restrict__ A, const void* __restrict__ B, const float* __restrict__ gamma, const uint16_t* R,
    const float* __restrict__ rowsc, const float* __restrict__ colsc, uint16_t* out, uint16_t* __restrict__ out2,
    float* __restrict__ part, int M, int K, int Nb, int group_m, RopeParams rope, RowFold fold, uint8_t* mxs,
    int panels, KSplit ks) {
  gemm_epilogue_body<MODE, false, false, false, true>(A, B, gamma, R, rowsc, colsc, out, out2, part, M, K, Nb, group_m, rope, fold, mxs, panels, ks);
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


// wave-wide maximum (butterfly over the 64 lanes; every lane ends with the same value)
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

// K2 for e4m3 operands: one wave per row i.
//   r[i]     = 1 / sqrt((sum_t part[t][i]) / D + eps)    (t summed in order, as in prms_reduce_kernel)
//   a[i][j]  = h[i][j] * gamma[j] in fp32, h the stored bf16 value
//   s_a[i]   = amax_j |a[i][j]| / 448  (1 for an all-zero row)
//   hq[i][j] = e4m3(a[i][j] * (1 / s_a[i]))               (the second GEMM's A operand; the reciprocal is
//                                                          rounded to fp32 once per row)
//   rs2[i]   = s_a[i] * r[i]                               (the second GEMM's epilogue row scale)
// hq is written row-major, or with panels != 0 in K panels of 64 bytes ([D / 64][M][64]).
// Each lane keeps up to CACHED 8-column chunks of a[i] in registers between the amax and the quantisation
// (D <= 4096 reads h and gamma once); wider rows recompute the rest.
__global__ __launch_bounds__(256) void prms_reduce_quant_kernel(const float* __restrict__ part, int T, int M, int D,
                                                                float eps, const uint16_t* __restrict__ h,
                                                                const float* __restrict__ gamma,
                                                                uint8_t* __restrict__ hq, float* __restrict__ r,
                                                                float* __restrict__ sa, float* __restrict__ rs2,
                                                                int panels) {
  constexpr int CACHED = 8;
  const int lane = threadIdx.x & 63;
  const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (i >= M) return;  // whole waves only: the row index is uniform across the wave
  const uint16_t* row = h + i * D;
  const int nch = D / 8;
  auto scaled = [&](int c, float (&a)[8]) {
    const u32x4 v = *(const u32x4*)(row + 8 * c);
    const f32x4 g0 = *(const f32x4*)(gamma + 8 * c);
    const f32x4 g1 = *(const f32x4*)(gamma + 8 * c + 4);
    a[0] = bf16_lo(v[0]) * g0[0];
    a[1] = bf16_hi(v[0]) * g0[1];
    a[2] = bf16_lo(v[1]) * g0[2];
    a[3] = bf16_hi(v[1]) * g0[3];
    a[4] = bf16_lo(v[2]) * g1[0];
    a[5] = bf16_hi(v[2]) * g1[1];
    a[6] = bf16_lo(v[3]) * g1[2];
    a[7] = bf16_hi(v[3]) * g1[3];
  };
  float av[CACHED][8];
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < CACHED; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) {
      scaled(c, av[k]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(av[k][e]));
    }
  }
  for (int c = lane + 64 * CACHED; c < nch; c += 64) {
    float a[8];
    scaled(c, a);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(a[e]));
  }
  float ss = 0.0f;
  for (int t = 0; t < T; ++t) ss += part[(int64_t)t * M + i];
  const float ri = 1.0f / sqrtf(ss / (float)D + eps);
  amax = wave_max(amax);
  const float s = amax > 0.0f ? amax / E4M3_MAX : 1.0f;
  const float inv = 1.0f / s;
  uint8_t* qrow = hq + i * D;
  auto quant = [&](const float (&a)[8], int c) {
    u32x2 o;
    o[0] = pack_e4m3x4(a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv);
    o[1] = pack_e4m3x4(a[4] * inv, a[5] * inv, a[6] * inv, a[7] * inv);
    // panels: [D / 64][M][64] bytes (the second GEMM's stage width), else row-major
    uint8_t* dq = panels ? hq + (int64_t)((8 * c) >> 6) * M * 64 + i * 64 + ((8 * c) & 63) : qrow + 8 * c;
    store_nt(dq, o);
  };
#pragma unroll
  for (int k = 0; k < CACHED; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) quant(av[k], c);
  }
  for (int c = lane + 64 * CACHED; c < nch; c += 64) {
    float a[8];
    scaled(c, a);
    quant(a, c);
  }
  if (lane == 0) {
    r[i] = ri;
    sa[i] = s;
    rs2[i] = s * ri;
  }
}

// K2 for e4m3 operands where D <= 4096, two rows per wave: the same arithmetic per row as prms_reduce_quant_kernel
// (the same codes, scales and r bit for bit), with gamma loaded once per wave into registers (NC chunks of 8 columns
// per lane, NC * 512 >= D) and the second row's h loaded while the first row is reduced and quantised.  The first
// kernel re-read gamma (8 KiB) for every row: 15.2 -> 11.8 us at M = 8192, D = 2048.
template <int NC>
__global__ __launch_bounds__(256) void prms_reduce_quant_rows2_kernel(const float* __restrict__ part, int T, int M,
                                                                      int D, float eps,
                                                                      const uint16_t* __restrict__ h,
                                                                      const float* __restrict__ gamma,
                                                                      uint8_t* __restrict__ hq, float* __restrict__ r,
                                                                      float* __restrict__ sa, float* __restrict__ rs2,
                                                                      int panels) {
  const int lane = threadIdx.x & 63;
  const int64_t i0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 2;
  if (i0 >= M) return;  // whole waves only: the row index is uniform across the wave
  const int nch = D / 8;
  float g[NC][8];
  u32x4 hv[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = lane + 64 * k;
    if (c < nch) {
      const f32x4 g0 = *(const f32x4*)(gamma + 8 * c);
      const f32x4 g1 = *(const f32x4*)(gamma + 8 * c + 4);
      g[k][0] = g0[0]; g[k][1] = g0[1]; g[k][2] = g0[2]; g[k][3] = g0[3];
      g[k][4] = g1[0]; g[k][5] = g1[1]; g[k][6] = g1[2]; g[k][7] = g1[3];
      hv[k] = *(const u32x4*)(h + i0 * D + 8 * c);
    }
  }
#pragma unroll 1
  for (int rr = 0; rr < 2; ++rr) {
    const int64_t i = i0 + rr;
    if (i >= M) break;
    float ss = 0.0f;
    for (int t = 0; t < T; ++t) ss += part[(int64_t)t * M + i];
    float av[NC][8];
    float amax = 0.0f;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      if (lane + 64 * k < nch) {
        av[k][0] = bf16_lo(hv[k][0]) * g[k][0];
        av[k][1] = bf16_hi(hv[k][0]) * g[k][1];
        av[k][2] = bf16_lo(hv[k][1]) * g[k][2];
        av[k][3] = bf16_hi(hv[k][1]) * g[k][3];
        av[k][4] = bf16_lo(hv[k][2]) * g[k][4];
        av[k][5] = bf16_hi(hv[k][2]) * g[k][5];
        av[k][6] = bf16_lo(hv[k][3]) * g[k][6];
        av[k][7] = bf16_hi(hv[k][3]) * g[k][7];
#pragma unroll
        for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(av[k][e]));
      }
    }
    if (rr == 0 && i + 1 < M) {  // the next row's h, in flight while this row finishes
#pragma unroll
      for (int k = 0; k < NC; ++k)
        if (lane + 64 * k < nch) hv[k] = *(const u32x4*)(h + (i + 1) * D + 8 * (lane + 64 * k));
    }
    const float ri = 1.0f / sqrtf(ss / (float)D + eps);
    amax = wave_max(amax);
    const float s = amax > 0.0f ? amax / E4M3_MAX : 1.0f;
    const float inv = 1.0f / s;
#pragma unroll
    for (int k = 0; k < NC; ++k) {
      const int c = lane + 64 * k;
      if (c < nch) {
        u32x2 o;
        o[0] = pack_e4m3x4(av[k][0] * inv, av[k][1] * inv, av[k][2] * inv, av[k][3] * inv);
        o[1] = pack_e4m3x4(av[k][4] * inv, av[k][5] * inv, av[k][6] * inv, av[k][7] * inv);
        uint8_t* dq = panels ? hq + (int64_t)((8 * c) >> 6) * M * 64 + i * 64 + ((8 * c) & 63) : hq + i * D + 8 * c;
        store_nt(dq, o);
      }
    }
    if (lane == 0) {
      r[i] = ri;
      sa[i] = s;
      rs2[i] = s * ri;
    }
  }
}

// U2: one workgroup per row.  hf = T + R (fp32); h = bf16(hf); r = 1/sqrt(mean(hf^2) + eps);
// n = hf * r * gamma, stored as bf16 (QUANT = false) or, for e4m3 operands, quantised per row to
// e4m3(n / s_n) with s_n = amax |n| / 448 (QUANT = true; s_n goes to sn).  Each thread keeps up to 4
// chunks of 8 columns in registers (D <= 8192).
template <bool QUANT>
__global__ __launch_bounds__(256) void add_rmsnorm_kernel(const uint16_t* __restrict__ Tm, const uint16_t* R,
                                                          const float* __restrict__ gamma, uint16_t* H,
                                                          void* __restrict__ Nout, float* __restrict__ rout,
                                                          float* __restrict__ sn, int D, float eps) {
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
  float nv[MAXC][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + 256 * i;
    if (c < nchunks) {
      u32x4 ho;
      const float4 g0 = *(const float4*)(gamma + 8 * c);
      const float4 g1 = *(const float4*)(gamma + 8 * c + 4);
      const float gg[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) ho[q] = pack_bf16(hv[i][2 * q], hv[i][2 * q + 1]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        nv[i][e] = hv[i][e] * r * gg[e];
        amax = fmaxf(amax, fabsf(nv[i][e]));
      }
      store_nt(H + row * D + 8 * c, ho);
    }
  }
  float qs = 1.0f;
  if (QUANT) {
    __syncthreads();  // red[] is reused
    amax = wave_max(amax);
    if ((t & 63) == 0) red[t >> 6] = amax;
    __syncthreads();
    const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    qs = m > 0.0f ? m / E4M3_MAX : 1.0f;
    if (t == 0) sn[row] = qs;
  }
#pragma unroll
  for (int i = 0; i < MAXC; ++i) {
    const int c = t + 256 * i;
    if (c < nchunks) {
      if (QUANT) {
        u32x2 o;
        o[0] = pack_e4m3x4(nv[i][0] / qs, nv[i][1] / qs, nv[i][2] / qs, nv[i][3] / qs);
        o[1] = pack_e4m3x4(nv[i][4] / qs, nv[i][5] / qs, nv[i][6] / qs, nv[i][7] / qs);
        store_nt((uint8_t*)Nout + row * D + 8 * c, o);
      } else {
        u32x4 no;
#pragma unroll
        for (int q = 0; q < 4; ++q) no[q] = pack_bf16(nv[i][2 * q], nv[i][2 * q + 1]);
        store_nt((uint16_t*)Nout + row * D + 8 * c, no);
      }
    }
  }
}

// ------------------------------------------------------------------------------------------------------
// launchers (host)

static int group_m_for(int tiles_m) { return tiles_m < 4 ? tiles_m : 4; }

template <int MODE, bool FP8, bool MX = false>
static hipError_t launch_gemm(const void* A, const void* B, const float* gamma, const uint16_t* R, const float* rowsc,
                              const float* colsc, uint16_t* out, uint16_t* out2, float* part, int M, int K, int Nb,
                              hipStream_t stream, RopeParams rope = RopeParams{}, RowFold fold = RowFold{},
                              uint8_t* mxs = nullptr, int panels = 0, KSplit ks = KSplit{}) {
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = Nb / BN;
  const int ntiles = tiles_m * tiles_n;
  constexpr KSplitRule rule = FP8 ? KSPLIT_E4M3 : KSPLIT_BF16;
  static_assert(rule.gran == (FP8 ? K8_MULTIPLE : K_MULTIPLE), "the split's K granule is one ring fill");
  dim3 block(NTHREADS);
  constexpr bool ROWSCALE_MODE = MODE == MODE_ROWSCALE || MODE == MODE_ROWSCALE_SWIGLU || MODE == MODE_ROWSCALE_ROPE;
  if constexpr (!FP8 && ROWSCALE_MODE) {
    if (ks.halves && ks.full >= 0 && ks.full < ntiles && M > SMALL_MAX_ROWS) {
      // the whole tiles (a grid of `full`: tile_coords_split deals them all as whole tiles), then the last wave's tiles
      // as 128-row halves in a launch of their own
      KSplit whole;
      whole.full = ks.full;
      if (ks.full > 0) {
        hipLaunchKernelGGL((gemm_epilogue_kernel<MODE, false, MX>), dim3(ks.full), block, 0, stream, A, B, gamma, R,
                           rowsc, colsc, out, out2, part, M, K, Nb, group_m_for(tiles_m), rope, fold, mxs, panels, whole);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      hipLaunchKernelGGL((gemm_epilogue_half_kernel<MODE>), dim3(2 * (ntiles - ks.full)), block, 0, stream, A, B, gamma,
                         R, rowsc, colsc, out, out2, part, M, K, Nb, group_m_for(tiles_m), rope, fold, mxs, panels,
                         whole);
      return hipGetLastError();
    }
  }
  if (ks.halves) ks.full = -1;  // other kernels (or shapes) run whole tiles
  int nwg = ntiles;
  if (ks.full >= 0 && ks.full < ntiles && ks.part && ks.cnt && ks.lg >= 1 && ks.lg <= KSPLIT_MAX_LG &&
      K % (rule.gran << ks.lg) == 0 && (K >> ks.lg) >= rule.min_piece)
    nwg = ks.full + ((ntiles - ks.full) << ks.lg);
  else
    ks.full = -1;  // nothing to split, or a split this kernel or K cannot take: whole tiles
  dim3 grid(nwg);
  if constexpr (!FP8) {
    if (M <= SMALL_MAX_ROWS) {  // the small-row form: a quarter of the MFMAs per SIMD
      hipLaunchKernelGGL((gemm_epilogue_kernel<MODE, FP8, MX, true>), grid, block, 0, stream, A, B, gamma, R, rowsc,
                         colsc, out, out2, part, M, K, Nb, group_m_for(tiles_m), rope, fold, mxs, panels, ks);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_epilogue_kernel<MODE, FP8, MX>), grid, block, 0, stream, A, B, gamma, R, rowsc, colsc, out,
                     out2, part, M, K, Nb, group_m_for(tiles_m), rope, fold, mxs, panels, ks);
  return hipGetLastError();
}

KSplit halves_plan(int64_t ntiles, int64_t M, int cus) {
  KSplit ks;
  if (cus <= 0 || ntiles <= 0 || M <= SMALL_MAX_ROWS) return ks;
  const int64_t rem = ntiles % cus, tail_rows = M % BM;
  if (rem == 0 || 2 * rem > cus || (tail_rows != 0 && tail_rows <= 128)) return ks;
  ks.full = (int)(ntiles - rem);
  ks.halves = 1;
  return ks;
}

__global__ __launch_bounds__(256) void clear_tickets_kernel(int* __restrict__ cnt, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) cnt[i] = 0;
}

hipError_t launch_clear_tickets(int* cnt, int n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(clear_tickets_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, cnt, n);
  return hipGetLastError();
}

int ksplit_plan(int64_t ntiles, int64_t K, int cus, int fp8, int* lg) {
  const KSplitRule& u = fp8 ? KSPLIT_E4M3 : KSPLIT_BF16;
  *lg = 0;
  if (cus <= 0 || ntiles <= 0) return (int)ntiles;
  const int64_t rem = ntiles % cus;
  if (rem == 0) return (int)ntiles;
  // a last wave of at most cus / tail_den tiles, or of at most three eighths of the CUs where K >= long_k
  if (u.tail_den * rem > cus && !(8 * rem <= 3 * cus && K >= u.long_k)) return (int)ntiles;
  if (K % (2 * u.gran) || K / 2 < u.min_piece) return (int)ntiles;  // two pieces of at least min_piece
  int g = 1;  // more pieces while they stay within half of the CUs and each keeps tree_piece of K
  while (g < KSPLIT_MAX_LG && 2 * (rem << (g + 1)) <= cus && K % ((int64_t)u.gran << (g + 1)) == 0 &&
         (K >> (g + 1)) >= u.tree_piece)
    ++g;
  *lg = g;
  return (int)(ntiles - rem);
}

hipError_t launch_gemm1_res_prms(const uint16_t* X, const uint16_t* W1, const uint16_t* R, const float* gamma,
                                 uint16_t* H, uint16_t* HG, float* part, int M, int K1, int D, hipStream_t stream,
                                 int panels, KSplit ks) {
  return launch_gemm<MODE_RES_PRMS, false>(X, W1, gamma, R, nullptr, nullptr, H, HG, part, M, K1, D, stream,
                                           RopeParams{}, RowFold{}, nullptr, panels, ks);
}

hipError_t launch_gemm1_res_prms_fp8(const uint8_t* Xq, const float* sx, const uint8_t* W1q, const float* sw1,
                                     const uint16_t* R, uint16_t* H, float* part, int M, int K1, int D,
                                     hipStream_t stream, KSplit ks) {
  return launch_gemm<MODE_RES_PRMS, true>(Xq, W1q, nullptr, R, sx, sw1, H, nullptr, part, M, K1, D, stream,
                                          RopeParams{}, RowFold{}, nullptr, 0, ks);
}

hipError_t launch_gemm1_res_prms_fp8_mx(const uint8_t* Xq, const float* sx, const uint8_t* W1q, const float* sw1,
                                        const uint16_t* R, const float* gamma, uint16_t* H, uint8_t* HQ, uint8_t* HS,
                                        float* part, int M, int K1, int D, hipStream_t stream, int panels,
                                        KSplit ks) {
  return launch_gemm<MODE_RES_PRMS, true, true>(Xq, W1q, gamma, R, sx, sw1, H, (uint16_t*)HQ, part, M, K1, D, stream,
                                                RopeParams{}, RowFold{}, HS, panels, ks);
}

hipError_t launch_gemm2_rowscale_fp8_mx(const uint8_t* HQ, const uint8_t* HS, const uint8_t* W2q, const float* sw2,
                                        const float* r_in, const float* part, float eps, float* r_out, int swiglu,
                                        uint16_t* Y, int M, int D, int N2, hipStream_t stream, int panels,
                                        KSplit ks) {
  const RowFold f = part ? RowFold{D / BN, (float)D, eps, r_out} : RowFold{};
  if (swiglu)
    return launch_gemm<MODE_ROWSCALE_SWIGLU, true, true>(HQ, W2q, nullptr, nullptr, part ? nullptr : r_in, sw2, Y,
                                                         nullptr, (float*)part, M, D, N2, stream, RopeParams{}, f,
                                                         (uint8_t*)HS, panels, ks);
  return launch_gemm<MODE_ROWSCALE, true, true>(HQ, W2q, nullptr, nullptr, part ? nullptr : r_in, sw2, Y, nullptr,
                                                (float*)part, M, D, N2, stream, RopeParams{}, f, (uint8_t*)HS, panels,
                                                ks);
}

hipError_t launch_prms_reduce(const float* part, int T, int M, int D, float eps, float* r, hipStream_t stream) {
  dim3 grid((M + 255) / 256), block(256);
  hipLaunchKernelGGL(prms_reduce_kernel, grid, block, 0, stream, part, T, M, (float)D, eps, r);
  return hipGetLastError();
}

hipError_t launch_prms_reduce_quant(const float* part, int T, int M, int D, float eps, const uint16_t* H,
                                    const float* gamma, uint8_t* HQ, float* r, float* sa, float* rs2,
                                    hipStream_t stream, int panels) {
  const int nc = (D / 8 + 63) / 64;  // 8-column chunks per lane
  if (nc <= 8) {
    dim3 grid((M + 7) / 8), block(256);
#define CODA_Q2(N) hipLaunchKernelGGL(prms_reduce_quant_rows2_kernel<N>, grid, block, 0, stream, part, T, M, D, eps, H, \
                                      gamma, HQ, r, sa, rs2, panels)
    if (nc <= 1) CODA_Q2(1);
    else if (nc <= 2) CODA_Q2(2);
    else if (nc <= 4) CODA_Q2(4);
    else CODA_Q2(8);
#undef CODA_Q2
    return hipGetLastError();
  }
  dim3 grid((M + 3) / 4), block(256);
  hipLaunchKernelGGL(prms_reduce_quant_kernel, grid, block, 0, stream, part, T, M, D, eps, H, gamma, HQ, r, sa, rs2,
                     panels);
  return hipGetLastError();
}

hipError_t launch_gemm2_rowscale(const uint16_t* A, const uint16_t* W2, const float* r, int swiglu, uint16_t* Y,
                                 int M, int D, int N2, hipStream_t stream, uint16_t* Z, int panels, KSplit ks) {
  if (swiglu)
    return launch_gemm<MODE_ROWSCALE_SWIGLU, false>(A, W2, nullptr, nullptr, r, nullptr, Y, Z, nullptr, M, D, N2,
                                                    stream, RopeParams{}, RowFold{}, nullptr, panels, ks);
  return launch_gemm<MODE_ROWSCALE, false>(A, W2, nullptr, nullptr, r, nullptr, Y, nullptr, nullptr, M, D, N2, stream,
                                           RopeParams{}, RowFold{}, nullptr, panels, ks);
}

int fold_supported(int D) { return D / BN <= FOLD_MAX_T; }

hipError_t launch_gemm2_rowscale_fold(const uint16_t* A, const uint16_t* W2, const float* part, float eps, float* r,
                                      int swiglu, uint16_t* Y, int M, int D, int N2, hipStream_t stream,
                                      uint16_t* Z, int panels, KSplit ks) {
  const RowFold f{D / BN, (float)D, eps, r};
  if (swiglu)
    return launch_gemm<MODE_ROWSCALE_SWIGLU, false>(A, W2, nullptr, nullptr, nullptr, nullptr, Y, Z,
                                                    (float*)part, M, D, N2, stream, RopeParams{}, f, nullptr, panels,
                                                    ks);
  return launch_gemm<MODE_ROWSCALE, false>(A, W2, nullptr, nullptr, nullptr, nullptr, Y, nullptr, (float*)part, M, D,
                                           N2, stream, RopeParams{}, f, nullptr, panels, ks);
}

static RopeParams rope_params(int seq_len, int n_rot, float base) {
  RopeParams p;
  p.seq_len = seq_len;
  p.n_rot = n_rot;
  for (int i = 0; i < 32; ++i) p.rev[i] = (float)(pow((double)base, -(double)(2 * i) / 64.0) / (2.0 * M_PI));
  return p;
}

hipError_t launch_gemm2_rowscale_rope(const uint16_t* A, const uint16_t* W2, const float* r, int seq_len, int n_rot,
                                      float base, uint16_t* Y, int M, int D, int N2, hipStream_t stream,
                                      int panels, KSplit ks) {
  return launch_gemm<MODE_ROWSCALE_ROPE, false>(A, W2, nullptr, nullptr, r, nullptr, Y, nullptr, nullptr, M, D, N2,
                                                stream, rope_params(seq_len, n_rot, base), RowFold{}, nullptr,
                                                panels, ks);
}

hipError_t launch_gemm2_rowscale_rope_fold(const uint16_t* A, const uint16_t* W2, const float* part, float eps,
                                           float* r, int seq_len, int n_rot, float base, uint16_t* Y, int M, int D,
                                           int N2, hipStream_t stream, int panels, KSplit ks) {
  return launch_gemm<MODE_ROWSCALE_ROPE, false>(A, W2, nullptr, nullptr, nullptr, nullptr, Y, nullptr, (float*)part,
                                                M, D, N2, stream, rope_params(seq_len, n_rot, base),
                                                RowFold{D / BN, (float)D, eps, r}, nullptr, panels, ks);
}

// Standalone rotary embedding, in place on bf16 Y [M,N] (the unfused counterpart): one thread per pair.
__global__ __launch_bounds__(256) void rope_rows_kernel(uint16_t* Y, int M, int N, RopeParams rope) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int pairs = rope.n_rot / 2;
  if (idx >= (int64_t)M * pairs) return;
  const int m = (int)(idx / pairs), p = (int)(idx % pairs);
  const int head = p / 32, i = p % 32;
  float c, sn;
  rope_sincos((float)(m % rope.seq_len), rope.rev[i], c, sn);
  uint16_t* row = Y + (int64_t)m * N + head * 64;
  const float a = __uint_as_float((uint32_t)row[i] << 16), b = __uint_as_float((uint32_t)row[i + 32] << 16);
  const uint32_t o = pack_bf16(a * c - b * sn, b * c + a * sn);
  row[i] = (uint16_t)(o & 0xffff);
  row[i + 32] = (uint16_t)(o >> 16);
}

hipError_t launch_rope_rows(uint16_t* Y, int M, int N, int seq_len, int n_rot, float base, hipStream_t stream) {
  const int64_t n = (int64_t)M * (n_rot / 2);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, Y, M, N,
                     rope_params(seq_len, n_rot, base));
  return hipGetLastError();
}

hipError_t launch_gemm2_rowscale_fp8(const uint8_t* Aq, const uint8_t* W2q, const float* rowsc, const float* sw2,
                                     int swiglu, uint16_t* Y, int M, int D, int N2, hipStream_t stream, int panels,
                                     KSplit ks) {
  if (swiglu)
    return launch_gemm<MODE_ROWSCALE_SWIGLU, true>(Aq, W2q, nullptr, nullptr, rowsc, sw2, Y, nullptr, nullptr, M, D,
                                                   N2, stream, RopeParams{}, RowFold{}, nullptr, panels, ks);
  return launch_gemm<MODE_ROWSCALE, true>(Aq, W2q, nullptr, nullptr, rowsc, sw2, Y, nullptr, nullptr, M, D, N2, stream,
                                          RopeParams{}, RowFold{}, nullptr, panels, ks);
}

hipError_t launch_gemm_store(const uint16_t* X, const uint16_t* W, uint16_t* T, int M, int K, int N,
                             hipStream_t stream, int a_panels, KSplit ks) {
  return launch_gemm<MODE_STORE, false>(X, W, nullptr, nullptr, nullptr, nullptr, T, nullptr, nullptr, M, K, N, stream,
                                        RopeParams{}, RowFold{}, nullptr, a_panels, ks);
}

hipError_t launch_gemm_store_fp8(const uint8_t* Xq, const float* sx, const uint8_t* Wq, const float* sw, uint16_t* T,
                                 int M, int K, int N, hipStream_t stream, KSplit ks) {
  return launch_gemm<MODE_STORE, true>(Xq, Wq, nullptr, nullptr, sx, sw, T, nullptr, nullptr, M, K, N, stream,
                                       RopeParams{}, RowFold{}, nullptr, 0, ks);
}

hipError_t launch_add_rmsnorm(const uint16_t* T, const uint16_t* R, const float* gamma, uint16_t* H, uint16_t* N,
                              float* r, int M, int D, float eps, hipStream_t stream) {
  dim3 grid(M), block(256);
  hipLaunchKernelGGL(add_rmsnorm_kernel<false>, grid, block, 0, stream, T, R, gamma, H, (void*)N, r, (float*)nullptr,
                     D, eps);
  return hipGetLastError();
}

hipError_t launch_add_rmsnorm_quant(const uint16_t* T, const uint16_t* R, const float* gamma, uint16_t* H,
                                    uint8_t* NQ, float* r, float* sn, int M, int D, float eps, hipStream_t stream) {
  dim3 grid(M), block(256);
  hipLaunchKernelGGL(add_rmsnorm_kernel<true>, grid, block, 0, stream, T, R, gamma, H, (void*)NQ, r, sn, D, eps);
  return hipGetLastError();
}

}  // namespace coda
