// gemm_core.h -- bf16 MFMA GEMM mainloop for gfx950 (CDNA4) shared by the block's GEMMs.
//
// The CODA write-up ("CODA: new research optimizes Transformer training with GEMM-epilogue programming",
// section "CODA: the treasure hidden in the epilogue") splits a GEMM into a mainloop (tiled
// multiply-accumulate) and an epilogue (finishing work done while the output tile is still in registers).
// This file is the mainloop; the epilogues live with the kernels.
//
// Tiling: one workgroup of 8 waves (512 lanes, two waves per SIMD) computes a 256 x 256 tile.  Wave w owns
// rows 128 (w % 2) .. +128 and columns 64 (w / 2) .. +64 as 4 x 2 blocks of 32 x 32 fp32 accumulators
// (128 registers per lane).
//
// Operands: A [M,K] row-major (K contiguous), or in K panels of the stage width (ALayout below); B [K,N]
// row-major (N contiguous), the layout weights are stored in.  K advances 32 at a time through a ring of 4 LDS
// stages (4 x 32 KiB): stage k+3 is fetched
// while stage k is multiplied, with global_load_lds_dwordx4 (global memory straight into LDS, no VGPR
// staging), so each tile's loads have three K steps of latency budget.  One barrier per K step, placed
// half-way so that the next step's first fragments are read from LDS while the current step's last
// MFMAs run.  The barrier carries no memory fence: the wait is an explicit vmcnt for the stage about to be
// read, which keeps the later stages' loads in flight.  As the ring drains in the last K steps, the freed
// stages can take the epilogue's own operand tile (the drain hook).
//
// B stays N-contiguous in LDS and is read K-contiguous with ds_read_b64_tr_b16 (the gfx950 transposing
// LDS read), so the weights need no transpose pass.  The MFMA (v_mfma_f32_32x32x16_bf16) takes the B
// fragment as its first operand and the A fragment as its second, which yields the transposed tile: each
// lane owns output rows, so row-wise epilogue work (sums of squares, the row scale) stays inside a lane.
//
// LDS swizzles (verified conflict-free with the SQ_LDS_BANK_CONFLICT counter): A rows are 64 bytes, chunk
// c of row r sits at slot c ^ ((r / 4) % 4); B rows are 512 bytes, chunk c of row k at c ^ 4 (k % 4).
//
// Lane layouts (verified on the device):
//   v_mfma_f32_32x32x16_bf16(a, b, c): a lane l holds a[row l%32][k 8(l/32)+e], b lane l holds
//   b[k 8(l/32)+e][col l%32]; result register r of lane l is c[row 8(r/4)+4(l/32)+r%4][col l%32].
//   ds_read_b64_tr_b16: inside each group of 16 lanes, element e of lane i is element i%4 of the 8 bytes
//   addressed by lane 4e + i/4 of the group.
//   global_load_lds_dwordx4: lane i's 16 bytes land at the wave-uniform LDS base + 16 i.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace coda {

typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256;            // rows of a workgroup tile
constexpr int BN = 256;            // accumulator columns of a workgroup tile
constexpr int BK = 32;             // K per stage
constexpr int NSTAGE = 4;          // LDS ring depth
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int NB = 2;              // 32-column accumulator blocks per wave
constexpr int A_BYTES = BM * BK * 2;      // 16 KiB
constexpr int B_BYTES = BK * BN * 2;      // 16 KiB
constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
constexpr int LDS_BYTES = NSTAGE * STAGE_BYTES;  // 128 KiB
constexpr int K_MULTIPLE = BK * NSTAGE;           // K must be a multiple of this

// ---- small conversions ------------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), lo in the low half
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// ---- LDS layout -------------------------------------------------------------------------------------
__device__ __forceinline__ int a_off(int r, int c) { return r * 64 + ((c ^ ((r >> 2) & 3)) << 4); }
__device__ __forceinline__ int b_off(int k, int c) { return k * 512 + ((c ^ ((k & 3) << 2)) << 4); }

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ s16x4 lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}
// 16 bytes per lane from global memory into LDS at the wave-uniform base + 16 * lane
__device__ __forceinline__ void g2lds16(const void* g, char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)lds_wave_base, 16, 0, 0);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] + vmcnt_hi[15:14], expcnt[6:4], lgkmcnt[11:8]),
// then a workgroup barrier the compiler may not move memory operations across.
template <int N>
__device__ __forceinline__ void wait_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
  asm volatile("s_barrier" ::: "memory");
}

struct Frags {
  s16x8 a[4];   // A rows mb*32 .. +32 of the wave, 8 K values per lane
  s16x8 b[NB];  // B columns nb*32 .. +32 of the wave, 8 K values per lane
};

// Per-lane LDS offsets of the fragments inside a stage (sub-step s of 16 K values adds immediates).
struct LaneOffs {
  int a[2];
  int b[NB];
};

// HALF: the half-tile form (gemm_mainloop), where wave row block wm covers rows 64 wm .. +64.
template <bool HALF = false>
__device__ __forceinline__ void lane_offsets(int wm, int wn, int lane, LaneOffs& o) {
  const int q = lane >> 4, j = lane & 15;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // lane j of 16-lane group q points at row k0 + j/4, columns n0 + 4 (j%4) .. +3, so that after the
    // transposing read lane i of the group holds rows k0..k0+3 of column n0 + i
    const int n0 = wn * (32 * NB) + nb * 32 + 16 * (q & 1);
    const int krow = 8 * (q >> 1) + (j >> 2);
    const int piece = (n0 >> 2) + (j & 3);  // 8-byte piece within the 512-byte row
    o.b[nb] = A_BYTES + b_off(krow, piece >> 1) + ((piece & 1) << 3);
  }
  const int m = wm * (HALF ? 64 : 128) + (lane & 31);
#pragma unroll
  for (int s = 0; s < 2; ++s) o.a[s] = a_off(m, 2 * s + (lane >> 5));
}

// RB: the wave's 32-row blocks that are computed (4; 2 in the small-row and half-tile forms)
template <int RB = 4>
__device__ __forceinline__ void read_frags(const char* st, const LaneOffs& o, int s, Frags& f) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const char* p = st + o.b[nb] + s * (16 * 512);
    const s16x4 lo = lds_read_tr16(p);
    const s16x4 hi = lds_read_tr16(p + 4 * 512);  // rows k0+4..k0+7 share the swizzle of rows k0..k0+3
    f.b[nb] = (s16x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
#pragma unroll
  for (int mb = 0; mb < RB; ++mb) f.a[mb] = *(const s16x8*)(st + o.a[s] + mb * 32 * 64);
}

template <int RB = 4>
__device__ __forceinline__ void mma(const Frags& f, f32x16 (&acc)[4][NB]) {
#pragma unroll
  for (int mb = 0; mb < RB; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, f.b[nb]),
                                                           __builtin_bit_cast(bf16x8, f.a[mb]), acc[mb][nb], 0, 0, 0);
}

// The wave's place in the tile: rows 128 wm .. +128, columns 64 wn .. +64.  The 2 x 4 layout puts the two waves of a
// SIMD (waves w and w + 4) on the same rows.  The small-row form (tiles of at most 64 rows, SMALL) puts them on the
// same columns instead, so that each SIMD holds one wave of rows 0 .. 127: those waves compute the tile's first two
// 32-row blocks, the waves of rows 128 .. 255 no product at all, and each SIMD runs a quarter of the MFMAs.
template <bool SMALL = false>
__device__ __forceinline__ void wave_pos(int wave, int& wm, int& wn) {
  wm = SMALL ? wave >> 2 : wave & 1;
  wn = SMALL ? wave & 3 : wave >> 1;
}
constexpr int SMALL_MAX_ROWS = 64;

// Interleave the 8 MFMAs of a sub-step one-to-one with the 8 LDS reads of the next fragments.
__device__ __forceinline__ void interleave_mma_reads() {
#pragma unroll
  for (int i = 0; i < 4 + 2 * NB; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
  }
}

// Where the A operand's K steps live.  Element (m, k) of A sits at m * row + (k / S) * step + k % S, S being
// the mainloop's K per stage (32 bf16 values, 64 e4m3 bytes).  Row-major A [M,K] has row = its row stride and
// step = S.  A written in K panels [K / S][M][S] has row = S and step = M * S: then a stage's A tile (256 rows
// of one panel) is one contiguous block and every direct load covers whole 128-byte cache lines, where the
// row-major tile's 64-byte row pieces each take a line of their own through the L1 (measured: 5-8% off the
// product's time at the 1B GEMM2 shape).
struct ALayout {
  int64_t row;
  int64_t step;
};

// The mainloop: acc = A[m0:m0+256, :] * B[:, tile columns] over the full K (K % K_MULTIPLE == 0).
//   A: [M,K] bf16 laid out as `al` says; rows >= M are read as row M-1 (their results are never stored).
//   B: [K,*] bf16, row stride ldb.  bcol(c) gives the global column of the tile's 8-column chunk c
//      (0..31), which lets a tile gather column segments (the gate | up halves of SwiGLU).
struct NoHook {
  __device__ void operator()() const {}
};

// hook() runs once, after the first stage has landed and every wave has passed the barrier: global loads (or
// global -> LDS loads) issued before the mainloop have completed by then.  It must issue no global memory
// operation of its own (the mainloop's wait counts assume its own loads only).
//
// drain(s) lets the epilogue's own operands start to arrive while the last K steps run: it is called for
// s = 0, 1, 2 right after the barrier behind which every wave has finished reading ring stage s for the last
// time (in the last four K steps), and may fill that stage's STAGE_BYTES with direct loads; it must issue
// exactly Drain::LOADS vector memory instructions per wave, which the remaining waits count.  Stage 3 is read
// until the mainloop returns; the caller waits for the drain's loads (vmcnt) and synchronises the workgroup.
struct NoDrain {
  static constexpr int LOADS = 0;
  __device__ void operator()(int) const {}
};
// SMALL: the small-row form (at most SMALL_MAX_ROWS rows; wave_pos): every wave fetches and waits as usual, the
// waves of rows 128 .. 255 skip the fragment reads and MFMAs, the others compute their first two row blocks only
// (the other accumulators stay zero).
// HALF: the half-tile form, a 128 x 256 tile (rows m0 .. m0+127) on the same eight waves: each wave computes two
// row blocks, rows 64 wm .. +64 (lane_offsets), the A stage holds 128 rows (one direct load per wave and stage) and
// acc[2], acc[3] stay zero.  Each output is the same chain of MFMAs over K as in the full tile, so the results are
// the same bit for bit.
template <class BCol, class Hook = NoHook, class Drain = NoDrain, bool SMALL = false, bool HALF = false>
__device__ __forceinline__ void gemm_mainloop(const uint16_t* __restrict__ A, ALayout al, int M, int m0,
                                              const uint16_t* __restrict__ B, int64_t ldb, BCol bcol, int K,
                                              char* smem, f32x16 (&acc)[4][NB], Hook hook = Hook{},
                                              Drain drain = Drain{}, std::integral_constant<bool, SMALL> = {},
                                              std::integral_constant<bool, HALF> = {}) {
  static_assert(!(SMALL && HALF), "one row form at a time");
  constexpr int LPW = 16 / NWAVES;              // 1 KiB direct loads per wave per operand per stage
  constexpr int LPA = HALF ? LPW / 2 : LPW;     // the A operand's (128 rows in the half-tile form)
  constexpr int PER = LPA + LPW;  // VMEM instructions per wave per stage
  constexpr int RB = (SMALL || HALF) ? 2 : 4;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  int wm, wn;
  wave_pos<SMALL>(wave, wm, wn);
  const bool computes = !SMALL || wm == 0;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = (f32x16){};

  // Direct-load unit q (1 KiB) of a stage: A rows 16q .. 16q+15 (lane -> row 16q + lane/4, slot lane%4),
  // B rows 2q, 2q+1 (lane -> row 2q + lane/32, slot lane%32).  Each lane fetches the logical chunk that
  // the swizzle places in its slot.  Wave w issues A units LPA w .. and B units LPW w .. .
  const uint16_t* aptr[LPW];
  const uint16_t* bptr[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int q = LPW * wave + i;
    const int r = 16 * (LPA * wave + i) + (lane >> 2);  // only i < LPA is issued
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int row = m0 + r;
    row = row < M ? row : M - 1;
    aptr[i] = A + (int64_t)row * al.row + 8 * c;
    const int kr = 2 * q + (lane >> 5);
    const int cb = (lane & 31) ^ ((kr & 3) << 2);
    bptr[i] = B + (int64_t)kr * ldb + bcol(cb);
  }
  LaneOffs lo;
  lane_offsets<HALF>(wm, wn, lane, lo);
  const int nk = K / BK;

  auto issue = [&](int kt, int stage) {
    char* st = smem + stage * STAGE_BYTES;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LPA; ++i) g2lds16(aptr[i] + (int64_t)kt * al.step, st + (LPA * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < LPW; ++i) g2lds16(bptr[i] + (int64_t)k0 * ldb, st + A_BYTES + (LPW * wave + i) * 1024);
  };

  Frags f0, f1;
  // One K step on stage U.  ISSUE: fetch tile kt+3 into the stage tile kt-1 used (every wave has passed
  // the barrier that followed its last read of it).  WAIT >= 0: the vmcnt that guarantees tile kt+1 has
  // landed, then the barrier and the first fragments of tile kt+1; WAIT < 0: the last tile.  DRAIN >= 0:
  // drain(DRAIN) after the barrier (stage U is then free).
  auto step = [&](int kt, auto U_c, auto issue_c, auto wait_c, auto drain_c) {
    constexpr int U = decltype(U_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr int WAIT = decltype(wait_c)::value;
    constexpr int DRAIN = decltype(drain_c)::value;
    const char* cur = smem + U * STAGE_BYTES;
    if (ISSUE) issue(kt + NSTAGE - 1, (U + NSTAGE - 1) % NSTAGE);
    if (computes) {
      read_frags<RB>(cur, lo, 1, f1);
      mma<RB>(f0, acc);
      if (RB == 4) interleave_mma_reads();
    }
    if (WAIT >= 0) {
      wait_barrier<(WAIT < 0 ? 0 : WAIT)>();
      if (DRAIN >= 0 && Drain::LOADS > 0) drain(DRAIN);
      if (computes) read_frags<RB>(smem + ((U + 1) % NSTAGE) * STAGE_BYTES, lo, 0, f0);
    }
    if (computes) {
      mma<RB>(f1, acc);
      if (RB == 4) interleave_mma_reads();
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  using WaitFull = std::integral_constant<int, 2 * PER>;
  static_assert(NSTAGE == 4, "the step sequence below is written for four stages");

  // prologue: tiles 0..2 in flight, wait for tile 0
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) issue(p, p);
  wait_barrier<2 * PER>();
  hook();
  if (computes) read_frags<RB>(smem, lo, 0, f0);

  using NoD = std::integral_constant<int, -1>;
  constexpr int DL = Drain::LOADS;
  static_assert(PER + DL < 64 && 2 * DL < 64, "vmcnt range");
  const int nblk = nk / NSTAGE;
  for (int bi = 0; bi < nblk - 1; ++bi) {
    const int kt = bi * NSTAGE;
    step(kt + 0, S0{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 1, S1{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 2, S2{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 3, S3{}, Yes{}, WaitFull{}, NoD{});
  }
  // last block: only its first step fetches (the last tile); the waits shrink as the ring drains, and count
  // the drain's loads issued after the stage loads they wait for
  const int kt = (nblk - 1) * NSTAGE;
  step(kt + 0, S0{}, Yes{}, std::integral_constant<int, 2 * PER>{}, S0{});
  step(kt + 1, S1{}, No{}, std::integral_constant<int, PER + DL>{}, S1{});
  step(kt + 2, S2{}, No{}, std::integral_constant<int, 2 * DL>{}, S2{});
  step(kt + 3, S3{}, No{}, std::integral_constant<int, -1>{}, NoD{});
}

// The same mainloop with B given transposed: Bt [N,K] with K contiguous (a weight read as [out,in], or W^T of
// an [in,out] weight).  The B stage then has the A stage's layout (tile row = output column, 64-byte rows,
// the same swizzle) and is read with ds_read_b128 like A.  brow(r) = global row of Bt that feeds tile-local
// output column r (0..255).
template <class BRow, class Drain = NoDrain>
__device__ __forceinline__ void gemm_mainloop_nt(const uint16_t* __restrict__ A, int64_t lda, int M, int m0,
                                                 const uint16_t* __restrict__ Bt, int64_t ldbt, BRow brow, int K,
                                                 char* smem, f32x16 (&acc)[4][NB], Drain drain = Drain{}) {
  constexpr int LPW = 16 / NWAVES;
  constexpr int PER = 2 * LPW;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = (f32x16){};
  // direct-load unit q: rows 16q .. 16q+15 of both stages (lane -> row 16q + lane/4, slot lane%4)
  const uint16_t* aptr[LPW];
  const uint16_t* bptr[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int q = LPW * wave + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int row = m0 + r;
    row = row < M ? row : M - 1;
    aptr[i] = A + (int64_t)row * lda + 8 * c;
    bptr[i] = Bt + brow(r) * ldbt + 8 * c;
  }
  // per-lane fragment offsets: sub-step s reads chunk 2 s + lane/32 of its row
  int oa[2], ob[2][NB];
  {
    const int m = wm * 128 + (lane & 31);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      oa[s] = a_off(m, 2 * s + (lane >> 5));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        ob[s][nb] = A_BYTES + a_off(wn * (32 * NB) + nb * 32 + (lane & 31), 2 * s + (lane >> 5));
    }
  }
  auto rd = [&](const char* st, int s, Frags& f) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) f.b[nb] = *(const s16x8*)(st + ob[s][nb]);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) f.a[mb] = *(const s16x8*)(st + oa[s] + mb * 32 * 64);
  };
  const int nk = K / BK;
  auto issue = [&](int kt, int stage) {
    char* st = smem + stage * STAGE_BYTES;
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < LPW; ++i) g2lds16(aptr[i] + k0, st + (LPW * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < LPW; ++i) g2lds16(bptr[i] + k0, st + A_BYTES + (LPW * wave + i) * 1024);
  };
  Frags f0, f1;
  auto step = [&](int kt, auto U_c, auto issue_c, auto wait_c, auto drain_c) {
    constexpr int U = decltype(U_c)::value;
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr int WAIT = decltype(wait_c)::value;
    constexpr int DRAIN = decltype(drain_c)::value;
    const char* cur = smem + U * STAGE_BYTES;
    if (ISSUE) issue(kt + NSTAGE - 1, (U + NSTAGE - 1) % NSTAGE);
    rd(cur, 1, f1);
    mma(f0, acc);
    interleave_mma_reads();
    if (WAIT >= 0) {
      wait_barrier<(WAIT < 0 ? 0 : WAIT)>();
      if (DRAIN >= 0 && Drain::LOADS > 0) drain(DRAIN);
      rd(smem + ((U + 1) % NSTAGE) * STAGE_BYTES, 0, f0);
    }
    mma(f1, acc);
    interleave_mma_reads();
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  using WaitFull = std::integral_constant<int, 2 * PER>;
#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) issue(p, p);
  wait_barrier<2 * PER>();
  rd(smem, 0, f0);
  using NoD = std::integral_constant<int, -1>;
  constexpr int DL = Drain::LOADS;
  static_assert(PER + DL < 64 && 2 * DL < 64, "vmcnt range");
  const int nblk = nk / NSTAGE;
  for (int bi = 0; bi < nblk - 1; ++bi) {
    const int kt = bi * NSTAGE;
    step(kt + 0, S0{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 1, S1{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 2, S2{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 3, S3{}, Yes{}, WaitFull{}, NoD{});
  }
  // the last block with the drain (as in gemm_mainloop)
  const int kt = (nblk - 1) * NSTAGE;
  step(kt + 0, S0{}, Yes{}, std::integral_constant<int, 2 * PER>{}, S0{});
  step(kt + 1, S1{}, No{}, std::integral_constant<int, PER + DL>{}, S1{});
  step(kt + 2, S2{}, No{}, std::integral_constant<int, 2 * DL>{}, S2{});
  step(kt + 3, S3{}, No{}, std::integral_constant<int, -1>{}, NoD{});
}

// ======================================================================================================
// fp8 (OCP e4m3fn) mainloop: same tile, ring and barrier structure; K advances 64 values (64 bytes) per
// stage, so the A stage has the bf16 A stage's byte layout (256 rows x 64 B).  The B stage is 64 rows x
// 256 B (chunk c of row k at slot c ^ 2 (k % 8)) and is read K-contiguous with ds_read_b64_tr_b8.  One
// v_mfma_f32_32x32x64_f8f6f4 per 32 x 32 block and stage.  Operand layout of that instruction (measured on the
// device with per-lane block scales, which expose it): lane l, h = l/32, holds in bytes 0..15 the K values
// 16h .. 16h+15 and in bytes 16..31 the K values 32+16h .. 32+16h+15 of its row / column; the scale of lane l
// covers K block h, i.e. K 32h .. 32h+31, half of which sits in each lane half.  Both fragments are gathered
// in that order, so the block scales line up with 32 consecutive K values.
//   ds_read_b64_tr_b8: inside each group of 16 lanes, byte e of lane i is byte i%8 of the 8 bytes addressed
//   by lane 2e + i/8 of the group (verified on the device).
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
constexpr int BK8 = 64;                         // e4m3 values of K per stage
constexpr int K8_MULTIPLE = BK8 * NSTAGE;       // K must be a multiple of this

__device__ __forceinline__ int b8_off(int k, int c) { return k * 256 + ((c ^ ((k & 7) << 1)) << 4); }

__device__ __forceinline__ i32x2 lds_read_tr8(const char* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

struct LaneOffs8 {
  int a;      // A fragment (rows mb*32 add 2 KiB each; the second 16 bytes sit two chunks on, a ^ 32)
  int b[NB];  // B fragment, n-block nb (read r = 0..3 adds 2 KiB each)
};

__device__ __forceinline__ void lane_offsets8(int wm, int wn, int lane, LaneOffs8& o) {
  const int q = lane >> 4, j = lane & 15;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    // lane j of 16-lane group q points at row k0 + j/2, bytes n0 + 8 (j%2) .. +7; after the transposing
    // read lane i of the group holds rows k0..k0+7 of column n0 + i.  Lane half h = q/2 reads rows 16h ..
    // 16h+15 and 32+16h .. 32+16h+15 (four reads of 8 rows, see read_b8)
    const int n0 = wn * (32 * NB) + nb * 32 + 16 * (q & 1);
    const int krow = 16 * (q >> 1) + (j >> 1);
    o.b[nb] = A_BYTES + b8_off(krow, n0 >> 4) + ((j & 1) << 3);
  }
  const int m = wm * 128 + (lane & 31);
  // lane half h takes chunks h and h + 2 of its row (K 16h.. and 32+16h..); chunk h + 2 = h ^ 2 sits at
  // a_off(m, h) ^ 32 (the swizzle is an XOR)
  o.a = a_off(m, lane >> 5);
}

// Fragment reads: B for both 32-column blocks (four transposing reads each), A for one 32-row block.
__device__ __forceinline__ void read_b8(const char* st, const LaneOffs8& o, i32x8 (&b)[NB]) {
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const char* p = st + o.b[nb];
    const i32x2 r0 = lds_read_tr8(p);              // rows 16h + 0..7
    const i32x2 r1 = lds_read_tr8(p + 8 * 256);    // rows 16h + 8..15
    const i32x2 r2 = lds_read_tr8(p + 32 * 256);   // rows 32 + 16h + 0..7
    const i32x2 r3 = lds_read_tr8(p + 40 * 256);   // rows 32 + 16h + 8..15
    b[nb] = (i32x8){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
  }
}
__device__ __forceinline__ i32x8 read_a8(const char* st, const LaneOffs8& o, int mb) {
  const u32x4 lo = *(const u32x4*)(st + o.a + mb * 32 * 64);
  const u32x4 hi = *(const u32x4*)(st + (o.a ^ 32) + mb * 32 * 64);
  return (i32x8){(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Row blocks mb0 and mb0+1 times both column blocks.  Operand formats 0 = e4m3 (cbsz for the first operand,
// blgp for the second).  E8M0 block scales: the B side always 127 = 1.0 (its per-column scales go to the
// epilogue); the A side 127 too, or (MX) byte mb of asc: the scale of the 32 K values this lane holds of its
// row in row block mb.
template <bool MX, int mb0>
__device__ __forceinline__ void mma8_rows(const i32x8 (&b)[NB], const i32x8& a0, const i32x8& a1, int asc,
                                          f32x16 (&acc)[4][NB]) {
  const int s = MX ? asc : 127;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    acc[mb0][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[nb], a0, acc[mb0][nb], 0, 0, 0, 127,
                                                                   MX ? mb0 : 0, s);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    acc[mb0 + 1][nb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[nb], a1, acc[mb0 + 1][nb], 0, 0, 0, 127,
                                                                       MX ? mb0 + 1 : 0, s);
}

// MX scales of the A operand, staged per K step next to the ring: MX_STAGE_BYTES per stage, 256 bytes per
// wave.  In global memory they are laid out so that each wave's 256 bytes for a K step are contiguous and
// lane l of the wave reads its four row blocks' bytes as one word:
//   byte (((kt * tiles_m + tm) * 2 + wm) * 64 + 32 h + j) * 4 + mb
// is the scale of row tm*256 + wm*128 + mb*32 + j, K values 64 kt + 32 h .. +31 (lane l = 32 h + j supplies
// the scale of that K block of that row in row block mb).
constexpr int MX_STAGE_BYTES = NWAVES * 256;
__device__ __forceinline__ int64_t mx_scale_index(int kt, int tiles_m, int m, int h) {
  const int tm = m >> 8, r = m & 255;
  return ((((int64_t)kt * tiles_m + tm) * 2 + (r >> 7)) * 64 + 32 * h + (r & 31)) * 4 + ((r >> 5) & 3);
}

// acc = A[m0:m0+256, :] * B[:, tile columns], e4m3 operands, fp32 accumulation (K % K8_MULTIPLE == 0).
//   A: [M,K] bytes laid out as `al` says (S = 64); B: [K,*] bytes, row stride ldb bytes; bcol(c) = global column of
//   the tile's 16-column chunk c (0..15).
// A step's fragments are split into X = {B blocks, A row blocks 0,1}, double-buffered across steps, and
// Y = {A row blocks 2,3}: the first half multiplies row blocks 0,1 while Y is read; after the barrier the
// second half multiplies row blocks 2,3 while the next stage's X is read into the other buffer.
// MX: asc_g is the A operand's scale array (layout above, tiles_m row tiles) and mx_smem the MX_STAGE_BYTES x
// NSTAGE staging area; each wave adds one 4-byte-per-lane direct load per stage.  hook() as in gemm_mainloop.
template <bool MX = false, class BCol, class Hook = NoHook, class Drain = NoDrain>
__device__ __forceinline__ void gemm_mainloop_fp8(const uint8_t* __restrict__ A, ALayout al, int M, int m0,
                                                  const uint8_t* __restrict__ B, int64_t ldb, BCol bcol, int K,
                                                  char* smem, f32x16 (&acc)[4][NB], Hook hook = Hook{},
                                                  const uint8_t* __restrict__ asc_g = nullptr,
                                                  char* mx_smem = nullptr, Drain drain = Drain{}) {
  constexpr int LPW = 16 / NWAVES;
  constexpr int PER = 2 * LPW + (MX ? 1 : 0);
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave & 1, wn = wave >> 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = (f32x16){};

  // direct-load unit q: A rows 16q .. 16q+15 (as the bf16 A stage); B rows 4q .. 4q+3 (lane -> row
  // 4q + lane/16, slot lane%16)
  // 32-bit byte offsets from the operand bases (every e4m3 operand is below 2^31 bytes): half the registers
  // of per-lane pointers
  uint32_t aoff[LPW], boff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int q = LPW * wave + i;
    const int r = 16 * q + (lane >> 2);
    const int c = (lane & 3) ^ ((r >> 2) & 3);
    int row = m0 + r;
    row = row < M ? row : M - 1;
    aoff[i] = (uint32_t)((int64_t)row * al.row + 16 * c);
    const int kr = 4 * q + (lane >> 4);
    const int cb = (lane & 15) ^ ((kr & 7) << 1);
    boff[i] = (uint32_t)((int64_t)kr * ldb + bcol(cb));
  }
  const uint32_t astep = (uint32_t)al.step;  // bytes per K step of A (below 2^31 as A is)
  LaneOffs8 lo;
  lane_offsets8(wm, wn, lane, lo);
  const int nk = K / BK8;
  // MX: this wave's 256 scale bytes of K step kt start at asc_g + ((kt * tiles_m + tm) * 2 + wm) * 256
  // (wave-uniform; only the lane's 4-byte offset is per lane)
  const int tiles_m = (M + BM - 1) / BM;
  const uint8_t* asc_w = MX ? asc_g + ((int64_t)(m0 >> 8) * 2 + wm) * 256 : nullptr;
  const int64_t asc_step = (int64_t)tiles_m * 512;

  auto issue = [&](int kt, int stage) {
    char* st = smem + stage * STAGE_BYTES;
    const int k0 = kt * BK8;
    const uint32_t ak = (uint32_t)kt * astep;  // wave-uniform
#pragma unroll
    for (int i = 0; i < LPW; ++i) g2lds16(A + ak + aoff[i], st + (LPW * wave + i) * 1024);
#pragma unroll
    for (int i = 0; i < LPW; ++i) g2lds16(B + (int64_t)k0 * ldb + boff[i], st + A_BYTES + (LPW * wave + i) * 1024);
    if (MX)
      __builtin_amdgcn_global_load_lds(asc_w + kt * asc_step + 4 * lane,
                                       (lds_void*)(mx_smem + stage * MX_STAGE_BYTES + wave * 256), 4, 0, 0);
  };
  // MX: lane l's word of the stage: the scales of its four row blocks
  auto read_asc = [&](int stage) {
    return MX ? *(const int*)(mx_smem + stage * MX_STAGE_BYTES + wave * 256 + 4 * lane) : 127;
  };

  i32x8 xb[2][NB], xa[2][2], ya[2];
  // one K step on stage U; X[U % 2] holds the stage's B and A row blocks 0,1 on entry.  Every fragment of stage U
  // is in registers by the mid-step barrier (B and A blocks 0,1 from the previous step, A blocks 2,3 read before
  // the barrier), so DRAIN >= 0 hands the stage to drain(DRAIN) right after it, as in gemm_mainloop
  auto step = [&](int kt, auto U_c, auto issue_c, auto wait_c, auto drain_c) {
    constexpr int U = decltype(U_c)::value;
    constexpr int P = U & 1;
    constexpr bool ISSUE = decltype(issue_c)::value;
    constexpr int WAIT = decltype(wait_c)::value;
    constexpr int DRAIN = decltype(drain_c)::value;
    const char* cur = smem + U * STAGE_BYTES;
    if (ISSUE) issue(kt + NSTAGE - 1, (U + NSTAGE - 1) % NSTAGE);
    // MX: this stage's scale word, read first so that the first MFMAs wait for it alone (one register: a
    // prefetched copy per buffer would not fit)
    const int sc = read_asc(U);
    ya[0] = read_a8(cur, lo, 2);
    ya[1] = read_a8(cur, lo, 3);
    mma8_rows<MX, 0>(xb[P], xa[P][0], xa[P][1], sc, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // DS read
    }
    if (WAIT >= 0) {
      wait_barrier<(WAIT < 0 ? 0 : WAIT)>();
      if (DRAIN >= 0 && Drain::LOADS > 0) drain(DRAIN);
      const char* nxt = smem + ((U + 1) % NSTAGE) * STAGE_BYTES;
      read_b8(nxt, lo, xb[1 - P]);
      xa[1 - P][0] = read_a8(nxt, lo, 0);
      xa[1 - P][1] = read_a8(nxt, lo, 1);
    }
    mma8_rows<MX, 2>(xb[P], ya[0], ya[1], sc, acc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;
  using Yes = std::true_type;
  using No = std::false_type;
  using WaitFull = std::integral_constant<int, 2 * PER>;

#pragma unroll
  for (int p = 0; p < NSTAGE - 1; ++p) issue(p, p);
  wait_barrier<2 * PER>();
  hook();
  read_b8(smem, lo, xb[0]);
  xa[0][0] = read_a8(smem, lo, 0);
  xa[0][1] = read_a8(smem, lo, 1);

  using NoD = std::integral_constant<int, -1>;
  constexpr int DL = Drain::LOADS;
  static_assert(PER + DL < 64 && 2 * DL < 64, "vmcnt range");
  const int nblk = nk / NSTAGE;
  for (int bi = 0; bi < nblk - 1; ++bi) {
    const int kt = bi * NSTAGE;
    step(kt + 0, S0{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 1, S1{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 2, S2{}, Yes{}, WaitFull{}, NoD{});
    step(kt + 3, S3{}, Yes{}, WaitFull{}, NoD{});
  }
  // the last block: the waits shrink as the ring drains and count the drain's loads issued after the stage loads
  const int kt = (nblk - 1) * NSTAGE;
  step(kt + 0, S0{}, Yes{}, std::integral_constant<int, 2 * PER>{}, S0{});
  step(kt + 1, S1{}, No{}, std::integral_constant<int, PER + DL>{}, S1{});
  step(kt + 2, S2{}, No{}, std::integral_constant<int, 2 * DL>{}, S2{});
  step(kt + 3, S3{}, No{}, std::integral_constant<int, -1>{}, NoD{});
}

// Global column of the tile's column chunk c when the tile's 256 accumulator columns are one contiguous
// range starting at n0 (W columns per chunk: 8 for bf16, 16 for e4m3).
template <int W>
struct ContiguousCols {
  int64_t n0;
  __device__ int64_t operator()(int c) const { return n0 + W * c; }
};

// ---- output tile staging in LDS -----------------------------------------------------------------------
// Output tiles are written with the non-temporal hint (global_store ... nt).  Measured on the block's two GEMMs
// back to back: with plain stores the pair took about 12 us more than the two kernels alone (the boundary
// between them waits for the first kernel's written lines to leave the L2s); with the hint it takes their sum.
__device__ __forceinline__ void store16_nt(uint16_t* p, u32x4 v) { __builtin_nontemporal_store(v, (u32x4*)p); }
// The same hint for the other kernels' outputs (any vector type).
template <class T>
__device__ __forceinline__ void store_nt(void* p, T v) { __builtin_nontemporal_store(v, (T*)p); }

// A bf16 tile of 256 rows x 8 CH columns: row r is 16 CH bytes, its 16-byte chunk c at slot c ^ (r % CH), so
// both the lanes that write 32 rows of one chunk and the lanes that read one row's chunks spread over the
// banks.
template <int CH>
__device__ __forceinline__ int tile_off(int r, int c) { return r * (16 * CH) + ((c ^ (r & (CH - 1))) << 4); }

// Whole rows of the staged tile to dst[(m0 + r) * ld + n0 ...], 16 bytes per lane; rows >= M are skipped.  ROWS:
// the staged rows read (the first ROWS of the tile).
template <int CH, int ROWS = BM>
__device__ __forceinline__ void store_tile_rows(const char* smem, uint16_t* dst, int ld, int m0, int n0, int M) {
  constexpr int ROWS_PER_PASS = NTHREADS / CH;
  static_assert(ROWS % ROWS_PER_PASS == 0, "whole passes");
  const int t = threadIdx.x;
  const int c = t % CH;
#pragma unroll
  for (int p = 0; p < ROWS / ROWS_PER_PASS; ++p) {
    const int r = p * ROWS_PER_PASS + t / CH;
    const u32x4 v = *(const u32x4*)(smem + tile_off<CH>(r, c));
    const int m = m0 + r;
    if (m < M) store16_nt(dst + (int64_t)m * ld + n0 + 8 * c, v);
  }
}

// The staged tile to K panels of 32 columns: column n0 + 32 p + j of row m0 + r goes to
// dst[(n0 / 32 + p) * panel + (m0 + r) * 32 + j] (panel = rows * 32 elements, the panel stride); rows >= M are
// skipped.  Each wave writes 1 KiB of one panel per pass (16 rows x 64 bytes, contiguous).  ROWS as in
// store_tile_rows.
template <int CH, int ROWS = BM>
__device__ __forceinline__ void store_tile_panels(const char* smem, uint16_t* dst, int64_t panel, int m0, int n0,
                                                  int M) {
  static_assert(ROWS * CH % NTHREADS == 0, "whole passes");
  const int t = threadIdx.x;
#pragma unroll
  for (int p = 0; p < ROWS * CH / NTHREADS; ++p) {
    const int g = p * NTHREADS + t;       // 16-byte chunk of the tile in panel order
    const int pn = g / (ROWS * 4);        // panel (4 chunks of 16 bytes per row)
    const int w = g % (ROWS * 4);
    const int r = w >> 2, c4 = w & 3;
    const u32x4 v = *(const u32x4*)(smem + tile_off<CH>(r, 4 * pn + c4));
    const int m = m0 + r;
    if (m < M) store16_nt(dst + (int64_t)(n0 / 32 + pn) * panel + (int64_t)m * 32 + 8 * c4, v);
  }
}

// Rows m0 .. m0+255 of src (columns n0 .. n0 + 8 CH) into the staged-tile layout with direct global -> LDS
// loads (rows past M read row M-1).  The caller waits for the loads (vmcnt) and synchronises the workgroup.
template <int CH>
__device__ __forceinline__ void load_tile_rows(const uint16_t* src, int ld, int m0, int n0, int M, char* smem) {
  constexpr int ROWS_PER_INST = 64 / CH;  // one wave instruction fills 1 KiB
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < BM / (NWAVES * ROWS_PER_INST); ++j) {
    const int r0 = (wave * (BM / NWAVES)) + j * ROWS_PER_INST;
    const int r = r0 + lane / CH;
    const int slot = lane % CH;
    int m = m0 + r;
    m = m < M ? m : M - 1;
    g2lds16(src + (int64_t)m * ld + n0 + 8 * (slot ^ (r & (CH - 1))), smem + r0 * (16 * CH));
  }
}

// Rows row0 .. row0+63 of the staged-tile layout (as load_tile_rows), 64 / (NWAVES * 64 / CH) direct loads per
// wave: with CH = 32 the 32 KiB of one ring stage, 4 loads per wave.
template <int CH>
__device__ __forceinline__ void load_tile_rows64(const uint16_t* src, int ld, int m0, int n0, int M, char* smem,
                                                 int row0) {
  constexpr int ROWS_PER_INST = 64 / CH;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#pragma unroll
  for (int j = 0; j < 64 / (NWAVES * ROWS_PER_INST); ++j) {
    const int r0 = row0 + wave * (64 / NWAVES) + j * ROWS_PER_INST;
    const int r = r0 + lane / CH;
    const int slot = lane % CH;
    int m = m0 + r;
    m = m < M ? m : M - 1;
    g2lds16(src + (int64_t)m * ld + n0 + 8 * (slot ^ (r & (CH - 1))), smem + r0 * (16 * CH));
  }
}

// The epilogue's 256 x 256 bf16 tile of a row-major [*, ld] operand (the residual, or h), rows 64 s .. 64 s + 63
// into ring stage s as the ring drains (see NoDrain); the caller loads rows 192 .. 255 after the mainloop.
struct TileRowsDrain {
  static constexpr int LOADS = 4;
  const uint16_t* src;
  int ld, m0, n0, M;
  char* smem;
  __device__ void operator()(int s) const { load_tile_rows64<32>(src, ld, m0, n0, M, smem, 64 * s); }
};

// Maps the linear workgroup id to a (row tile, column tile) pair.
// Workgroups are dealt to the 8 XCDs round-robin (id % 8), each XCD with its own L2.  The id is first
// remapped so that XCD x receives a contiguous range of the tile order, then tiles are ordered in groups of
// `group_m` row tiles (row tile fastest inside a group), so the tiles one XCD runs together share A row
// tiles and B column tiles in its L2.
__device__ __forceinline__ void tile_of_order(int b, int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  const int group_size = group_m * tiles_n;
  const int group = b / group_size;
  const int first_m = group * group_m;
  const int gm = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
  const int in_group = b - group * group_size;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int group_m, int& tm, int& tn) {
  int b = blockIdx.x;
  const int ntiles = tiles_m * tiles_n;
  if ((ntiles & 7) == 0) b = (b & 7) * (ntiles >> 3) + (b >> 3);
  tile_of_order(b, tiles_m, tiles_n, group_m, tm, tn);
}

// The same with the tiles from `full` on (in tile order) split in 2^lg pieces along K: workgroups 0 .. full-1 take
// whole tiles as tile_coords deals them (over `full` tiles), the next (ntiles - full) 2^lg take pieces, XCD by XCD in
// contiguous ranges of the piece order, with all pieces of a tile on one XCD where the count allows.  Returns the
// piece (0 .. 2^lg - 1: its place along K) or -1 for a whole tile; b_out is the tile's place in the tile order.
__device__ __forceinline__ int tile_coords_split(int tiles_m, int tiles_n, int group_m, int full, int lg, int& tm,
                                                 int& tn, int& b_out) {
  const int ntiles = tiles_m * tiles_n;
  int b = blockIdx.x;
  int piece = -1;
  if (b < full) {
    if ((full & 7) == 0) b = (b & 7) * (full >> 3) + (b >> 3);
  } else {
    int p = b - full;
    const int np = (ntiles - full) << lg;
    if ((np & ((8 << lg) - 1)) == 0) p = (p & 7) * (np >> 3) + (p >> 3);  // np / 8 a multiple of 2^lg
    piece = p & ((1 << lg) - 1);
    b = full + (p >> lg);
  }
  b_out = b;
  tile_of_order(b, tiles_m, tiles_n, group_m, tm, tn);
  return piece;
}

}  // namespace coda
