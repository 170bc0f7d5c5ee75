// launch.h -- host-side launchers of the block's kernels (kernels.hip).  All of them enqueue on `stream`
// and return hipGetLastError() after the launch.  Shapes are checked by the C ABI before these run.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace coda {

// Split of a GEMM's last, partial wave of output tiles.  When the tile count leaves a last wave that fills a small
// part of the CUs (ksplit_plan), the tiles of that wave (the last ones in the tile order) are each computed as
// S = 2^lg pieces over S equal ranges of K, so the last wave runs on S times as many CUs: the grid holds `full` whole
// tiles, then (ntiles - full) S pieces.  The pieces of a tile meet in a binary tree of S - 1 nodes: at each level a piece stores
// its fp32 accumulators in its slot of `part`, then takes a ticket from its node's counter; the piece that draws the
// node's second ticket adds its sibling's slot to its own accumulators (fp32 addition is commutative, so each node's
// sum does not depend on which of its two pieces comes second, and the tree fixes the order of the rest) and goes
// on to the next level; the first one exits.  The root's second arrival runs the epilogue.  No piece waits for
// another.  The counters must be zero at launch: the block's first GEMM clears those of its second GEMM (`clear`,
// `nclear`), and launch_clear_tickets clears the first GEMM's own before it runs.  Both GEMMs of every block (K1 or
// U1, and K3 or U3; bf16 and e4m3) can be split.
//
// The other form of a partial last wave (`halves`, the bf16 row-scale GEMMs: K3 and U3): each of its tiles is computed
// as two 128-row halves over the whole of K, in a launch of its own right after the `full` whole tiles, so the last
// wave runs on twice as many CUs with no exchange (gemm_mainloop's half-tile form; the results are the whole tiles'
// bit for bit).  halves_plan chooses it where the split along K does not apply.
struct KSplit {
  int full = -1;          // whole tiles; negative: no split
  int lg = 1;             // S = 2^lg pieces per split tile (1 .. 3)
  int halves = 0;         // 1: the tiles from `full` on run as two 128-row halves (lg, part, cnt unused)
  float* part = nullptr;  // (ntiles - full) (2 S - 2) slots of KSPLIT_SLOT_FLOATS fp32: level l's 2^(lg-l) slots
                          // per tile follow the lower levels'
  int* cnt = nullptr;     // (ntiles - full) (S - 1) tickets: level l's 2^(lg-l-1) per tile after the lower levels'
  int* clear = nullptr;   // the block's first GEMM: the second GEMM's tickets, zeroed by its workgroup 0
  int nclear = 0;
};
constexpr int KSPLIT_SLOT_FLOATS = 512 * 128;  // one workgroup's accumulators (512 lanes x 128)
constexpr int KSPLIT_MAX_LG = 3;  // at most 8 pieces per tile
// The split rule of one operand type (all K in elements): a last wave of at most cus / tail_den tiles splits, or of at
// most three eighths of the CUs where K >= long_k, if K gives two pieces of at least min_piece (K a multiple of
// 2 gran, gran = one fill of the 4-stage ring); into 4 or 8 pieces while all the pieces stay within half of the CUs
// and each keeps tree_piece of K (K a multiple of gran times the pieces).
struct KSplitRule {
  int gran, min_piece, tree_piece, long_k, tail_den;
};
// bf16, measured on MI355X (the block's time): with two pieces, a last wave of 16 or 32 tiles at K = 2048 gains
// 7-10 us, one of 64 about 2 us, one of 96 or 128 loses 2-7 us (the pieces' fp32 slots cross the memory system, 256 KiB
// written per piece and level, and a last wave of whole tiles on part of the chip runs at a higher clock than the
// full chip does); over longer K the savings grow and the exchange does not: last waves of 80 and 96 tiles gain 8-15
// us at K = 4096 and 32-53 us at K = 8192, one of 128 still loses up to 7 us.  More pieces pay where each keeps 1024
// of K or more (one tile over K1 = 8192 in eight: 150 -> 57 us; 32 tiles over K1 = 8192 in four rather than two:
// 123 -> 105 us) and lose below that (32 tiles over K = 2048 in four: 113 -> 120 us).
constexpr KSplitRule KSPLIT_BF16{128, 512, 1024, 4096, 4};
// e4m3 (an e4m3 K value costs the MFMAs half a bf16 one, the exchange the same): in two pieces, last waves of 16 or
// 32 tiles lose up to 3 us at K = 2048 and gain 4-9 us at K = 4096, one of 64 loses 3-8 us at K = 2048 and 2-6 us at
// K = 4096; 32 tiles over K1 = 8192 in four gain 20 us (107 -> 87 us), 96 tiles over K1 = 8192 in two 4-5 us.
constexpr KSplitRule KSPLIT_E4M3{256, 2048, 2048, 8192, 8};
// The split of `ntiles` output tiles over K on `cus` CUs, by the rule of the operands' type (fp8 != 0: e4m3):
// returns the number of whole tiles (ntiles when no split pays) and sets *lg to log2 of the pieces per split tile.
int ksplit_plan(int64_t ntiles, int64_t K, int cus, int fp8, int* lg);
// The half-tile form of a last wave of `ntiles` tiles of a bf16 row-scale GEMM with M rows on `cus` CUs: a KSplit with
// halves set and `full` the whole tiles where the last wave's halves fit on the CUs (at most half of them filled by
// whole tiles) and the last row tile has more than 128 rows or none missing; else no split.  Measured on MI355X: the
// 1B MLP-out -> QKV second GEMM (a last wave of 128 tiles over K = 2048) 98 -> 93 us, 8192 x 2816 over K = 256
// (96 tiles) 95 -> 89 us, a SwiGLU one with 128 tiles 98 -> 93 us.
KSplit halves_plan(int64_t ntiles, int64_t M, int cus);
// Zeroes n tickets (a small kernel on `stream`; graph-capturable, unlike a memset node).
hipError_t launch_clear_tickets(int* cnt, int n, hipStream_t stream);

// K1: H = bf16(X W1 + R), HG = bf16((X W1 + R) * gamma) and part[t][m] = sum over tile t's 256 columns of
// the fp32 (X W1 + R)^2.
// `panels` (here and below): HG / HQ are written, and the second GEMM's A operand is read, in K panels of the
// mainloop's stage width ([D / 32][M][32] bf16, [D / 64][M][64] e4m3 bytes) instead of row-major [M, D].
hipError_t launch_gemm1_res_prms(const uint16_t* X, const uint16_t* W1, const uint16_t* R, const float* gamma,
                                 uint16_t* H, uint16_t* HG, float* part, int M, int K1, int D, hipStream_t stream,
                                 int panels = 0, KSplit ks = KSplit());
// K2: r[m] = 1 / sqrt(sum_t part[t][m] / D + eps).
hipError_t launch_prms_reduce(const float* part, int T, int M, int D, float eps, float* r, hipStream_t stream);
// K3 (r non-null; A = h * gamma) and U3 (r null; A = the normalised rows): Y = bf16(epi(r * (A W2))).
// ks (here, in the fold and rope launchers, and for K1 and U1): the split of the GEMM's last wave (KSplit).
// Z (SwiGLU only, may be null): also store the pre-activation z = [gate | up] = r (A W2) as bf16 [M, N2].
hipError_t launch_gemm2_rowscale(const uint16_t* A, const uint16_t* W2, const float* r, int swiglu, uint16_t* Y,
                                 int M, int D, int N2, hipStream_t stream, uint16_t* Z = nullptr, int panels = 0,
                                 KSplit ks = KSplit());
// K2 folded into K3 (D / 256 <= 16, see fold_supported): the row scales come from the partial sums of K1, are
// formed per workgroup as launch_prms_reduce forms them, and are written to r by the tiles of column 0.
int fold_supported(int D);
hipError_t launch_gemm2_rowscale_fold(const uint16_t* A, const uint16_t* W2, const float* part, float eps, float* r,
                                      int swiglu, uint16_t* Y, int M, int D, int N2, hipStream_t stream,
                                      uint16_t* Z = nullptr, int panels = 0, KSplit ks = KSplit());
// K3 with a rotary embedding after the row scale (identity epilogue): Y = bf16(rope(r * (A W2))); the first n_rot
// columns form heads of 64 rotated at position row mod seq_len with frequencies base^(-2i/64).
hipError_t launch_gemm2_rowscale_rope(const uint16_t* A, const uint16_t* W2, const float* r, int seq_len, int n_rot,
                                      float base, uint16_t* Y, int M, int D, int N2, hipStream_t stream,
                                      int panels = 0, KSplit ks = KSplit());
hipError_t launch_gemm2_rowscale_rope_fold(const uint16_t* A, const uint16_t* W2, const float* part, float eps,
                                           float* r, int seq_len, int n_rot, float base, uint16_t* Y, int M, int D,
                                           int N2, hipStream_t stream, int panels = 0, KSplit ks = KSplit());
// The same rotation as a separate in-place pass over bf16 Y [M,N] (the unfused counterpart).
hipError_t launch_rope_rows(uint16_t* Y, int M, int N, int seq_len, int n_rot, float base, hipStream_t stream);
// U1: T = bf16(X W); a_panels: X given in K panels of 32 ([K/32][M][32], as launch_panelize_bf16 writes).
hipError_t launch_gemm_store(const uint16_t* X, const uint16_t* W, uint16_t* T, int M, int K, int N,
                             hipStream_t stream, int a_panels = 0, KSplit ks = KSplit());
// U2: H = bf16(T + R), N = bf16((T + R) r gamma), r[m] (optional).  D <= 8192.
hipError_t launch_add_rmsnorm(const uint16_t* T, const uint16_t* R, const float* gamma, uint16_t* H, uint16_t* N,
                              float* r, int M, int D, float eps, hipStream_t stream);

// ---- e4m3 operands (scales: dequantised value = code * scale) ----
// K1: as launch_gemm1_res_prms with X W1 = (Xq W1q) * sx[m] * sw1[n].
hipError_t launch_gemm1_res_prms_fp8(const uint8_t* Xq, const float* sx, const uint8_t* W1q, const float* sw1,
                                     const uint16_t* R, uint16_t* H, float* part, int M, int K1, int D,
                                     hipStream_t stream, KSplit ks = KSplit());
// MX variant of K1: also HQ = e4m3 codes of a = bf16(H) * gamma in blocks of 32 columns with power-of-two scales
// (HS: one byte e + 127 per block, laid out as mx_scale_index in gemm_core.h; ceil(M / 256) * 256 rows * D / 32
// bytes).  D % 256 == 0.
hipError_t launch_gemm1_res_prms_fp8_mx(const uint8_t* Xq, const float* sx, const uint8_t* W1q, const float* sw1,
                                        const uint16_t* R, const float* gamma, uint16_t* H, uint8_t* HQ, uint8_t* HS,
                                        float* part, int M, int K1, int D, hipStream_t stream, int panels = 0,
                                        KSplit ks = KSplit());
// MX variant of K3: Y = bf16(epi(r * (HQ W2q) * sw2[n])) with HQ's block scales inside the MFMA.  With part
// non-null the reduce is folded in (D / 256 <= 16; r written to r_out), else the row scale is r_in.
hipError_t launch_gemm2_rowscale_fp8_mx(const uint8_t* HQ, const uint8_t* HS, const uint8_t* W2q, const float* sw2,
                                        const float* r_in, const float* part, float eps, float* r_out, int swiglu,
                                        uint16_t* Y, int M, int D, int N2, hipStream_t stream, int panels = 0,
                                        KSplit ks = KSplit());
// K2: r from the partial sums; with a = H * gamma (fp32), HQ = e4m3(a * (1 / sa)) per row, sa = amax|a row| / 448;
// rs2 = sa * r.
hipError_t launch_prms_reduce_quant(const float* part, int T, int M, int D, float eps, const uint16_t* H,
                                    const float* gamma, uint8_t* HQ, float* r, float* sa, float* rs2,
                                    hipStream_t stream, int panels = 0);
// K3 / U3: Y = bf16(epi((Aq W2q) * rowsc[m] * sw2[n])).
hipError_t launch_gemm2_rowscale_fp8(const uint8_t* Aq, const uint8_t* W2q, const float* rowsc, const float* sw2,
                                     int swiglu, uint16_t* Y, int M, int D, int N2, hipStream_t stream,
                                     int panels = 0, KSplit ks = KSplit());
// U1: T = bf16((Xq Wq) * sx[m] * sw[n]).
hipError_t launch_gemm_store_fp8(const uint8_t* Xq, const float* sx, const uint8_t* Wq, const float* sw, uint16_t* T,
                                 int M, int K, int N, hipStream_t stream, KSplit ks = KSplit());
// U2: H = bf16(T + R); NQ = e4m3(n / sn) per row with n = (T + R) r gamma and sn = amax|n row| / 448.
hipError_t launch_add_rmsnorm_quant(const uint16_t* T, const uint16_t* R, const float* gamma, uint16_t* H,
                                    uint8_t* NQ, float* r, float* sn, int M, int D, float eps, hipStream_t stream);

// ---- backward (bwd_kernels.hip) ----
// B1: P = dz W2^T (W2 [D,N2] read as rows); G = bf16(r gamma P) [M,D]; part[D/256][M] row partials of
// gamma P h; part2[ceil(M/256)][D] column partials of P r h.
hipError_t launch_bwd_p(const uint16_t* dz, const uint16_t* W2, const uint16_t* h, const float* r, const float* gamma,
                        uint16_t* G, float* part, float* part2, int M, int D, int N2, hipStream_t stream);
// The unfused counterpart of B1's epilogue: the same outputs from a stored P [M,D] (bf16).
hipError_t launch_bwd_p_from_mem(const uint16_t* P, const uint16_t* h, const float* r, const float* gamma, uint16_t* G,
                                 float* part, float* part2, int M, int D, hipStream_t stream);
// C [M,N] = bf16(A Bt^T), A [M,K], Bt [N,K].
// B1 with the NN mainloop on W2T = W2^T [N2, D] (same outputs as launch_bwd_p).
hipError_t launch_bwd_p_nn(const uint16_t* dz, const uint16_t* W2T, const uint16_t* h, const float* r,
                           const float* gamma, uint16_t* G, float* part, float* part2, int M, int D, int N2,
                           hipStream_t stream);
// C [M,N] = bf16(A [M,K] B [K,N]) on the NN mainloop.
hipError_t launch_gemm_nn_store(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int K, int N,
                                hipStream_t stream);
// dst [C, R] = src [R, C]^T, bf16; R and C multiples of 64.
hipError_t launch_transpose_bf16(const uint16_t* src, int R, int C, uint16_t* dst, hipStream_t stream);
hipError_t launch_gemm_nt_store(const uint16_t* A, const uint16_t* Bt, uint16_t* C, int M, int K, int N,
                                hipStream_t stream);
// Number of K ranges the fp32 products below split K into (1, 2, 4 or 8): enough workgroups to cover the
// CUs when the output has few tiles.  The partial products go to `slabs` (gemm_ksplit(...) * M * N floats,
// unused when it is 1) and are summed in order by a second kernel.
int gemm_ksplit(int M, int N, int K);
// C [M,N] = fp32 rowsc[m] * (A B), A [M,K], B [K,N] (rowsc may be null).  a_panels: A in K panels
// [K/32][M][32] (as launch_bwd_dh writes dh^T and n^T with panels set), else row-major.
hipError_t launch_gemm_f32_rowscale(const uint16_t* A, const uint16_t* B, const float* rowsc, float* C, int M, int K,
                                    int N, float* slabs, hipStream_t stream, int a_panels = 0);
// Ct [N,M] = fp32 (A B)^T, A [M,K], B [K,N]; a_panels as above.
hipError_t launch_gemm_f32_trans(const uint16_t* A, const uint16_t* B, float* Ct, int M, int K, int N, float* slabs,
                                 hipStream_t stream, int a_panels = 0);
// B2: a[i] = r_i^3 / D * sum_t part[t][i]; dgamma[j] = sum_q part2[q][j].
hipError_t launch_bwd_reduce(const float* part, int T, const float* part2, int Q, const float* r, int M, int D,
                             float* a, float* dgamma, hipStream_t stream);
// B3: dR = bf16(G - a h + dh_out) [M,D]; dhT, nT [D,M] = dR and bf16(r h), transposed.  M, D multiples of 64.
// panels: dhT and nT in K panels over M for the weight-gradient products ([M/32][D][32]), else [D,M] rows.
hipError_t launch_bwd_dh(const uint16_t* G, const uint16_t* h, const uint16_t* dh_out, const float* r, const float* a,
                         int M, int D, uint16_t* dR, uint16_t* dhT, uint16_t* nT, hipStream_t stream,
                         int panels = 0);

// ---- cross-entropy of a vocabulary projection (ce_kernels.hip) ----
// C1: logits z = H W by 256 x 256 tiles; per tile t and row i, part_m[t][i] = max z, part_s[t][i] = sum exp(z -
// max); zlab[i] = z[i][labels[i]] from the tile holding that column.  D % 128 == 0, V % 256 == 0.
hipError_t launch_ce_gemm(const uint16_t* H, const uint16_t* W, const int* labels, float* part_m, float* part_s,
                          float* zlab, int M, int D, int V, hipStream_t stream, int a_panels = 0);
// dst = src [M,D] bf16 in K panels of 32 columns ([D/32][M][32]); D % 32 == 0.
hipError_t launch_panelize_bf16(const uint16_t* src, int M, int D, uint16_t* dst, hipStream_t stream);
// C2: lse[i] = merge of the T pairs of row i in tile order; loss[i] = lse[i] - zlab[i] (0 for a negative label,
// NaN for a label >= V).
hipError_t launch_ce_reduce(const float* part_m, const float* part_s, const float* zlab, const int* labels, int T,
                            int M, int V, float* loss, float* lse, hipStream_t stream);
// CU: the same from stored bf16 logits Z [M,V] (the unfused baseline).
hipError_t launch_ce_rows(const uint16_t* Z, const int* labels, int M, int V, float* loss, float* lse,
                          hipStream_t stream);

// ---- backward of the SwiGLU epilogue (bwd_kernels.hip) ----
// S1: dy = dout Wd^T (dout [M,D], Wd [F,D] read as its own rows; D % 128 == 0, F % 256 == 0) with the SwiGLU
// backward in the epilogue: dz[:, f] = dy u silu'(g), dz[:, F + f] = dy silu(g), g = z[:, f], u = z[:, F + f];
// dy is never stored.
hipError_t launch_swiglu_bwd(const uint16_t* dout, const uint16_t* Wd, const uint16_t* z, uint16_t* dz, int M, int D,
                             int F, hipStream_t stream);
// The baseline's second kernel: the same from a stored dy [M,F] bf16.
hipError_t launch_swiglu_bwd_rows(const uint16_t* dy, const uint16_t* z, uint16_t* dz, int M, int F,
                                  hipStream_t stream);

}  // namespace coda
