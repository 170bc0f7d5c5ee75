/*
 * oracle.h -- plain, slow, fp64 CPU reference for the fused GEMM -> residual -> RMSNorm -> GEMM block.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU-baseline leg of the
 * benchmark may load this library.  The GPU library never links it, includes it or calls it, and the two
 * share no code, headers, tables or helpers.
 *
 * What it computes (CODA write-up: "CODA: new research optimizes Transformer training with GEMM-epilogue
 * programming", KuCoin news flash, section "CODA: the treasure hidden in the epilogue"):
 *   a GEMM whose output gets a residual added, is RMS-normalised per row and then multiplied by a second
 *   weight matrix, optionally followed by a SwiGLU activation ("a similar reparameterization applies to
 *   SwiGLU", same section).  The fused form moves the per-row RMS factor r past the second GEMM because a
 *   per-row scalar commutes with a matrix product.
 *
 * Readings of points the pages leave open (each is a choice, not a quotation):
 *   - r_i = 1 / sqrt(mean_j h_ij^2 + eps): eps inside the square root, mean over the hidden dim D.
 *   - the RMSNorm weight gamma multiplies the normalised row elementwise; in the fused form it is folded
 *     into the second weight, W2' = diag(gamma) W2.
 *   - SwiGLU on a fused gate|up product: columns [0, N2/2) are the gate, [N2/2, N2) the up projection,
 *     y = silu(gate) * up with silu(x) = x / (1 + exp(-x)); r multiplies both halves before silu.
 *
 * Layouts: every matrix is dense row-major.  X [M,K1], W1 [K1,D], R and h [M,D], gamma [D], W2 [D,N2],
 * y [M,N2] (identity) or [M,N2/2] (SwiGLU).  All arrays are caller-owned.  Functions return 0 on success
 * and a negative value on a bad argument; they never abort.
 */
#ifndef CODA_ORACLE_H
#define CODA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_EPI_IDENTITY 0
#define ORACLE_EPI_SWIGLU 1

/* Threads used when nthreads <= 0: the CPUs this process may run on. */
int oracle_default_threads(void);

/* h = X W1 + R (R may be NULL for a plain product). */
int oracle_gemm_residual_f64(int64_t M, int64_t K1, int64_t D, const double* X, const double* W1,
                             const double* R, double* out_h, int nthreads);

/* r_i = 1 / sqrt(mean_j h_ij^2 + eps) for each row of h [M,D]. */
int oracle_rms_scale_f64(int64_t M, int64_t D, const double* h, double eps, double* out_r);

/* The row scale computed from per-tile partial sums of squares part[T][M]:
 * r_i = 1 / sqrt((sum_t part[t][i]) / D + eps).  The partials are the "local partial RMS" values of the
 * write-up (section "CODA: the treasure hidden in the epilogue"); summing them over t gives sum_j h_ij^2. */
int oracle_rms_from_partials_f64(int64_t T, int64_t M, const double* part, int64_t D, double eps,
                                 double* out_r);

/* Unfused order: h = X W1 + R; n = h * r * gamma; z = n W2; y = epi(z).
 * out_h [M,D] and out_r [M] may be NULL. */
int oracle_block_unfused_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                             const double* W1, const double* R, const double* gamma, const double* W2,
                             double eps, int epi, double* out_h, double* out_r, double* out_y,
                             int nthreads);

/* Reparameterised order: W2' = diag(gamma) W2; u = h W2'; z = r * u (row scale applied after the
 * product); y = epi(z).  Same arguments as the unfused form. */
int oracle_block_fused_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                           const double* W1, const double* R, const double* gamma, const double* W2,
                           double eps, int epi, double* out_h, double* out_r, double* out_y,
                           int nthreads);

/* Diagnostic: the reparameterised order with the storage roundings a bf16 implementation makes when it
 * broadcasts gamma onto h in the first GEMM's epilogue: a_ij = bf16(h_ij * gamma_j) (r still comes from the
 * unrounded h), z = r_i * (a W2), y = bf16(epi(z)).  Not the contract; a sharp bug detector. */
int oracle_block_roundpts_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                              const double* W1, const double* R, const double* gamma, const double* W2,
                              double eps, int epi, double* out_h, double* out_r, double* out_y,
                              int nthreads);

/* Backward of the block (chain rule of the unfused order; see oracle.c): given dz [M,N2], the gradient of
 * z = (h * r * gamma) W2 (the second product's output before the epilogue), and dh_out [M,D] (the gradient
 * arriving at h from downstream, NULL for none), computes dX [M,K1], dW1 [K1,D], dR [M,D] (= dh),
 * dgamma [D] and dW2 [D,N2].  h and r are recomputed from X, W1, R. */
int oracle_block_bwd_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X, const double* W1,
                         const double* R, const double* gamma, const double* W2, double eps, const double* dz,
                         const double* dh_out, double* out_dX, double* out_dW1, double* out_dR,
                         double* out_dgamma, double* out_dW2, int nthreads);

/* Rotary position embedding, in place on y [M,N] ("rotate half" pairing; see oracle.c): for each head of
 * head_dim columns among the first n_rot, the pair (i, i + head_dim/2) is rotated by
 * (row mod seq_len) * base^(-2 i / head_dim). */
int oracle_rope_rows_f64(int64_t M, int64_t N, double* y, int64_t head_dim, int64_t n_rot, int64_t seq_len,
                         double base);

/* Cross-entropy of a vocabulary projection (see oracle.c): logits z = H W with H [M,D], W [D,V];
 * out_lse[i] = log sum_j exp(z_ij) (max-shifted); out_loss[i] = out_lse[i] - z[i][labels[i]], or 0 where
 * labels[i] < 0 (ignored).  Labels must be < V. */
int oracle_cross_entropy_f64(int64_t M, int64_t D, int64_t V, const double* H, const double* W,
                             const int64_t* labels, double* out_loss, double* out_lse, int nthreads);

/* Block-scaled (MX-style) e4m3 (see oracle.c): the scale exponent of a block with largest magnitude amax is the
 * smallest e with amax <= 448 * 2^e (0 for amax = 0; limited to [-127, 127]). */
int oracle_mx_scale_exp(double amax);
/* Quantise x [rows, cols] in blocks of `block` consecutive values of a row: exps[i][b] = the block's scale
 * exponent, codes[i][j] = e4m3(x[i][j] / 2^exps[i][j / block]).  cols must be a multiple of block. */
int oracle_mx_quant_rows_e4m3(int64_t rows, int64_t cols, int64_t block, const double* x, uint8_t* codes,
                              int32_t* exps);

/* Backward of y = silu(g) * u (see oracle.c): z [M, 2F] = [g | u], dout [M,D], Wd [F,D] (the next product's
 * weight, stored [in = F, out = D]); dy = dout Wd^T; out_dz [M, 2F] = [dy u silu'(g) | dy silu(g)]. */
int oracle_swiglu_bwd_f64(int64_t M, int64_t F, int64_t D, const double* dout, const double* Wd, const double* z,
                          double* out_dz, int nthreads);

/* silu(x) = x / (1 + exp(-x)) */
double oracle_silu(double x);

/* Round to the nearest bfloat16 value (8 significant bits, fp32 exponent range), ties to even;
 * overflow gives +-inf, NaN stays NaN. */
double oracle_bf16_round(double x);

/* OCP float8 e4m3fn: 1 sign, 4 exponent bits (bias 7), 3 mantissa bits, no infinities,
 * S.1111.111 is NaN, largest finite 448. */
double oracle_e4m3_decode(uint8_t code);
/* Round to nearest e4m3fn, ties to even, saturating to +-448; NaN -> 0x7F. */
uint8_t oracle_e4m3_encode(double x);

/* The codecs above applied element by element to arrays of n values. */
int oracle_bf16_round_array(int64_t n, const double* x, double* out);
int oracle_e4m3_encode_array(int64_t n, const double* x, uint8_t* out);
int oracle_e4m3_decode_array(int64_t n, const uint8_t* q, double* out);

/* Dequantise e4m3 codes: per-row scales  out[i][k] = decode(q[i][k]) * s[i]   (activations)
 *                        per-column       out[k][n] = decode(q[k][n]) * s[n]   (weights)      */
int oracle_dequant_rows_e4m3(int64_t rows, int64_t cols, const uint8_t* q, const float* s, double* out);
int oracle_dequant_cols_e4m3(int64_t rows, int64_t cols, const uint8_t* q, const float* s, double* out);

#ifdef __cplusplus
}
#endif
#endif
