/* oracle_driver.c -- runs every entry point of the fp64 oracle on small inputs, for a build with the address and
 * undefined-behaviour sanitizers (tests/test_sanitize_cpu.py).  Test infrastructure only.  Each call must return
 * its documented status; the values themselves are pinned by the Python pin tests, so only a few closed forms
 * are checked here (exit status 1 on a mismatch, the sanitizers abort on a memory or UB error). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "oracle.h"

static int failures = 0;
#define EXPECT(cond)                                                   \
  do {                                                                 \
    if (!(cond)) {                                                     \
      fprintf(stderr, "%s:%d: expected %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                      \
    }                                                                  \
  } while (0)

static double* filled(int64_t n, double scale, unsigned seed) {
  double* p = (double*)malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) {
    seed = seed * 1664525u + 1013904223u;
    p[i] = scale * ((double)(seed >> 8) / (double)(1u << 24) - 0.5);
  }
  return p;
}

int main(void) {
  const int64_t M = 5, K1 = 8, D = 12, N2 = 10;
  double *X = filled(M * K1, 2.0, 1), *W1 = filled(K1 * D, 0.5, 2), *R = filled(M * D, 1.0, 3);
  double *g = filled(D, 0.2, 4), *W2 = filled(D * N2, 0.5, 5);
  for (int64_t j = 0; j < D; ++j) g[j] += 1.0;
  double *h = malloc(sizeof(double) * M * D), *r = malloc(sizeof(double) * M), *y = malloc(sizeof(double) * M * N2);
  for (int epi = 0; epi < 2; ++epi) {
    EXPECT(oracle_block_unfused_f64(M, K1, D, N2, X, W1, R, g, W2, 1e-5, epi, h, r, y, 3) == 0);
    EXPECT(oracle_block_fused_f64(M, K1, D, N2, X, W1, R, g, W2, 1e-5, epi, h, r, y, 2) == 0);
    EXPECT(oracle_block_roundpts_f64(M, K1, D, N2, X, W1, R, g, W2, 1e-5, epi, NULL, NULL, y, 0) == 0);
  }
  EXPECT(oracle_block_fused_f64(-1, K1, D, N2, X, W1, R, g, W2, 1e-5, 0, h, r, y, 1) < 0);
  EXPECT(oracle_gemm_residual_f64(M, K1, D, X, W1, R, h, 4) == 0);
  EXPECT(oracle_gemm_residual_f64(M, K1, D, X, W1, NULL, h, 1) == 0);
  EXPECT(oracle_rms_scale_f64(M, D, h, 1e-5, r) == 0);
  double part[3 * 5];
  for (int i = 0; i < 15; ++i) part[i] = 1.0 + i;
  EXPECT(oracle_rms_from_partials_f64(3, M, part, D, 0.0, r) == 0);
  EXPECT(fabs(r[0] - 1.0 / sqrt((1.0 + 6.0 + 11.0) / 12.0)) < 1e-15);
  /* backward, with and without dh_out */
  double *dz = filled(M * N2, 1.0, 6), *dho = filled(M * D, 1.0, 7);
  double *dX = malloc(sizeof(double) * M * K1), *dW1 = malloc(sizeof(double) * K1 * D);
  double *dR = malloc(sizeof(double) * M * D), *dg = malloc(sizeof(double) * D), *dW2 = malloc(sizeof(double) * D * N2);
  EXPECT(oracle_block_bwd_f64(M, K1, D, N2, X, W1, R, g, W2, 1e-5, dz, dho, dX, dW1, dR, dg, dW2, 3) == 0);
  EXPECT(oracle_block_bwd_f64(M, K1, D, N2, X, W1, R, g, W2, 1e-5, dz, NULL, dX, dW1, dR, dg, dW2, 0) == 0);
  EXPECT(oracle_block_bwd_f64(M, K1, D, N2, X, W1, R, g, W2, -1.0, dz, NULL, dX, dW1, dR, dg, dW2, 0) < 0);
  /* rotary embedding: 2 heads of 4 columns, the second head past n_rot */
  double yr[3 * 8];
  for (int i = 0; i < 24; ++i) yr[i] = 1.0;
  EXPECT(oracle_rope_rows_f64(3, 8, yr, 4, 4, 2, 10000.0) == 0);
  EXPECT(yr[0] == 1.0 && yr[7] == 1.0 && yr[2 * 8 + 4] == 1.0);
  /* cross-entropy with an ignored row */
  int64_t labels[5] = {0, 3, -100, 9, 1};
  double loss[5], lse[5];
  EXPECT(oracle_cross_entropy_f64(M, D, N2, h, W2, labels, loss, lse, 2) == 0);
  EXPECT(loss[2] == 0.0);
  /* SwiGLU backward: z [M, 2F] with F = 6, dout [M, D], Wd [F, D] */
  double *z = filled(M * 12, 3.0, 8), *Wd = filled(6 * D, 0.5, 9), *dzz = malloc(sizeof(double) * M * 12);
  EXPECT(oracle_swiglu_bwd_f64(M, 6, D, dho, Wd, z, dzz, 3) == 0);
  /* codecs and the quantisers */
  EXPECT(oracle_silu(0.0) == 0.0);
  EXPECT(oracle_bf16_round(1.0 + 1.0 / 512.0) == 1.0);
  EXPECT(oracle_e4m3_encode(448.0) == 0x7E && oracle_e4m3_encode(1e9) == 0x7E && oracle_e4m3_encode(NAN) == 0x7F);
  EXPECT(isnan(oracle_e4m3_decode(0x7F)) && oracle_e4m3_decode(0x01) == ldexp(1.0, -9));
  double xs[6] = {0.0, -0.0, 1.0, 1e-40, 3e38, -448.5};
  double rs[6];
  uint8_t cs[6];
  EXPECT(oracle_bf16_round_array(6, xs, rs) == 0 && oracle_e4m3_encode_array(6, xs, cs) == 0);
  EXPECT(oracle_e4m3_decode_array(6, cs, rs) == 0 && rs[2] == 1.0);
  EXPECT(oracle_bf16_round_array(-1, xs, rs) < 0);
  uint8_t q[2 * 3] = {0x38, 0x40, 0x7E, 0x00, 0x81, 0xB8};
  float sr[2] = {2.0f, 0.5f}, sc[3] = {1.0f, 2.0f, 4.0f};
  double dq[6];
  EXPECT(oracle_dequant_rows_e4m3(2, 3, q, sr, dq) == 0 && dq[0] == 2.0);
  EXPECT(oracle_dequant_cols_e4m3(2, 3, q, sc, dq) == 0 && dq[1] == 4.0);
  EXPECT(oracle_mx_scale_exp(448.0) == 0 && oracle_mx_scale_exp(449.0) == 1 && oracle_mx_scale_exp(0.0) == 0);
  double xq[2 * 64];
  for (int i = 0; i < 128; ++i) xq[i] = (i - 64) * 0.37;
  uint8_t codes[128];
  int32_t exps[4];
  EXPECT(oracle_mx_quant_rows_e4m3(2, 64, 32, xq, codes, exps) == 0);
  EXPECT(oracle_mx_quant_rows_e4m3(2, 60, 32, xq, codes, exps) < 0);
  EXPECT(oracle_default_threads() >= 1);
  free(X); free(W1); free(R); free(g); free(W2); free(h); free(r); free(y); free(dz); free(dho); free(dX); free(dW1);
  free(dR); free(dg); free(dW2); free(z); free(Wd); free(dzz);
  if (failures) fprintf(stderr, "%d expectation(s) failed\n", failures);
  else printf("oracle driver: all entry points ran\n");
  return failures ? 1 : 0;
}
