/*
 * oracle.c -- plain fp64 CPU reference for the GEMM -> residual -> RMSNorm -> GEMM block.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Written to be checked by eye, not to be fast: the products are
 * textbook triple loops (the k loop sits outside the column loop so the inner loop runs along a row, which
 * leaves every output's sum in plain k order), rows are shared between threads, and nothing is blocked,
 * fused or reordered beyond that.
 *
 * Source of the method: the CODA write-up ("CODA: new research optimizes Transformer training with
 * GEMM-epilogue programming", KuCoin news flash; the same article on itsolotime.com), section "CODA: the
 * treasure hidden in the epilogue": a GEMM, a residual add, RMS normalisation and a second GEMM; the per-row
 * RMS factor is a scalar per row, so it commutes with the second GEMM and can be applied after it, with a
 * light reduction merging per-tile partial RMS values; the same section says SwiGLU admits a similar
 * rewrite.
 */
#define _GNU_SOURCE
#include "oracle.h"

#include <fenv.h>
#include <math.h>
#include <pthread.h>
#include <sched.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

int oracle_default_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------------------------------------ */
/* scalar helpers                                                                                   */

double oracle_silu(double x) { return x / (1.0 + exp(-x)); }

/* Round x to the grid of a binary format with `sig` significant bits whose smallest normal exponent is
 * emin (the weight of the leading bit of the smallest normal number is 2^emin).  Ties go to even because
 * nearbyint follows the default rounding mode, round-to-nearest-even. */
static double round_to_grid(double x, int sig, int emin) {
  if (x == 0.0 || !isfinite(x)) return x;
  int e;
  frexp(x, &e);          /* |x| = m * 2^e with 0.5 <= m < 1: the leading bit has weight 2^(e-1) */
  int lead = e - 1;
  if (lead < emin) lead = emin; /* subnormal range: fixed spacing */
  double ulp = ldexp(1.0, lead - (sig - 1));
  return nearbyint(x / ulp) * ulp;
}

double oracle_bf16_round(double x) {
  if (isnan(x)) return x;
  /* bfloat16: 8 significant bits, same exponent range as fp32 (smallest normal 2^-126). */
  double r = round_to_grid(x, 8, -126);
  const double bf16_max = 3.38953138925153547590470800371487866880e+38; /* (2 - 2^-7) * 2^127 */
  if (fabs(r) > bf16_max) return copysign(INFINITY, x);
  return r;
}

double oracle_e4m3_decode(uint8_t code) {
  int sign = code >> 7;
  int exp_bits = (code >> 3) & 0xF;
  int mant = code & 0x7;
  double v;
  if (exp_bits == 0xF && mant == 0x7) return NAN; /* the only NaN pattern; e4m3fn has no infinities */
  if (exp_bits == 0)
    v = ldexp((double)mant, -9); /* subnormal: mant/8 * 2^(1-7) */
  else
    v = ldexp(1.0 + mant / 8.0, exp_bits - 7);
  return sign ? -v : v;
}

uint8_t oracle_e4m3_encode(double x) {
  if (isnan(x)) return 0x7F;
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  double a = fabs(x);
  if (a > 448.0) a = 448.0;             /* saturate */
  double r = round_to_grid(a, 4, -6);   /* 4 significant bits, smallest normal 2^-6 */
  if (r > 448.0) r = 448.0;
  if (r == 0.0) return sign;
  int e;
  frexp(r, &e);
  int lead = e - 1;
  if (lead < -6) { /* subnormal: value = mant * 2^-9 */
    int mant = (int)nearbyint(r / ldexp(1.0, -9));
    return sign | (uint8_t)mant;
  }
  int mant = (int)nearbyint((r / ldexp(1.0, lead) - 1.0) * 8.0);
  return sign | (uint8_t)(((lead + 7) << 3) | mant);
}

/* The three codecs above applied element by element to arrays (the same scalar functions in a loop). */
int oracle_bf16_round_array(int64_t n, const double* x, double* out) {
  if (n < 0 || (n && (!x || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_round(x[i]);
  return 0;
}

int oracle_e4m3_encode_array(int64_t n, const double* x, uint8_t* out) {
  if (n < 0 || (n && (!x || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
  return 0;
}

int oracle_e4m3_decode_array(int64_t n, const uint8_t* q, double* out) {
  if (n < 0 || (n && (!q || !out))) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(q[i]);
  return 0;
}

int oracle_dequant_rows_e4m3(int64_t rows, int64_t cols, const uint8_t* q, const float* s, double* out) {
  if (rows < 0 || cols < 0 || !q || !s || !out) return -1;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t k = 0; k < cols; ++k) out[i * cols + k] = oracle_e4m3_decode(q[i * cols + k]) * (double)s[i];
  return 0;
}

int oracle_dequant_cols_e4m3(int64_t rows, int64_t cols, const uint8_t* q, const float* s, double* out) {
  if (rows < 0 || cols < 0 || !q || !s || !out) return -1;
  for (int64_t k = 0; k < rows; ++k)
    for (int64_t n = 0; n < cols; ++n) out[k * cols + n] = oracle_e4m3_decode(q[k * cols + n]) * (double)s[n];
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* row-parallel driver                                                                              */

typedef void (*row_fn)(void* ctx, int64_t row, double* scratch);

typedef struct {
  row_fn fn;
  void* ctx;
  int64_t row_begin, row_end;
  size_t scratch_doubles;
  int failed;
} row_job;

static void* row_worker(void* p) {
  row_job* job = (row_job*)p;
  double* scratch = NULL;
  if (job->scratch_doubles) {
    scratch = (double*)malloc(job->scratch_doubles * sizeof(double));
    if (!scratch) { job->failed = 1; return NULL; }
  }
  for (int64_t i = job->row_begin; i < job->row_end; ++i) job->fn(job->ctx, i, scratch);
  free(scratch);
  return NULL;
}

/* Runs fn(ctx, i, scratch) for every row i in [0, M), spread over contiguous row ranges. */
static int for_each_row(int64_t M, int nthreads, size_t scratch_doubles, row_fn fn, void* ctx) {
  if (nthreads <= 0) nthreads = oracle_default_threads();
  if (nthreads > M) nthreads = M > 0 ? (int)M : 1;
  row_job* jobs = (row_job*)calloc((size_t)nthreads, sizeof(row_job));
  pthread_t* tids = (pthread_t*)calloc((size_t)nthreads, sizeof(pthread_t));
  if (!jobs || !tids) { free(jobs); free(tids); return -2; }
  int64_t per = (M + nthreads - 1) / nthreads;
  int started = 0, failed = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t].fn = fn;
    jobs[t].ctx = ctx;
    jobs[t].row_begin = t * per < M ? t * per : M;
    jobs[t].row_end = (t + 1) * per < M ? (t + 1) * per : M;
    jobs[t].scratch_doubles = scratch_doubles;
    if (pthread_create(&tids[t], NULL, row_worker, &jobs[t]) != 0) { /* run it here instead */
      row_worker(&jobs[t]);
      tids[t] = 0;
      continue;
    }
    ++started;
  }
  for (int t = 0; t < nthreads; ++t) {
    if (tids[t]) pthread_join(tids[t], NULL);
    failed |= jobs[t].failed;
  }
  (void)started;
  free(jobs);
  free(tids);
  return failed ? -2 : 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* first product plus residual: h_ij = sum_k X_ik W1_kj + R_ij                                     */

typedef struct {
  int64_t K1, D;
  const double *X, *W1, *R;
  double* h;
} gemm_res_ctx;

static void gemm_res_row(void* p, int64_t i, double* scratch) {
  gemm_res_ctx* c = (gemm_res_ctx*)p;
  (void)scratch;
  double* hi = c->h + i * c->D;
  for (int64_t j = 0; j < c->D; ++j) hi[j] = 0.0;
  for (int64_t k = 0; k < c->K1; ++k) {
    double x = c->X[i * c->K1 + k];
    const double* w = c->W1 + k * c->D;
    for (int64_t j = 0; j < c->D; ++j) hi[j] += x * w[j];
  }
  if (c->R)
    for (int64_t j = 0; j < c->D; ++j) hi[j] += c->R[i * c->D + j];
}

int oracle_gemm_residual_f64(int64_t M, int64_t K1, int64_t D, const double* X, const double* W1,
                             const double* R, double* out_h, int nthreads) {
  if (M < 0 || K1 < 0 || D < 0 || !X || !W1 || !out_h) return -1;
  gemm_res_ctx c = {K1, D, X, W1, R, out_h};
  return for_each_row(M, nthreads, 0, gemm_res_row, &c);
}

/* ------------------------------------------------------------------------------------------------ */
/* RMS row scale                                                                                    */

static double rms_scale_of_row(const double* h, int64_t D, double eps) {
  double ss = 0.0;
  for (int64_t j = 0; j < D; ++j) ss += h[j] * h[j];
  return 1.0 / sqrt(ss / (double)D + eps);
}

int oracle_rms_scale_f64(int64_t M, int64_t D, const double* h, double eps, double* out_r) {
  if (M < 0 || D <= 0 || !h || !out_r) return -1;
  for (int64_t i = 0; i < M; ++i) out_r[i] = rms_scale_of_row(h + i * D, D, eps);
  return 0;
}

int oracle_rms_from_partials_f64(int64_t T, int64_t M, const double* part, int64_t D, double eps,
                                 double* out_r) {
  if (T <= 0 || M < 0 || D <= 0 || !part || !out_r) return -1;
  for (int64_t i = 0; i < M; ++i) {
    double ss = 0.0;
    for (int64_t t = 0; t < T; ++t) ss += part[t * M + i];
    out_r[i] = 1.0 / sqrt(ss / (double)D + eps);
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* the whole block                                                                                  */

enum { FORM_UNFUSED = 0, FORM_FUSED = 1, FORM_ROUNDPTS = 2 };

typedef struct {
  int form;
  int64_t K1, D, N2;
  const double *X, *W1, *R, *gamma, *W2;
  const double* W2g; /* diag(gamma) W2 (fused forms), bf16-rounded for the round-points form */
  double eps;
  int epi;
  double *h, *r, *y;
} block_ctx;

/* scratch per thread: h row (D), second operand row (D), z row (N2) */
static void block_row(void* p, int64_t i, double* scratch) {
  block_ctx* c = (block_ctx*)p;
  const int64_t K1 = c->K1, D = c->D, N2 = c->N2;
  double* hrow = scratch;
  double* arow = scratch + D;
  double* z = scratch + 2 * D;

  /* h = X W1 + R */
  for (int64_t j = 0; j < D; ++j) hrow[j] = 0.0;
  for (int64_t k = 0; k < K1; ++k) {
    double x = c->X[i * K1 + k];
    const double* w = c->W1 + k * D;
    for (int64_t j = 0; j < D; ++j) hrow[j] += x * w[j];
  }
  for (int64_t j = 0; j < D; ++j) hrow[j] += c->R[i * D + j];

  /* r = 1 / sqrt(mean(h^2) + eps), from the unrounded h in every form */
  double r = rms_scale_of_row(hrow, D, c->eps);

  const double* w2;
  if (c->form == FORM_UNFUSED) {
    /* normalise first: n_j = h_j * r * gamma_j, then z = n W2 */
    for (int64_t j = 0; j < D; ++j) arow[j] = hrow[j] * r * c->gamma[j];
    w2 = c->W2;
  } else if (c->form == FORM_FUSED) {
    /* reparameterised: the product runs on h itself against W2' = diag(gamma) W2, and r scales the
     * product's row afterwards */
    for (int64_t j = 0; j < D; ++j) arow[j] = hrow[j];
    w2 = c->W2g;
  } else {
    /* round-points form: gamma broadcast onto h and rounded once to bf16, (h * gamma) W2, then r */
    for (int64_t j = 0; j < D; ++j) arow[j] = oracle_bf16_round(hrow[j] * c->gamma[j]);
    w2 = c->W2;
  }
  for (int64_t n = 0; n < N2; ++n) z[n] = 0.0;
  for (int64_t j = 0; j < D; ++j) {
    double a = arow[j];
    const double* w = w2 + j * N2;
    for (int64_t n = 0; n < N2; ++n) z[n] += a * w[n];
  }
  if (c->form != FORM_UNFUSED)
    for (int64_t n = 0; n < N2; ++n) z[n] *= r;

  /* epilogue */
  if (c->epi == ORACLE_EPI_IDENTITY) {
    for (int64_t n = 0; n < N2; ++n) {
      double v = z[n];
      c->y[i * N2 + n] = c->form == FORM_ROUNDPTS ? oracle_bf16_round(v) : v;
    }
  } else {
    const int64_t half = N2 / 2;
    for (int64_t n = 0; n < half; ++n) {
      double v = oracle_silu(z[n]) * z[half + n]; /* gate in the first half, up in the second */
      c->y[i * half + n] = c->form == FORM_ROUNDPTS ? oracle_bf16_round(v) : v;
    }
  }

  if (c->h)
    for (int64_t j = 0; j < D; ++j) c->h[i * D + j] = hrow[j];
  if (c->r) c->r[i] = r;
}

static int run_block(int form, int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                     const double* W1, const double* R, const double* gamma, const double* W2, double eps,
                     int epi, double* out_h, double* out_r, double* out_y, int nthreads) {
  if (M < 0 || K1 <= 0 || D <= 0 || N2 <= 0) return -1;
  if (!X || !W1 || !R || !gamma || !W2 || !out_y) return -1;
  if (epi != ORACLE_EPI_IDENTITY && epi != ORACLE_EPI_SWIGLU) return -1;
  if (epi == ORACLE_EPI_SWIGLU && (N2 % 2) != 0) return -1;
  if (!(eps >= 0.0)) return -1;

  double* W2g = NULL;
  if (form == FORM_FUSED) {
    /* W2'_jn = gamma_j * W2_jn */
    W2g = (double*)malloc((size_t)D * (size_t)N2 * sizeof(double));
    if (!W2g) return -2;
    for (int64_t j = 0; j < D; ++j)
      for (int64_t n = 0; n < N2; ++n) W2g[j * N2 + n] = gamma[j] * W2[j * N2 + n];
  }
  block_ctx c = {form, K1, D, N2, X, W1, R, gamma, W2, W2g, eps, epi, out_h, out_r, out_y};
  int rc = for_each_row(M, nthreads, (size_t)(2 * D + N2), block_row, &c);
  free(W2g);
  return rc;
}

int oracle_block_unfused_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                             const double* W1, const double* R, const double* gamma, const double* W2,
                             double eps, int epi, double* out_h, double* out_r, double* out_y,
                             int nthreads) {
  return run_block(FORM_UNFUSED, M, K1, D, N2, X, W1, R, gamma, W2, eps, epi, out_h, out_r, out_y, nthreads);
}

int oracle_block_fused_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                           const double* W1, const double* R, const double* gamma, const double* W2,
                           double eps, int epi, double* out_h, double* out_r, double* out_y,
                           int nthreads) {
  return run_block(FORM_FUSED, M, K1, D, N2, X, W1, R, gamma, W2, eps, epi, out_h, out_r, out_y, nthreads);
}

int oracle_block_roundpts_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X,
                              const double* W1, const double* R, const double* gamma, const double* W2,
                              double eps, int epi, double* out_h, double* out_r, double* out_y,
                              int nthreads) {
  return run_block(FORM_ROUNDPTS, M, K1, D, N2, X, W1, R, gamma, W2, eps, epi, out_h, out_r, out_y, nthreads);
}

/* ------------------------------------------------------------------------------------------------ */
/* backward of the block                                                                            */
/*
 * The CODA write-up (section "CODA: the treasure hidden in the epilogue", and its results section on the
 * backward kernels) applies the same epilogue programming to back-propagation.  The reference here is the
 * textbook chain rule of the forward definition above, in the unfused order, with the gradient dz of the
 * second product's output (before any epilogue) and the gradient dh_out arriving at h from downstream
 * (h is the residual stream):
 *   h = X W1 + R;  r_i = 1/sqrt(mean_j h_ij^2 + eps);  n = r h;  u = n * gamma;  z = u W2
 *   du = dz W2^T;  dW2 = u^T dz;  dgamma_j = sum_i du_ij n_ij;  dn = du * gamma
 *   dh_ij = r_i (dn_ij - n_ij mean_j'(dn_ij' n_ij')) + dh_out_ij;  dR = dh;  dX = dh W1^T;  dW1 = X^T dh
 * Sums over rows run in row order, sums over columns in column order.
 */

typedef struct {
  int64_t K1, D, N2;
  const double *X, *W1, *R, *gamma, *W2, *dz, *dh_out;
  double eps;
  double *u, *n, *du, *dh, *dX;
} bwd_ctx;

/* scratch per thread: h row (D) */
static void bwd_row(void* p, int64_t i, double* scratch) {
  bwd_ctx* c = (bwd_ctx*)p;
  const int64_t K1 = c->K1, D = c->D, N2 = c->N2;
  double* hrow = scratch;
  for (int64_t j = 0; j < D; ++j) hrow[j] = 0.0;
  for (int64_t k = 0; k < K1; ++k) {
    double x = c->X[i * K1 + k];
    const double* w = c->W1 + k * D;
    for (int64_t j = 0; j < D; ++j) hrow[j] += x * w[j];
  }
  for (int64_t j = 0; j < D; ++j) hrow[j] += c->R[i * D + j];
  const double r = rms_scale_of_row(hrow, D, c->eps);
  double* n = c->n + i * D;
  double* u = c->u + i * D;
  double* du = c->du + i * D;
  double* dh = c->dh + i * D;
  for (int64_t j = 0; j < D; ++j) {
    n[j] = r * hrow[j];
    u[j] = n[j] * c->gamma[j];
  }
  /* du_ij = sum_n dz_in W2_jn */
  const double* dzi = c->dz + i * N2;
  for (int64_t j = 0; j < D; ++j) {
    const double* w = c->W2 + j * N2;
    double s = 0.0;
    for (int64_t q = 0; q < N2; ++q) s += dzi[q] * w[q];
    du[j] = s;
  }
  /* RMSNorm backward: dn = du * gamma; dh = r (dn - n mean(dn n)) (+ dh_out) */
  double dot = 0.0;
  for (int64_t j = 0; j < D; ++j) dot += du[j] * c->gamma[j] * n[j];
  const double mean = dot / (double)D;
  for (int64_t j = 0; j < D; ++j) {
    double v = r * (du[j] * c->gamma[j] - n[j] * mean);
    if (c->dh_out) v += c->dh_out[i * D + j];
    dh[j] = v;
  }
  /* dX_ik = sum_j dh_ij W1_kj */
  for (int64_t k = 0; k < K1; ++k) {
    const double* w = c->W1 + k * D;
    double s = 0.0;
    for (int64_t j = 0; j < D; ++j) s += dh[j] * w[j];
    c->dX[i * K1 + k] = s;
  }
}

typedef struct {
  int64_t M, K1, D, N2;
  const double *X, *dz;
  const double *u, *n, *du, *dh;
  double *dW1, *dgamma, *dW2;
} bwd_w_ctx;

/* one row j of dW2 [D,N2] and dgamma_j; sums over the data rows i in order */
static void bwd_w2_row(void* p, int64_t j, double* scratch) {
  bwd_w_ctx* c = (bwd_w_ctx*)p;
  (void)scratch;
  const int64_t D = c->D, N2 = c->N2;
  double* out = c->dW2 + j * N2;
  for (int64_t q = 0; q < N2; ++q) out[q] = 0.0;
  double g = 0.0;
  for (int64_t i = 0; i < c->M; ++i) {
    const double a = c->u[i * D + j];
    const double* dzi = c->dz + i * N2;
    for (int64_t q = 0; q < N2; ++q) out[q] += a * dzi[q];
    g += c->du[i * D + j] * c->n[i * D + j];
  }
  c->dgamma[j] = g;
}

/* one row k of dW1 [K1,D]: dW1_kj = sum_i X_ik dh_ij */
static void bwd_w1_row(void* p, int64_t k, double* scratch) {
  bwd_w_ctx* c = (bwd_w_ctx*)p;
  (void)scratch;
  const int64_t K1 = c->K1, D = c->D;
  double* out = c->dW1 + k * D;
  for (int64_t j = 0; j < D; ++j) out[j] = 0.0;
  for (int64_t i = 0; i < c->M; ++i) {
    const double x = c->X[i * K1 + k];
    const double* d = c->dh + i * D;
    for (int64_t j = 0; j < D; ++j) out[j] += x * d[j];
  }
}

int oracle_block_bwd_f64(int64_t M, int64_t K1, int64_t D, int64_t N2, const double* X, const double* W1,
                         const double* R, const double* gamma, const double* W2, double eps, const double* dz,
                         const double* dh_out, double* out_dX, double* out_dW1, double* out_dR,
                         double* out_dgamma, double* out_dW2, int nthreads) {
  if (M < 0 || K1 <= 0 || D <= 0 || N2 <= 0) return -1;
  if (!X || !W1 || !R || !gamma || !W2 || !dz || !out_dX || !out_dW1 || !out_dR || !out_dgamma || !out_dW2)
    return -1;
  if (!(eps >= 0.0)) return -1;
  const size_t md = (size_t)M * (size_t)D;
  double* buf = (double*)malloc(3 * md * sizeof(double) + 1);
  if (!buf) return -2;
  double *u = buf, *n = buf + md, *du = buf + 2 * md;
  bwd_ctx c = {K1, D, N2, X, W1, R, gamma, W2, dz, dh_out, eps, u, n, du, out_dR, out_dX};
  int rc = for_each_row(M, nthreads, (size_t)D, bwd_row, &c);
  if (rc == 0) {
    bwd_w_ctx w = {M, K1, D, N2, X, dz, u, n, du, out_dR, out_dW1, out_dgamma, out_dW2};
    rc = for_each_row(D, nthreads, 0, bwd_w2_row, &w);
    if (rc == 0) rc = for_each_row(K1, nthreads, 0, bwd_w1_row, &w);
  }
  free(buf);
  return rc;
}

/* ------------------------------------------------------------------------------------------------ */
/* rotary position embedding on the rows of a product                                               */
/*
 * The CODA write-up (section "CODA: the treasure hidden in the epilogue"; section "Five blocks and a Lego
 * language": elementwise transforms) lists RoPE among the operations that run in a GEMM epilogue.  The pages
 * fix no convention; this one is the "rotate half" form used by LLaMA-family checkpoints: for each head of
 * head_dim columns among the first n_rot columns, the pair (i, i + head_dim/2), i < head_dim/2, is rotated by
 * theta = pos * base^(-2 i / head_dim) with pos = row mod seq_len:
 *   (a, b) -> (a cos theta - b sin theta, b cos theta + a sin theta).
 */
int oracle_rope_rows_f64(int64_t M, int64_t N, double* y, int64_t head_dim, int64_t n_rot, int64_t seq_len,
                         double base) {
  if (M < 0 || N <= 0 || !y || head_dim <= 0 || (head_dim % 2) != 0 || n_rot < 0 || n_rot > N ||
      (n_rot % head_dim) != 0 || seq_len <= 0 || !(base > 0.0))
    return -1;
  const int64_t half = head_dim / 2;
  for (int64_t m = 0; m < M; ++m) {
    const double pos = (double)(m % seq_len);
    double* row = y + m * N;
    for (int64_t h0 = 0; h0 < n_rot; h0 += head_dim) {
      for (int64_t i = 0; i < half; ++i) {
        const double theta = pos * pow(base, -2.0 * (double)i / (double)head_dim);
        const double c = cos(theta), s = sin(theta);
        const double a = row[h0 + i], b = row[h0 + i + half];
        row[h0 + i] = a * c - b * s;
        row[h0 + i + half] = b * c + a * s;
      }
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* cross-entropy of a vocabulary projection                                                         */
/*
 * The CODA write-up names cross-entropy among the operations its epilogue programming covers (section "CODA:
 * the treasure hidden in the epilogue"), with reductions done inside the epilogue and merged by a light
 * kernel afterwards (section "Five blocks and a Lego language").  What is computed is the plain definition:
 * logits z = H W (H [M,D], W [D,V]); lse_i = log sum_j exp(z_ij), evaluated as m_i + log sum_j exp(z_ij - m_i)
 * with m_i = max_j z_ij so that no exponential overflows; loss_i = lse_i - z_{i,label_i}.  A negative label
 * marks an ignored position: its loss is 0 (its lse is still produced).
 */
typedef struct {
  int64_t D, V;
  const double *H, *W;
  const int64_t* labels;
  double *loss, *lse;
} ce_ctx;

static void ce_row(void* p, int64_t i, double* z) {
  ce_ctx* c = (ce_ctx*)p;
  for (int64_t j = 0; j < c->V; ++j) z[j] = 0.0;
  for (int64_t k = 0; k < c->D; ++k) {
    const double h = c->H[i * c->D + k];
    const double* w = c->W + k * c->V;
    for (int64_t j = 0; j < c->V; ++j) z[j] += h * w[j];
  }
  double m = -INFINITY;
  for (int64_t j = 0; j < c->V; ++j)
    if (z[j] > m) m = z[j];
  double s = 0.0;
  for (int64_t j = 0; j < c->V; ++j) s += exp(z[j] - m);
  const double l = m + log(s);
  const int64_t label = c->labels[i];
  c->lse[i] = l;
  c->loss[i] = label < 0 ? 0.0 : l - z[label];
}

int oracle_cross_entropy_f64(int64_t M, int64_t D, int64_t V, const double* H, const double* W,
                             const int64_t* labels, double* out_loss, double* out_lse, int nthreads) {
  if (M < 0 || D < 0 || V < 1 || !H || !W || !labels || !out_loss || !out_lse) return -1;
  for (int64_t i = 0; i < M; ++i)
    if (labels[i] >= V) return -1;
  ce_ctx c = {D, V, H, W, labels, out_loss, out_lse};
  return for_each_row(M, nthreads, (size_t)V, ce_row, &c);
}

/* ------------------------------------------------------------------------------------------------ */
/* block-scaled (MX-style) e4m3 quantisation of rows                                                */
/*
 * A variant of the e4m3 path in which the second product's A operand carries one power-of-two scale per 32
 * consecutive values of a row instead of one scale per row, so that the first product's epilogue can
 * quantise its own tile with no cross-tile amax (the pages give no quantisation granularity; they name fp8
 * operands and per-row activation scales among the epilogue's vector loads, section "Five blocks and a Lego
 * language").  Reading: the scale of a block is 2^e with e the smallest integer such that
 * amax_block <= 448 * 2^e (so no value needs saturating), e = 0 for an all-zero block, e limited to
 * [-127, 127] (the range of an 8-bit power-of-two scale); code = e4m3(x / 2^e), rounded to nearest even.
 */
int oracle_mx_scale_exp(double amax) {
  if (!(amax > 0.0)) return 0;
  if (isinf(amax)) return 127;
  int e2;
  const double m = frexp(amax, &e2); /* amax = m 2^e2, 0.5 <= m < 1 */
  /* amax <= 448 2^e  <=>  m 2^e2 <= 1.75 2^(e + 8)  <=>  e >= e2 - 9 when 2m <= 1.75, else e >= e2 - 8 */
  int e = (2.0 * m <= 1.75) ? e2 - 9 : e2 - 8;
  if (e < -127) e = -127;
  if (e > 127) e = 127;
  return e;
}

int oracle_mx_quant_rows_e4m3(int64_t rows, int64_t cols, int64_t block, const double* x, uint8_t* codes,
                              int32_t* exps) {
  if (rows < 0 || cols < 0 || block <= 0 || (cols % block) != 0 || !x || !codes || !exps) return -1;
  const int64_t nb = cols / block;
  for (int64_t i = 0; i < rows; ++i) {
    for (int64_t b = 0; b < nb; ++b) {
      const double* v = x + i * cols + b * block;
      double amax = 0.0;
      for (int64_t j = 0; j < block; ++j)
        if (fabs(v[j]) > amax) amax = fabs(v[j]);
      const int e = oracle_mx_scale_exp(amax);
      exps[i * nb + b] = e;
      for (int64_t j = 0; j < block; ++j) codes[i * cols + b * block + j] = oracle_e4m3_encode(ldexp(v[j], -e));
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------------------------------ */
/* backward of the SwiGLU epilogue                                                                  */
/*
 * The write-up reports the backward of the SwiGLU block among its largest gains (section "Experimental
 * results") and says a forward epilogue has a backward with the same structure (section "CODA: the treasure
 * hidden in the epilogue"); it gives no formulas.  What is computed is the chain rule of y = silu(g) * u with
 * z = [g | u] (the gate and up halves of the second product's output, F columns each):
 *   dy = dout Wd^T            (dout [M,D], Wd [F,D]: the gradient reaching y through the next product, whose
 *                             weight maps the F columns of y to D; Wd is stored [in = F, out = D])
 *   dg = dy * u * silu'(g),   silu'(g) = s (1 + g (1 - s)),  s = 1 / (1 + exp(-g))
 *   du = dy * silu(g)
 * and dz = [dg | du] [M, 2F].
 */
typedef struct {
  int64_t F, D;
  const double *dout, *Wd, *z;
  double* dz;
} swiglu_bwd_ctx;

static void swiglu_bwd_row(void* p, int64_t i, double* scratch) {
  swiglu_bwd_ctx* c = (swiglu_bwd_ctx*)p;
  (void)scratch;
  const int64_t F = c->F, D = c->D;
  for (int64_t f = 0; f < F; ++f) {
    double dy = 0.0;
    for (int64_t d = 0; d < D; ++d) dy += c->dout[i * D + d] * c->Wd[f * D + d];
    const double g = c->z[i * 2 * F + f], u = c->z[i * 2 * F + F + f];
    const double s = 1.0 / (1.0 + exp(-g));
    c->dz[i * 2 * F + f] = dy * u * s * (1.0 + g * (1.0 - s));
    c->dz[i * 2 * F + F + f] = dy * g * s;
  }
}

int oracle_swiglu_bwd_f64(int64_t M, int64_t F, int64_t D, const double* dout, const double* Wd, const double* z,
                          double* out_dz, int nthreads) {
  if (M < 0 || F <= 0 || D <= 0 || !dout || !Wd || !z || !out_dz) return -1;
  swiglu_bwd_ctx c = {F, D, dout, Wd, z, out_dz};
  return for_each_row(M, nthreads, 0, swiglu_bwd_row, &c);
}
