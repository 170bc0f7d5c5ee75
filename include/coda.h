/*
 * coda.h -- C ABI of the MI355X (gfx950) fused GEMM -> residual -> RMSNorm -> GEMM block.
 *
 * The method (CODA write-up, "CODA: new research optimizes Transformer training with GEMM-epilogue
 * programming", section "CODA: the treasure hidden in the epilogue"):
 *   h  = X W1 + R                      formed in the first GEMM's epilogue while the accumulator tile is
 *                                      still in registers; h is stored (it is the residual stream and the
 *                                      activation kept for backward, section "Five blocks and a Lego
 *                                      language": tiled matrix store)
 *   hg = h * gamma                     the RMSNorm weight broadcast along the rows in the same epilogue
 *                                      (vector-load primitive, same section), stored in the workspace
 *   part[t][i] = sum_{j in tile t} h_ij^2   per-row, per-column-tile partial sums from the same epilogue
 *                                      (block reduction primitive: "local RMS")
 *   r_i = 1 / sqrt(sum_t part[t][i] / D + eps)   a light reduction kernel
 *   y  = epi(r_i * (hg W2)) = epi(r_i * (h diag(gamma) W2)): the per-row scale commutes with the second
 *                                      GEMM, so r is applied in its epilogue, optionally followed by SwiGLU
 *                                      on a fused gate|up product (the same section: SwiGLU admits the same
 *                                      rewrite).
 * No normalised tensor is ever written to or read from HBM.  gamma is applied on the h side rather than
 * folded into W2's tiles: on gfx950 scaling the W2 tiles in the second GEMM costs 13-19% of its time (the
 * scaling work does not overlap the matrix cores), while writing hg costs one [M,D] bf16 store.
 *
 * Conventions shared by every entry point
 *   - All matrices are dense and row-major with no padding: X [M,K1], W1 [K1,D] (weights are [in,out]),
 *     R, out_h [M,D], gamma [D] fp32, W2 [D,N2], out_y [M,N2] (identity) or [M,N2/2] (SwiGLU: columns
 *     [0,N2/2) of W2 are the gate projection, [N2/2,N2) the up projection, y = silu(gate) * up with
 *     silu(x) = x / (1 + exp(-x)), r applied to both halves before silu).
 *   - bf16 tensors are IEEE bfloat16 bit patterns (uint16); fp8 tensors are OCP e4m3fn bytes with fp32
 *     scales: dequantised value = code * scale, per row for activations (sx [M]) and per output column for
 *     weights (sw1 [D], sw2 [N2]).
 *   - Every pointer is a device pointer (HBM of the current HIP device), 16-byte aligned.  The caller owns
 *     every buffer, including the workspace (size from coda_workspace_bytes).  The library allocates
 *     nothing, keeps no pointer after returning and has no mutable global state except a thread-local
 *     error string.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL is the default stream) and is asynchronous: buffers
 *     must stay alive until the stream has passed the call.  Calls on distinct streams with distinct
 *     workspaces may run concurrently; calls sharing a workspace must be ordered by the caller.
 *   - Shape rules: M >= 1 (any value; the last row tile is masked); K1 a multiple of 128; D and N2
 *     multiples of 256 (for SwiGLU N2/2 is then a multiple of 128).  Other shapes return
 *     CODA_ERR_UNSUPPORTED.  eps must be finite and >= 0.
 *   - Aliasing: no output may overlap an input or another output, except the exact in-place residual
 *     update out_h == R (same pointer), which is supported.
 *   - Errors: arguments are validated synchronously before anything is enqueued; a failed validation
 *     returns its code and enqueues nothing.  A launch failure returns CODA_ERR_HIP.  Device faults surface
 *     at the caller's next synchronisation.  No C++ exception crosses this boundary and nothing aborts.
 *     coda_last_error() gives a human-readable detail of the last failure on the calling thread.
 *   - Debugging: with CODA_SYNC_CHECK=1 in the environment every launch is followed by a device synchronisation
 *     and an error check, so a device-side failure is reported (CODA_ERR_HIP, the launch named in
 *     coda_last_error()) by the call that caused it.  It serialises the caller's streams and fails under graph
 *     capture; never set it for timing.
 */
#ifndef CODA_H
#define CODA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CODA_ABI_VERSION 1

typedef enum {
  CODA_OK = 0,
  CODA_ERR_INVALID_ARG = 1, /* null or misaligned pointer, bad dimension, bad eps or epilogue kind */
  CODA_ERR_UNSUPPORTED = 2, /* a shape the kernels do not tile (see shape rules) */
  CODA_ERR_ALIAS = 3,       /* overlapping input/output buffers (other than out_h == R) */
  CODA_ERR_WORKSPACE = 4,   /* workspace missing or smaller than coda_workspace_bytes() */
  CODA_ERR_HIP = 5,         /* the HIP runtime reported an error */
  CODA_ERR_INTERNAL = 6     /* unexpected internal failure */
} coda_status;

typedef enum { CODA_EPI_IDENTITY = 0, CODA_EPI_SWIGLU = 1 } coda_epi_kind;

/* Version of this interface (CODA_ABI_VERSION of the built library). */
int coda_abi_version(void);

/* Static name of a status code. */
const char* coda_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none).  Valid until the next call. */
const char* coda_last_error(void);

/* Workspace bytes an entry point needs for these dimensions (0 for invalid arguments).
 *   fp8:     0 for the bf16 entry points, 1 for the *_fp8 ones, 2 for coda_block_fwd_fp8_mx
 *   unfused: 0 for coda_block_fwd*, 1 for coda_block_unfused* (fp8 = 2 has no unfused form)
 * Layout (each piece 256-byte aligned): part [D/256][M] fp32 partial sums of squares, r [M] fp32, then
 *   fused:   bf16: hg = h * gamma, M * D bf16; fp8: the e4m3 quantisation of h * gamma, M * D bytes, its row
 *            scales s_a [M] and s_a * r [M]; fp8 = 2: the block-scaled e4m3 codes, M * D bytes, and their
 *            power-of-two scales, one byte per 32 values ((D/64) * ceil(M/256) * 512 bytes).  The fused paths
 *            keep hg and the codes in K panels of the second product's stage width: element (m, k) at
 *            ((k / P) * M + m) * P + k % P with P = 32 (bf16) or 64 (e4m3), so that the second product reads
 *            whole cache lines
 *   unfused: T [M,D] bf16 and n [M,D] bf16 (fp8: n as e4m3 [M,D] and its row scales [M]), row-major.
 * then the room to split a product's last wave of tiles along K, planned for 256 CUs: the second product
 * (ceil(M/256) * N2/256 tiles over K = D), then the first (ceil(M/256) * D/256 tiles over K1).  bf16 blocks: a
 * last wave splits where it fills at most a quarter of the CUs (three eighths where K >= 4096) and K >= 1024, into
 * S = 2 pieces per tile, or 4 or 8 while all the pieces fill at most half of the CUs and each keeps 1024 of K.
 * e4m3 blocks: at most an eighth of the CUs (three eighths where K >= 8192), K >= 4096, more pieces while each
 * keeps 2048 of K.  Per tile of the last wave: S - 1 int32 tickets (all of them 256-byte aligned), then 2 S - 2
 * fp32 slots of 256 KiB.  A block given a workspace of at least the size without that room
 * runs; it splits the last waves only where the room is there (the results of the two forms differ in the last
 * bits of the fp32 sums, nowhere else). */
size_t coda_workspace_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int epi_kind, int fp8, int unfused);

/* The part of coda_workspace_bytes (same arguments) that is the split room of the products' last waves: 0 where
 * there is none; coda_workspace_bytes minus this is the smallest workspace a block accepts. */
size_t coda_workspace_split_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int epi_kind, int fp8, int unfused);

/* The fused block, bf16 operands: the GEMM -> residual -> RMSNorm -> GEMM block of the write-up's section
 * "CODA: the treasure hidden in the epilogue" (the residual added and the partial sums of squares taken in the
 * first product's epilogue, the per-row RMS factor moved past the second product into its epilogue, SwiGLU
 * admitting the same rewrite), with the section "Five blocks and a Lego language"'s primitives: tiled store
 * of h, the RMSNorm weight as a broadcast vector, the block reduction for the local sums of squares.
 *   X [M,K1] bf16, W1 [K1,D] bf16, R [M,D] bf16, gamma [D] fp32, W2 [D,N2] bf16  (inputs)
 *   out_h [M,D] bf16 = bf16(X W1 + R) (the fp32 sum rounded once)                   (output)
 *   out_y [M,N2 or N2/2] bf16 = bf16(epi(r * (hg W2))), hg = bf16(h * gamma)          (output)
 * Two kernels on `stream` where D <= 4096: GEMM1 + residual + gamma + partial sums of squares, then GEMM2 on
 * hg whose workgroups reduce their rows' partial sums to r themselves and apply r (+ SwiGLU) in the epilogue.
 * Where D > 4096 the reduction runs as a kernel of its own between the two (three kernels).  Where a product's
 * last wave of 256 x 256 tiles would leave most of the CUs idle, each of its tiles is computed as 2, 4 or 8 equal
 * ranges of K whose fp32 sums meet in a fixed binary tree before the epilogue (coda_workspace_bytes gives the rule
 * and the room this takes); where the first product is split, a small kernel that zeroes its tickets runs first.
 * Where the second product's last wave fills at most half of the CUs and is not split along K, and M > 64 rows
 * with a last row tile that is whole or longer than 128 rows, that wave's tiles run as two 128-row halves each, in
 * a launch of their own after the whole tiles (no workspace; the results are the whole tiles' bit for bit).
 * After the call the workspace holds r [M] (fp32) at byte offset coda_workspace_r_offset(M, D).  Ownership, errors
 * and the asynchronous contract are the shared conventions above. */
int coda_block_fwd(const void* X, const void* W1, const void* R, const float* gamma, const void* W2,
                   float eps, int epi_kind, void* out_h, void* out_y,
                   int64_t M, int64_t K1, int64_t D, int64_t N2,
                   void* workspace, size_t workspace_bytes, void* stream);

/* Size of the library's fixed scratch used by coda_block_fwd_noalloc (64 MiB per device). */
#define CODA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* coda_block_fwd for callers that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Same arguments, outputs, shape rules, errors and kernels as
 * coda_block_fwd, without the workspace: the block's workspace (partial sums, r, h * gamma) lives in a fixed
 * array of CODA_NOALLOC_SCRATCH_BYTES in the library's device code, which each device the library runs on
 * holds from the moment the library is loaded there until the process ends.  Nothing is allocated by this
 * call (no hipMalloc, hipFree or allocating library routine); the first call on a device looks the array's
 * address up once (hipGetSymbolAddress).  Limit: the workspace without the split room (coda_workspace_bytes)
 * must not exceed CODA_NOALLOC_SCRATCH_BYTES (M * D up to about 33 million: the 1B shapes fit, M = 16384 with
 * D = 4096 does not), else CODA_ERR_WORKSPACE before anything is enqueued; the last waves are split as in
 * coda_block_fwd where the scratch also holds the split room, so the outputs equal coda_block_fwd's bit for bit
 * wherever coda_workspace_bytes(M, K1, D, N2, epi_kind, 0, 0) fits the scratch.  Every call on one device shares that
 * device's array and leaves its contents there (nothing in it needs clearing between calls: every byte the
 * kernels read was written earlier in the same call), so calls that overlap on one device race: order them on
 * one stream or otherwise.  r is not returned (it stays in the scratch); callers that need it use
 * coda_block_fwd. */
int coda_block_fwd_noalloc(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                           int epi_kind, void* out_h, void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2,
                           void* stream);

/* The fused block with fp8 (OCP e4m3fn) operands and fp32 accumulation: the same block (section "CODA: the
 * treasure hidden in the epilogue"); the write-up's section "Where training time goes" reports that the
 * non-GEMM share of training time grows once FP8 is introduced, and its section "Five blocks and a Lego
 * language" lists per-row / per-column scale vectors among the epilogue's broadcast loads.
 *   Xq [M,K1] e4m3 with per-row scales sx [M]; W1q [K1,D] e4m3 with per-column scales sw1 [D];
 *   W2q [D,N2] e4m3 with per-column scales sw2 [N2]; R [M,D] bf16; gamma [D] fp32.
 *   out_h = bf16(dequant(Xq) dequant(W1q) + R); out_y as coda_block_fwd.
 * The second product's A operand is a = h * gamma (fp32, h the stored bf16 out_h) quantised per row to
 * e4m3(a * (1 / s_a)) with s_a = amax_j |a_ij| / 448 (1 for an all-zero row; 1 / s_a rounded to fp32 once)
 * by the reduction kernel, which has the whole row; y = bf16(epi(acc * s_a_i * r_i * sw2_n)).  Shape rules as coda_block_fwd, and K1 a multiple
 * of 256.  Workspace: coda_workspace_bytes(..., fp8 = 1, unfused = 0); the products' last waves are split as in
 * coda_block_fwd, by the e4m3 rule given there. */
int coda_block_fwd_fp8(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                       const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                       void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                       size_t workspace_bytes, void* stream);

/* The unfused three-kernel baseline, kept to measure the HBM traffic the fusion saves: the conventional form
 * the write-up's section "CODA: the treasure hidden in the epilogue" contrasts with the fused one (three
 * operators, the intermediate written to and read back from memory twice):
 *   T = bf16(X W1)  ->  hf = fp32(T) + fp32(R), h = bf16(hf), r = 1 / sqrt(mean(hf^2) + eps),
 *   n = bf16(hf * r * gamma)  ->  y = bf16(epi(n W2)).
 * T and n live in the workspace (row-major).  Same arguments, outputs, errors and conventions as
 * coda_block_fwd, including the splits of the products' last waves; after the call the workspace holds r
 * at coda_workspace_r_offset(M, D). */
int coda_block_unfused(const void* X, const void* W1, const void* R, const float* gamma, const void* W2,
                       float eps, int epi_kind, void* out_h, void* out_y,
                       int64_t M, int64_t K1, int64_t D, int64_t N2,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The unfused baseline with e4m3 operands: T = bf16(dequant(Xq) dequant(W1q)) -> h = bf16(T + R),
 * n = (T + R) r gamma quantised per row to e4m3 (scale amax|n row| / 448) -> y = epi(dequant(nq) dequant(W2q)).
 * Same arguments as coda_block_fwd_fp8; workspace: coda_workspace_bytes(..., fp8 = 1, unfused = 1). */
int coda_block_unfused_fp8(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                           const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                           void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                           size_t workspace_bytes, void* stream);

/* The fused e4m3 block with a block-scaled (MX-style) A operand for the second GEMM, a variant that needs no
 * cross-tile amax: the first GEMM's epilogue quantises a = bf16(h) * gamma (fp32) itself, in blocks of 32
 * consecutive columns of a row, each with a power-of-two scale 2^e, e the smallest integer with
 * amax_block <= 448 * 2^e (e = 0 for an all-zero block; e limited to [-127, 127]), codes e4m3(a / 2^e) rounded to
 * nearest even; the second GEMM feeds the scales to the scaled MFMA and applies r (the partial-RMS reduce folded
 * in where D <= 4096) and sw2 in its epilogue:
 *   y = bf16(epi(r[i] * sw2[n] * sum_k dec(q[i][k]) 2^e(i, k/32) dec(W2q[k][n]))).
 * Two kernels (three where D > 4096).  The pages fix no quantisation granularity (they list per-row activation
 * scales among the epilogue's vector loads, section "Five blocks and a Lego language"); this is a variant of
 * coda_block_fwd_fp8 with the same arguments, outputs, shape rules and errors; workspace:
 * coda_workspace_bytes(..., fp8 = 2, unfused = 0), which also holds r at coda_workspace_r_offset. */
int coda_block_fwd_fp8_mx(const void* Xq, const float* sx, const void* W1q, const float* sw1, const void* R,
                          const float* gamma, const void* W2q, const float* sw2, float eps, int epi_kind, void* out_h,
                          void* out_y, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                          size_t workspace_bytes, void* stream);

/* The fused block with a rotary position embedding after the row scale (identity epilogue), for a block that
 * feeds attention (QKV projection).  The write-up lists RoPE among the epilogue-fusable operations (section
 * "CODA: the treasure hidden in the epilogue"; section "Five blocks and a Lego language": elementwise
 * transforms).  Convention (the pages fix none; this is the LLaMA-family "rotate half" form): the first
 * n_rope_cols columns of y form heads of 64 columns; in each, the pair (i, i + 32) is rotated by
 * theta = pos * rope_base^(-2 i / 64) with pos = row mod seq_len:
 *   (a, b) -> (a cos theta - b sin theta, b cos theta + a sin theta),  a, b = r * (h W2') in fp32;
 * y = bf16 of the result; columns >= n_rope_cols are y = bf16(r * (h W2')).  Arguments, outputs, shape rules
 * and workspace as coda_block_fwd with CODA_EPI_IDENTITY; n_rope_cols a multiple of 64 in [0, N2],
 * seq_len >= 1, rope_base finite and > 0 (else CODA_ERR_INVALID_ARG). */
int coda_block_fwd_rope(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                        int64_t seq_len, int64_t n_rope_cols, float rope_base, void* out_h, void* out_y, int64_t M,
                        int64_t K1, int64_t D, int64_t N2, void* workspace, size_t workspace_bytes, void* stream);

/* The same rotation as a separate pass, in place on bf16 y [M,N] (the unfused counterpart of
 * coda_block_fwd_rope, used to measure what the epilogue saves).  Same convention and argument rules. */
int coda_rope_rows(void* y, int64_t M, int64_t N, int64_t seq_len, int64_t n_rope_cols, float rope_base, void* stream);

/* Byte offset of r [M] (fp32) inside the workspace of every block entry point. */
size_t coda_workspace_r_offset(int64_t M, int64_t D);

/* ---- the three steps of coda_block_fwd, exposed one by one (same conventions) ---- */

/* Step 1: out_h = bf16(X W1 + R); out_hg = bf16((X W1 + R) * gamma) (the fp32 sum times gamma, rounded
 * once); part[t][i] = sum over the 256 columns of tile t of the fp32 (X W1 + R)_ij^2.
 * X [M,K1] bf16, W1 [K1,D] bf16, R [M,D] bf16, gamma [D] fp32 (inputs); out_h, out_hg [M,D] bf16 and
 * part [D/256][M] fp32 (outputs; out_h == R is allowed). */
int coda_gemm1_residual_partial_rms(const void* X, const void* W1, const void* R, const float* gamma, void* out_h,
                                    void* out_hg, float* part, int64_t M, int64_t K1, int64_t D, void* stream);

/* Step 2: r[i] = 1 / sqrt((sum_{t=0..T-1} part[t][i]) / D + eps), summed in t order.  part [T][M] fp32,
 * r [M] fp32 (device). */
int coda_partial_rms_reduce(const float* part, int64_t T, int64_t M, int64_t D, float eps, float* r,
                            void* stream);

/* Step 3: out_y = bf16(epi(r_i * (hg W2))).  hg [M,D] bf16 (h * gamma from step 1), W2 [D,N2] bf16,
 * r [M] fp32 (device). */
int coda_gemm2_rowscale(const void* hg, const void* W2, const float* r, int epi_kind, void* out_y, int64_t M,
                        int64_t D, int64_t N2, void* stream);

/* Steps 1 and 3 in the layout coda_block_fwd uses between them (the same arithmetic, bit for bit).
 * hg in K panels of 32 columns: element (m, k) of the logical [M,D] hg at ((k / 32) * M + m) * 32 + k % 32,
 * so that the second product's direct loads cover whole 128-byte lines.
 * _panels step 1: as coda_gemm1_residual_partial_rms with out_hg written in that layout (M * D bf16).
 * _panels step 3: as coda_gemm2_rowscale on hg in that layout.  With part non-NULL (part [D/256][M] fp32 from
 * step 1, D <= 4096, eps finite >= 0) step 2 is folded in: each workgroup sums its rows' partial sums in t order
 * and forms r as coda_partial_rms_reduce does (the same r bit for bit), and the workgroups of the first column
 * tile also write r [M] (output); with part NULL, r [M] is an input and eps is ignored.  Errors as
 * coda_gemm2_rowscale, plus CODA_ERR_UNSUPPORTED for part with D > 4096 and CODA_ERR_ALIAS for r overlapping
 * an input or out_y when it is an output. */
int coda_gemm1_residual_partial_rms_panels(const void* X, const void* W1, const void* R, const float* gamma,
                                           void* out_h, void* out_hg, float* part, int64_t M, int64_t K1, int64_t D,
                                           void* stream);
int coda_gemm2_rowscale_panels(const void* hg, const void* W2, const float* part, float eps, float* r, int epi_kind,
                               void* out_y, int64_t M, int64_t D, int64_t N2, void* stream);

/* ---- backward of the block ----
 * The CODA write-up (section "CODA: the treasure hidden in the epilogue"; section "Experimental results"
 * reports the backward kernels) applies the same epilogue rewrite to back-propagation.  With the forward
 * h = X W1 + R, r_i = 1/sqrt(mean_j h_ij^2 + eps), n = r h, u = n * gamma, z = u W2, and given dz (the
 * gradient of z, the second product's output before any epilogue) and dh_out (the gradient arriving at the
 * residual stream h from downstream; NULL for none):
 *   dR = dh = r (du gamma - n mean_j(du_ij gamma_j n_ij)) + dh_out,   du = dz W2^T
 *   dX = dh W1^T,  dW1 = X^T dh,  dgamma_j = sum_i du_ij n_ij,  dW2 = u^T dz
 * Inputs: X [M,K1] bf16, W1 [K1,D] bf16, h [M,D] bf16 and r [M] fp32 as the forward left them (out_h and
 * the workspace's r), gamma [D] fp32, W2 [D,N2] bf16, dz [M,N2] bf16, dh_out [M,D] bf16 or NULL.
 * Outputs: out_dX [M,K1] bf16, out_dW1 [K1,D] fp32, out_dR [M,D] bf16, out_dgamma [D] fp32, out_dW2 [D,N2]
 * fp32.  Kernels on `stream` (the fused path): W2's transpose (see coda_block_bwd_w2t), P = dz W2^T with the
 * RMSNorm-backward row and column statistics in its epilogue, a light reduction, dh (and its transpose and
 * n's), then the dX, dW1 and dW2 products (the weight gradients split along M into fp32 slabs, summed by a
 * small kernel, where their output has few tiles).  Shape rules: M a multiple of 128, K1 a multiple of 256, D and N2 multiples of 256.  No output
 * may overlap an input or another output.  Workspace: coda_bwd_workspace_bytes(..., unfused = 0); other
 * conventions as the forward entry points. */
size_t coda_bwd_workspace_bytes(int64_t M, int64_t K1, int64_t D, int64_t N2, int unfused);

int coda_block_bwd(const void* X, const void* W1, const void* h, const float* r, const float* gamma, const void* W2,
                   const void* dz, const void* dh_out, void* out_dX, float* out_dW1, void* out_dR, float* out_dgamma,
                   float* out_dW2, int64_t M, int64_t K1, int64_t D, int64_t N2, void* workspace,
                   size_t workspace_bytes, void* stream);

/* coda_block_bwd with W2 given transposed: W2t is W2^T [N2,D] bf16 row-major (the [out,in] layout in which
 * many frameworks keep their weights) in W2's place; the other arguments, the checks (W2t has W2's size), the
 * workspace and the results are coda_block_bwd's, bit for bit.  The transpose pass over W2 that
 * coda_block_bwd makes first (a read and a write of D * N2 * 2 bytes) is skipped. */
int coda_block_bwd_w2t(const void* X, const void* W1, const void* h, const float* r, const float* gamma,
                       const void* W2t, const void* dz, const void* dh_out, void* out_dX, float* out_dW1, void* out_dR,
                       float* out_dgamma, float* out_dW2, int64_t M, int64_t K1, int64_t D, int64_t N2,
                       void* workspace, size_t workspace_bytes, void* stream);

/* The unfused backward baseline: P = dz W2^T is stored (bf16) and its RMSNorm-backward statistics are
 * computed by a separate pass over P and h; the remaining kernels are shared.  Same arguments and outputs;
 * workspace: coda_bwd_workspace_bytes(..., unfused = 1). */
int coda_block_bwd_unfused(const void* X, const void* W1, const void* h, const float* r, const float* gamma,
                           const void* W2, const void* dz, const void* dh_out, void* out_dX, float* out_dW1,
                           void* out_dR, float* out_dgamma, float* out_dW2, int64_t M, int64_t K1, int64_t D,
                           int64_t N2, void* workspace, size_t workspace_bytes, void* stream);

/* Cross-entropy of a vocabulary projection without storing the logits.  The write-up names cross-entropy among
 * the operations its epilogue programming covers (section "CODA: the treasure hidden in the epilogue") and
 * builds reductions from per-tile partial results merged by a light kernel (section "Five blocks and a Lego
 * language").  Computes, per row i of H [M,D] (bf16) against W [D,V] (bf16, [in,out] like the other weights):
 *   z = H W (fp32 accumulation), out_lse[i] = log sum_j exp(z_ij), out_loss[i] = out_lse[i] - z[i][labels[i]];
 * labels [M] int32 on the device; a negative label marks an ignored row (loss 0, lse still written), a label
 * >= V gives a NaN loss.  Outputs fp32 [M].  Three kernels on `stream`: a copy of H into K panels of 32 columns
 * (the product's operand layout, see coda_workspace_bytes), the product whose epilogue reduces each 256-column
 * tile of a row to (max, sum of exp(z - max)) and picks the label's logit, then the merge of those pairs in
 * tile order.  Shape rules: D a multiple of 128, V a multiple of 256 (else CODA_ERR_UNSUPPORTED), M >= 1.  No
 * output may overlap an input, another output or the workspace.  Workspace: coda_ce_workspace_bytes(M, D, V, 0)
 * bytes, 256-byte aligned (the panel copy of H, M * D bf16, then the pairs and label logits); other conventions
 * as coda_block_fwd. */
size_t coda_ce_workspace_bytes(int64_t M, int64_t D, int64_t V, int unfused);

int coda_ce_fwd(const void* H, const void* W, const int32_t* labels, float* out_loss, float* out_lse, int64_t M,
                int64_t D, int64_t V, void* workspace, size_t workspace_bytes, void* stream);

/* The unfused baseline: the logits are stored in bf16 (workspace: coda_ce_workspace_bytes(M, D, V, 1) = the panel
 * copy of H and the M x V bf16 logits) and a second kernel reads each row back.  Same arguments and outputs; the
 * loss and lse come from the bf16-rounded logits. */
int coda_ce_unfused(const void* H, const void* W, const int32_t* labels, float* out_loss, float* out_lse, int64_t M,
                    int64_t D, int64_t V, void* workspace, size_t workspace_bytes, void* stream);

/* The fused block with the SwiGLU epilogue (as coda_block_fwd with CODA_EPI_SWIGLU) that also stores the
 * pre-activation out_z = [gate | up] = r * (h W2') as bf16 [M, N2], written from GEMM2's epilogue, for the
 * backward of the SwiGLU (coda_swiglu_bwd).  Arguments, shape rules, workspace and errors as coda_block_fwd;
 * out_z may not overlap any other buffer. */
int coda_block_fwd_save_z(const void* X, const void* W1, const void* R, const float* gamma, const void* W2, float eps,
                          void* out_h, void* out_y, void* out_z, int64_t M, int64_t K1, int64_t D, int64_t N2,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Backward of the SwiGLU epilogue y = silu(g) * u, z = [g | u] (F = N2/2 columns each), fused into the epilogue
 * of the product that brings the gradient back to y.  The write-up reports the SwiGLU backward among its
 * largest gains (section "Experimental results"; section "CODA: the treasure hidden in the epilogue" for the
 * backward's structure).  Inputs: dout [M,D] bf16, the gradient of out = y Wd; Wd [F,D] bf16, that product's
 * weight stored [in = F, out = D]; z [M, 2F] bf16 from coda_block_fwd_save_z.  Output: out_dz [M, 2F] bf16,
 *   dy = dout Wd^T (fp32 accumulation, never stored),
 *   out_dz[:, f] = bf16(dy u silu'(g)), out_dz[:, F + f] = bf16(dy silu(g)),  silu'(g) = s (1 + g (1 - s)),
 * s = 1 / (1 + exp(-g)); out_dz is the dz that coda_block_bwd takes.  One kernel on `stream`; no workspace
 * (coda_swiglu_bwd_workspace_bytes(M, F, 0) = 0; workspace may be NULL).  Shape rules: D a multiple of 128,
 * F a multiple of 256 (else CODA_ERR_UNSUPPORTED), M >= 1.  out_dz may not overlap an input. */
size_t coda_swiglu_bwd_workspace_bytes(int64_t M, int64_t F, int unfused);

int coda_swiglu_bwd(const void* dout, const void* Wd, const void* z, void* out_dz, int64_t M, int64_t D, int64_t F,
                    void* workspace, size_t workspace_bytes, void* stream);

/* The unfused baseline: dy is stored (bf16 [M,F] in the workspace, coda_swiglu_bwd_workspace_bytes(M, F, 1)
 * bytes) and a second kernel reads it back with z.  Same arguments and outputs (dy rounded to bf16 first). */
int coda_swiglu_bwd_unfused(const void* dout, const void* Wd, const void* z, void* out_dz, int64_t M, int64_t D,
                            int64_t F, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif
#endif
