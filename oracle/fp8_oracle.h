/*
 * fp8_oracle.h -- TEST INFRASTRUCTURE ONLY.
 *
 * A plain, slow, obviously-correct CPU implementation of the FP8 runtime
 * chain (amax -> scale -> saturating round-to-nearest-even cast -> scaled
 * GEMM).  It exists to check the HIP library; it is never part of the
 * product path.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg may load it.  It shares no source, header, table or
 * helper with the HIP library under dynamic_scaling_scaled_amd/.
 *
 * Sources followed (page title, then section):
 *  - "FP8 formats and scaling for LLM inference" (charlestar.github.io):
 *      sections "How the 8 bits are allocated" (formats, max finite values),
 *      "How a scale fits a tensor into E4M3" (quantize / dequantize / amax /
 *      s = amax/F_max), "Per-channel and block scaling" (s_g = a_g/F_max),
 *      "Delayed scaling" (s_{t+1} = f(a_t..a_{t-h+1})/F_max),
 *      "The full precision contract of one FP8 GEMM" (Y ~ s_x s_w X8 W8),
 *      "What numerical validation looks at" (saturation / underflow rates),
 *      "Weight-only FP8 and W8A8 FP8" (FP8 weights with BF16 activations).
 *  - "Quantization W8A16" (datawhalechina llm-algo-leetcode): the granularity
 *      comparison (scale count and bytes against reconstruction error).
 *  - "FP8 production quantization guide" (m.xxqk.cn): the dynamic per-tensor
 *      quantize listing (amax clamp, scale, inverse scale, clamp, cast).
 *  - "FP8 inference: E4M3/E5M2 and the NVIDIA FP8 ecosystem" (plumephp.com):
 *      section "numeric properties" (bias 7 / 15) and the dequantization
 *      example.
 *
 * Floating point: values that the method defines in binary32 are computed
 * in binary64 from exact binary32 operands and rounded once to binary32
 * (innocuous double rounding for + - * / since 53 >= 2*24+2); GEMM sums are
 * accumulated in binary64 and cross-checked against exact __int128 sums.
 *
 * Parity pins: every function here is pinned by tests/test_oracle_*.py
 * (closed forms, the pages' worked examples, brute force, a library cast).
 * Parity unpinned: the cold start of delayed scaling (step 0 uses the
 * current amax) and the default eps are readings the pages do not fix; the
 * HIP library follows the same readings.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_E4M3 = 0, ORC_E5M2 = 1 };
enum { ORC_F32 = 0, ORC_BF16 = 1 };
enum { ORC_DYNAMIC = 0, ORC_GIVEN = 1 };

/* Format constants: max finite magnitude, mantissa bits, exponent bias. */
double orc_fmax(int fmt);

/* Exact value of an 8-bit code (NaN / +-Inf where the format has them). */
double orc_decode(unsigned code, int fmt);

/* Saturating round-to-nearest-even encode of an already-scaled binary32 v. */
unsigned orc_encode(float v, int fmt);

/* Brute force: nearest finite code over all 256 decoded codes, ties to the
 * code with an even mantissa.  Used only to pin orc_encode. */
unsigned orc_encode_bruteforce(float v, int fmt);

/* Exact widening of element i of a binary32 / bfloat16 array to binary32. */
float orc_load(const void* x, int dtype, int64_t i);

/* Group extents: gr, gc <= 0 mean "whole dimension". */
int64_t orc_ngroups(int64_t n, int64_t g);

/* amax per group, row-major [ceil(rows/gr)][ceil(cols/gc)]. */
int orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
             int64_t gr, int64_t gc, float* amax);

/* s = fl32(max(a,eps)/F_max), r = fl32(F_max/max(a,eps)); pow2 rounds s up
 * to a power of two and sets r = 1/s.  Non-finite a gives NaN s and r. */
int orc_compute_scale(const float* amax, int64_t n, int fmt, float eps, int pow2,
                      float* s, float* r);

/* Quantize.  DYNAMIC: amax -> (s, r) per group, written to s / r.
 * GIVEN: s is read; r is read, or fl32(1/s) when r == NULL.
 * amax_out (nullable) receives the observed per-group amax.
 * counts (nullable) receives {saturated, underflowed}. */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                 int64_t gr, int64_t gc, int fmt, int mode, float eps, int pow2,
                 float* s, float* r, uint8_t* q, int64_t ldq,
                 float* amax_out, uint64_t* counts);

/* Cast-transpose: orc_quantize, plus qt[j * ldqt + i] = q[i * ldq + j]
 * (the codes also written K-major).  Requires ldqt >= rows. */
int orc_quantize_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t gr, int64_t gc, int fmt, int mode, float eps, int pow2,
                           float* s, float* r, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                           float* amax_out, uint64_t* counts);

/* y = fl32(s * dec(code)); out_dtype ORC_BF16 rounds that binary32 to bf16. */
int orc_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                   int64_t gr, int64_t gc, const float* s, void* y, int out_dtype,
                   int64_t ldy);

/* Delayed scaling: push a_t into a zero-initialised ring of length len,
 * advance head, derive (s, r) for the next step from the window maximum. */
int orc_history_update(float* hist, int len, int* head, float amax_new, int fmt,
                       float eps, int pow2, float* s_next, float* r_next);

/* Delayed-scaling recipe variants: the history function fn (ORC_HIST_MAX =
 * window maximum, ORC_HIST_LATEST = a_t alone) and a margin m in [0, 16]:
 * the scale is derived from f * 2^m.  The ring and head advance as in
 * orc_history_update. */
enum { ORC_HIST_MAX = 0, ORC_HIST_LATEST = 1 };
int orc_history_update_recipe(float* hist, int len, int* head, float amax_new, int fmt, int fn,
                              int margin, float eps, int pow2, float* s_next, float* r_next);

/* Scaled GEMM reference at selected output points (m[i], n[i]):
 *   y[i] = sum_k s_a(m,k) s_b(n,k) dec(A[m,k]) dec(B[n,k]) + bias[n]
 *   S[i] = sum_k |s_a(m,k) s_b(n,k) dec(A[m,k]) dec(B[n,k])|
 * A is [M x K] row-major (lda), B is [N x K] row-major (ldb).
 * Scale arrays are row-major [ceil(M/gra)][ceil(K/gca)] and
 * [ceil(N/grb)][ceil(K/gcb)].  bias may be NULL.  Accumulation in binary64. */
int orc_gemm_points(const uint8_t* a, int fa, int64_t lda, int64_t gra, int64_t gca,
                    const float* sa, const uint8_t* b, int fb, int64_t ldb,
                    int64_t grb, int64_t gcb, const float* sb, int64_t M, int64_t N,
                    int64_t K, const void* bias, int bias_dtype, const int64_t* m,
                    const int64_t* n, int64_t npts, double* y, double* S);

/* Weight-only FP8 GEMM reference at points (m[i], n[i]):
 *   y[i] = sum_k x[m,k] s_w(n,k) dec(W[n,k]) + bias[n],  S[i] = sum_k |term|
 * x: [M x K] bf16 / fp32 activations (ldx, elements); W: [N x K] codes (ldw);
 * s_w: [ceil(N/grw)][ceil(K/gcw)].  Accumulation in binary64. */
int orc_wonly_gemm_points(const void* x, int xdtype, int64_t ldx, const uint8_t* w, int fw,
                          int64_t ldw, int64_t grw, int64_t gcw, const float* sw, int64_t M,
                          int64_t N, int64_t K, const void* bias, int bias_dtype,
                          const int64_t* m, const int64_t* n, int64_t npts, double* y,
                          double* S);

/* Reconstruction error of a quantized weight (granularity ledger):
 * w [N x K] fp32 / bf16 (ldw), codes q (ldq) with scales [ceil(N/gr)][ceil(K/gc)],
 * optional bf16 inputs x [M x K] (ldx).  w_hat = fl32(s dec(q)), e = w_hat - w.
 * stats[7] = {sum e^2, sum w^2, max |e|, sum d^2, sum y_ref^2, sum y_q^2,
 * sum y_ref y_q} with y_ref = x W^T, y_q = x W_hat^T, d = y_q - y_ref, all in
 * binary64 (3..6 zero without x). */
int orc_quant_error(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw, const uint8_t* q,
                    int fmt, int64_t ldq, int64_t gr, int64_t gc, const float* scale, const void* x,
                    int64_t M, int64_t ldx, double* stats);

/* Fragment-ordered weight layout (16-row groups x 128-byte K steps, 2 KB
 * each, lane-major halves); see fp8_oracle.c.  Zero codes past row N. */
int orc_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp);

/* Exact inner sums: for point i and every maximal K-run on which both scales
 * are constant, the sum of dec*dec products as an exact integer multiple of
 * the product quantum (2^-18 E4M3xE4M3, 2^-25 E5M2xE4M3, 2^-32 E5M2xE5M2),
 * combined with the run's scales in binary64.  Used to pin orc_gemm_points. */
int orc_gemm_points_exact(const uint8_t* a, int fa, int64_t lda, int64_t gra, int64_t gca,
                          const float* sa, const uint8_t* b, int fb, int64_t ldb,
                          int64_t grb, int64_t gcb, const float* sb, int64_t M,
                          int64_t N, int64_t K, const void* bias, int bias_dtype,
                          const int64_t* m, const int64_t* n, int64_t npts, double* y);

/* Tolerance helper (fp8_dot_bound.c): bound on the truncation error of the
 * matrix-core FP8 dot product at points (m[i], n[i]); see that file. */
int orc_dot_truncation_bound(const uint8_t* a, int fa, int64_t lda, int64_t gra, int64_t gca,
                             const float* sa, const uint8_t* b, int fb, int64_t ldb,
                             int64_t grb, int64_t gcb, const float* sb, int64_t M, int64_t N,
                             int64_t K, const int64_t* m, const int64_t* n, int64_t npts,
                             double* bound);

/* Round a binary64 value to bfloat16 (nearest, ties to even); returns bits. */
uint16_t orc_round_bf16(double v);

/* Round a binary32 value to bfloat16 (nearest, ties to even); returns bits. */
uint16_t orc_round_bf16_from_f32(float v);

#ifdef __cplusplus
}
#endif
#endif
