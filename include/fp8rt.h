/*
 * fp8rt.h -- C ABI of the MI355X (gfx950) FP8 runtime chain:
 *   amax reduction -> scale s = amax / F_max -> saturating round-to-nearest-
 *   even cast to OCP E4M3 / E5M2 codes -> scaled GEMM with FP32 accumulation.
 *
 * Sources (page title, then section):
 *  [P2] "FP8 formats and scaling for LLM inference" (charlestar.github.io)
 *  [P4] "FP8 production quantization guide" (m.xxqk.cn)
 *  [P5] "FP8 inference: E4M3/E5M2 and the NVIDIA FP8 ecosystem" (plumephp.com)
 *  [P3] "Quantization W8A16" (datawhalechina llm-algo-leetcode ch.25)
 *
 * Conventions shared by every entry point
 *  - Every array pointer is a caller-owned DEVICE pointer (HBM of the current
 *    HIP device).  The library owns two kinds of device memory, both per
 *    (device, stream) pair, allocated (hipMalloc) on first use and kept, at
 *    the same address, until the process ends; nothing is zeroed and no call
 *    synchronizes the device or the stream:
 *      * a workspace of 256 KB for the per-block partial results of the
 *        quantize kernels and of the FP8-output GEMM;
 *      * a scratch buffer for the GEMM's repacked 1x32 exponents ((ceil(M/256)
 *        + ceil(N/256)) * K/128 * 1024 bytes) and transposed 1x128 A scales
 *        (ceil(M/256) * 256 * K/128 * 4 bytes), the FP32 parts of a last wave
 *        split along K (up to 4 parts x 256 KB per split 256 x 256 tile), the
 *        cast-transpose's per-group arrays and the ledger's partials.  When a
 *        call needs more, a larger buffer (at least twice the old) is
 *        allocated and the old one is KEPT, never freed: every address handed
 *        to a kernel stays valid for the process's life.
 *    Calls on one stream are ordered and share that stream's memory; calls on
 *    different streams never share it.  Work is enqueued on `stream` and the
 *    call returns without synchronizing; results are valid once the stream
 *    reaches that point.
 *  - HIP graph capture: a call that needs no new allocation only enqueues
 *    kernels and can be captured.  Warm each entry point up eagerly on the
 *    capture stream with the largest shapes the graph will use (a first call
 *    or a growth allocates with hipMalloc, which capture may reject: the call
 *    then returns FP8RT_EHIP and enqueues nothing).  A captured graph holds
 *    the capture stream's workspace and scratch addresses: replay it on that
 *    stream, or at least never while other calls on that stream run, since
 *    they would share the same memory.
 *  - Matrices are row-major with a leading dimension in ELEMENTS (ldx >= cols).
 *  - Arguments are validated on the host before anything is launched; on an
 *    error nothing is written and nothing is enqueued.
 *  - Non-finite data are not errors: a NaN in a group makes its amax, scale
 *    and inverse scale NaN and its codes 0x7F; +-Inf saturates to the largest
 *    finite code and is counted as saturated.
 *  - Scale arrays are fp32, row-major [ceil(rows/gr)][ceil(cols/gc)] where
 *    (gr, gc) is the granularity with 0 meaning "the whole dimension"; the last
 *    group along a dimension may be short and is kept [P3, Step 2 granularity
 *    table: per-group scale count out x ceil(in/group)].
 *  - s is the DEQUANTIZATION scale stored with the codes (x ~ s * dec(code),
 *    [P2 "How a scale fits a tensor into E4M3"]); r is the quantization
 *    multiplier.  Dynamic scales: a_c = max(amax, eps), s = fl32(a_c / F_max),
 *    r = fl32(F_max / a_c) [P2 same section; P4 dynamic quantize listing].
 */
#ifndef FP8RT_H
#define FP8RT_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations below are plain C enums (int-sized).  Compiled as C++
 * they get a fixed underlying type of int, so a value that is not one of the
 * enumerators (which the entry points reject with FP8RT_EINVAL) is still a
 * valid object of the type on both sides of the ABI. */
#ifdef __cplusplus
#define FP8RT_ENUM(name) enum name : int
#else
#define FP8RT_ENUM(name) enum name
#endif

typedef FP8RT_ENUM(fp8rt_status) {
    FP8RT_OK = 0,
    FP8RT_EINVAL = 1,       /* null required pointer, dims <= 0, ld < cols, bad eps /
                               history length / head, granularity not allowed for the op */
    FP8RT_EALIGN = 2,       /* cols, K, a leading dimension or a group width not a multiple
                               of 16, or a base pointer not 16-byte aligned ([P2 "Hardware
                               support ..." notes dims divisible by 16 for FP8 linears) */
    FP8RT_EUNSUPPORTED = 3, /* GEMM format pair / scale-granularity combination not built */
    FP8RT_EHIP = 4,         /* a HIP launch error */
    FP8RT_ESCRATCH = 5      /* fp8_scaled_gemm_noalloc: the shape needs more scratch than its
                               fixed buffer (FP8RT_NOALLOC_SCRATCH_BYTES) */
} fp8rt_status;

/* [P2 "How the 8 bits are allocated"]: E4M3 max finite 448, E5M2 max finite
 * 57344; [P5 "numeric properties"]: bias 7 and 15.  E4M3 is the OCP "fn"
 * variant (no Inf, NaN = 0x7F/0xFF); E5M2 has IEEE-style Inf/NaN. */
typedef FP8RT_ENUM(fp8rt_format) { FP8RT_E4M3 = 0, FP8RT_E5M2 = 1 } fp8rt_format;

typedef FP8RT_ENUM(fp8rt_dtype) { FP8RT_F32 = 0, FP8RT_BF16 = 1 } fp8rt_dtype;

/* Group extent of one scale [P2 "Per-channel and block scaling"]:
 *   per-tensor {0,0} | per-row / per-token / per-output-channel {1,0} |
 *   per-group along K {1,128} | per-block {128,128} | MX-style {1,32}. */
typedef struct fp8rt_gran {
    int32_t rows;
    int32_t cols;
} fp8rt_gran;

/* Where the scale comes from [P2 "Current scaling", "Delayed scaling",
 * "Weight scale and activation scale lifetimes"]. */
typedef FP8RT_ENUM(fp8rt_mode) {
    FP8RT_DYNAMIC = 0, /* current scaling: amax of this tensor -> s, r */
    FP8RT_GIVEN = 1    /* static or delayed: s (and optionally r) supplied */
} fp8rt_mode;

/* GEMM flags (fp8_scaled_gemm, fp8_scaled_gemm_fp8out, fp8_weight_only_gemm) */
#define FP8RT_POW2_SCALES 1u /* every scale is a power of two (enables 1x32 scaled MFMA) */
#define FP8RT_B_PACKED16 2u  /* the weight operand is fragment-ordered (fp8_pack_weights16) */
#define FP8RT_EXACT_PRODUCTS 4u /* products of codes formed exactly (decode shapes only) */

/* Per-group amax a_g = max |x| over each group [P2 "How a scale fits a tensor
 * into E4M3" (a_max = max|X|), "Per-channel and block scaling" (a_g)].
 *   x     : [rows x cols] fp32 or bf16, leading dimension ldx (elements)
 *   g     : granularity; amax receives ceil(rows/gr) * ceil(cols/gc) floats
 * Exact (integer max on |x| bit patterns); NaN propagates. */
fp8rt_status fp8_amax(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                      fp8rt_gran g, float* amax, hipStream_t stream);

/* Scales from amax [P2 "How a scale fits a tensor into E4M3": s = a/F_max and
 * the recipe option of power-of-two rounding; P4 dynamic quantize listing:
 * eps clamp, scale and inv_scale].
 *   amax[n] -> scale[n] = s, inv_scale[n] = r (inv_scale may be NULL).
 *   eps: finite, >= 2^-96 (keeps r finite).  pow2_round_up != 0: s is rounded
 *   up to 2^ceil(log2 s) and r = 1/s exactly. */
fp8rt_status fp8_compute_scale(const float* amax, int64_t n, fp8rt_format f, float eps,
                               int32_t pow2_round_up, float* scale, float* inv_scale,
                               hipStream_t stream);

/* Scale + saturating cast [P2 "How a scale fits a tensor into E4M3":
 * X_fp8 = cast(clip(X/s)); P4 listing: x * inv_scale, clamp to +-F_max, cast;
 * P2 "What numerical validation looks at": saturation and underflow rates].
 *   x        : [rows x cols] fp32 / bf16 (ldx); q: [rows x cols] uint8 codes (ldq)
 *   DYNAMIC  : per-group amax -> s, r written to scale / inv_scale (inv_scale
 *              may be NULL); codes use r.
 *   GIVEN    : scale is read (static calibration or delayed history); inv_scale
 *              is read if non-NULL, else r = fl32(1/s).  eps / pow2 ignored.
 *   amax_out : nullable; the observed per-group amax (for delayed scaling).
 *   sat_underflow : nullable uint64[2], OVERWRITTEN with {#|fl32(x*r)| > F_max,
 *              #(x != 0 and code is +-0)}.
 *   v = fl32(x * r); code = RNE onto the OCP grid (subnormals included) of
 *   clamp(v, -F_max, F_max); NaN -> 0x7F.
 * Alignment: cols, ldx, ldq and the group width (if not whole-row) are
 * multiples of 16, pointers 16-byte aligned.  Per-tensor DYNAMIC runs two
 * kernels (amax, then cast); all other granularities run one fused pass. */
fp8rt_status fp8_quantize(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                          int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                          float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                          uint8_t* q, int64_t ldq, float* amax_out, uint64_t* sat_underflow,
                          hipStream_t stream);

/* Cast-transpose [P2 "How the 8 bits are allocated": the hybrid recipe runs
 * the forward pass in E4M3 and the backward gradients in E5M2, and a backward
 * GEMM reads the operand in the other orientation; P5 QAT section: forward
 * and backward both through FP8].  Exactly fp8_quantize (same scales, codes,
 * amax_out and counters), with every code also written transposed:
 *   qt[j * ldqt + i] = q[i * ldq + j],  qt : [cols x rows] codes (ldqt >= rows).
 * Granularities: tensor {0,0}, row {1,0}, column {0,1} (one scale per column:
 * the row scale of the K-major copy); others return FP8RT_EUNSUPPORTED.
 * DYNAMIC runs an amax kernel (per-column: two), the scale kernel, then one
 * fused cast-transpose pass; GIVEN runs the pass alone (plus an amax pass
 * when amax_out is requested for row or column groups).
 * Alignment: rows, cols, ldx, ldq and ldqt multiples of 16; pointers 16-byte
 * aligned.  Scratch: the per-stream GEMM scratch buffer holds the amax and
 * r arrays when amax_out / inv_scale are NULL, and the per-column partials. */
fp8rt_status fp8_quantize_transpose(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                                    int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                                    float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                                    uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                    float* amax_out, uint64_t* sat_underflow, hipStream_t stream);

/* Dequantize [P2 "How a scale fits a tensor into E4M3": X_hat = s * X_fp8;
 * P5 dequantization example].  y = fl32(s_g * dec(code)); a bf16 output is
 * that binary32 rounded to nearest even.  q: [rows x cols] (ldq), y (ldy). */
fp8rt_status fp8_dequantize(const uint8_t* q, fp8rt_format f, int64_t rows, int64_t cols,
                            int64_t ldq, fp8rt_gran g, const float* scale, void* y,
                            fp8rt_dtype yt, int64_t ldy, hipStream_t stream);

/* Delayed scaling step [P2 "Delayed scaling": s_{t+1} = f(a_t..a_{t-h+1})/F_max,
 * f = window maximum].  One wave on the device:
 *   history[*head] = *amax_new; *head = (*head + 1) % len;
 *   a = max(history[0..len)); scale_next = s(a), inv_scale_next = r(a).
 *   history: fp32[len] caller-owned ring, zero-initialised by the caller;
 *   head: int32 device scalar in [0, len) (checked on the device: an out-of-
 *   range head is reduced modulo len); len in [1, 1024].
 * Cold start (no history yet): call fp8_amax on the first tensor, then this
 * function, and quantize step 0 with the result (current scaling). */
fp8rt_status fp8_amax_history_update(float* history, int32_t len, int32_t* head,
                                     const float* amax_new, fp8rt_format f, float eps,
                                     int32_t pow2_round_up, float* scale_next,
                                     float* inv_scale_next, hipStream_t stream);

/* History function of a delayed-scaling recipe. */
typedef FP8RT_ENUM(fp8rt_history_fn) {
  FP8RT_HIST_MAX = 0,    /* window maximum over the history ring */
  FP8RT_HIST_LATEST = 1  /* the newest amax alone */
} fp8rt_history_fn;

/* Delayed-scaling recipe variants ["FP8 formats and scaling for LLM
 * inference", section "Delayed scaling": the history function may be the
 * most recent value or the window maximum; section "How a scale fits a
 * tensor into E4M3": real recipes add a margin].  As
 * fp8_amax_history_update (same ring, head, eps and pow2 semantics), with
 *   f = window maximum (FP8RT_HIST_MAX) or a_t alone (FP8RT_HIST_LATEST;
 *       a non-positive a_t counts as 0, NaN propagates), and
 *   the scale derived from f * 2^margin, margin in [0, 16]: s_next grows by
 *       exactly 2^margin (an overflow to Inf gives NaN s and r).
 * FP8RT_HIST_MAX with margin 0 is fp8_amax_history_update.  Bad fn or
 * margin: FP8RT_EINVAL. */
fp8rt_status fp8_delayed_scale_update(float* history, int32_t len, int32_t* head,
                                      const float* amax_new, fp8rt_format f, fp8rt_history_fn fn,
                                      int32_t margin, float eps, int32_t pow2_round_up,
                                      float* scale_next, float* inv_scale_next, hipStream_t stream);

/* Scaled GEMM on FP8 MFMA [P2 "The full precision contract of one FP8 GEMM":
 * Y ~ s_x s_w (X8 W8), higher-precision accumulation, BF16/FP32 output, bias;
 * P4 GEMM listing: scale_a, scale_b, out_dtype, bias].
 *   Y[m,n] = sum_k s_a(m,k) s_b(n,k) dec(A[m,k]) dec(B[n,k]) + bias[n]
 *   a : [M x K] codes (lda), format fa, scales scale_a with granularity ga
 *   b : [N x K] codes (ldb) -- the nn.Linear weight layout, K contiguous
 *   bias : nullable, [N] fp32 / bf16;  y : [M x N] fp32 / bf16 (ldy)
 * Format pairs: E4M3 x E4M3 and E5M2 x E4M3.
 * Granularities: A in {tensor, row {1,0}, K-group {1,g}}, B in {tensor, row,
 * block {gr,g}} with g a multiple of 128 and equal for A and B when both are
 * K-blocked; or {1,32} on both with FP8RT_POW2_SCALES (hardware-scaled MFMA).
 * Accumulation is FP32 on the matrix cores; K-blocked scales are applied once
 * per 128-deep K step.  Alignment: K, lda, ldb multiples of 16; M, N any.
 * FP8RT_B_PACKED16: b is the fp8_pack_weights16 image of the [N x K] codes
 * (ldb ignored); decode shapes only (M <= 64, K a multiple of 128, no 1x32
 * power-of-two scales), else FP8RT_EUNSUPPORTED.  The result is
 * bit-identical to the row-major call.
 * Products: the FP8 matrix cores align the products of each 8-deep run of K
 * to the run's largest exponent and drop the bits below 2^-13 of it (toward
 * zero): a run loses less than 7 * 2^-13 of its largest |product|.  On
 * decode shapes (the packed-image
 * conditions above, row-major or packed) whose b holds at most
 * FP8RT_EXACT_AUTO_BYTES of codes -- launch-latency bound -- the library
 * instead widens the codes exactly to bf16 and multiplies them on the bf16
 * matrix cores, whose products are exact: only the FP32 accumulation rounds.
 * FP8RT_EXACT_PRODUCTS asks for that path on any decode shape (FP8RT_EUNSUPPORTED
 * on other shapes). */
#define FP8RT_EXACT_AUTO_BYTES (1u << 20)
fp8rt_status fp8_scaled_gemm(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                             const float* scale_a, const uint8_t* b, fp8rt_format fb,
                             int64_t ldb, fp8rt_gran gb, const float* scale_b, int64_t M,
                             int64_t N, int64_t K, const void* bias, fp8rt_dtype bias_t,
                             void* y, fp8rt_dtype yt, int64_t ldy, uint32_t flags,
                             hipStream_t stream);

/* fp8_scaled_gemm for callers that cannot allocate device memory: code
 * under HIP graph capture that has not warmed the library up on its stream,
 * tight serving loops, and harnesses that forbid hipMalloc.  Arguments,
 * results, validation and statuses are those of fp8_scaled_gemm, with one
 * difference in where the scratch comes from: this entry point never calls
 * hipMalloc / hipFree or any allocating routine.  Its scratch is a fixed
 * device array of the library, FP8RT_NOALLOC_SCRATCH_BYTES (16 MiB) on each
 * GPU, reserved when the library's code is loaded onto that GPU and kept
 * until the process ends; its address is looked up on the first call on each
 * device.
 *  - A call whose kernel needs more scratch than that (repacked 1x32
 *    exponents: (ceil(M/256) + ceil(N/256)) * K/128 * 1024 bytes; transposed
 *    1x128 A scales on large shapes: ceil(M/256) * 256 * K/128 * 4 bytes)
 *    returns FP8RT_ESCRATCH before anything is enqueued.
 *  - A ragged last wave of tiles, or a grid of tiles that fills at most half
 *    the CUs, is split along K into as many parts as fit beside the repacked
 *    exponents (256 KB per part and 256 x 256 tile), or not at all; the
 *    result can then differ from fp8_scaled_gemm's in FP32 summation order
 *    only, within the same tolerance.
 *  - Every call on a GPU shares that GPU's one array (whatever the stream),
 *    and the array keeps the last call's contents (nothing in it needs to
 *    start at zero): calls that overlap in time on one GPU race and give
 *    undefined results.  Order them on one stream, or synchronize. */
#define FP8RT_NOALLOC_SCRATCH_BYTES (16u << 20)
fp8rt_status fp8_scaled_gemm_noalloc(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                                     const float* scale_a, const uint8_t* b, fp8rt_format fb,
                                     int64_t ldb, fp8rt_gran gb, const float* scale_b, int64_t M,
                                     int64_t N, int64_t K, const void* bias, fp8rt_dtype bias_t,
                                     void* y, fp8rt_dtype yt, int64_t ldy, uint32_t flags,
                                     hipStream_t stream);

/* Scaled GEMM with an FP8 output [P2 "The full precision contract of one FP8
 * GEMM": the contract names the output scale / requantization when the next
 * op consumes FP8, applied in the epilogue instead of a BF16 write and a
 * separate cast].  y = the fp8_scaled_gemm result in binary32 (scales, FP32
 * accumulation, bias), then exactly the GIVEN-mode cast of fp8_quantize:
 *   yq[m, n] = RNE_fy(clamp(fl32(y * r_y), -F_max, F_max)),  NaN -> 0x7F,
 *   r_y = inv_scale_y[0], or fl32(1 / scale_y[0]) when inv_scale_y is NULL;
 *   amax_y (nullable, [1]): max |y| over the output (binary32, before the
 *   cast) -- the amax a delayed output scale pushes into its history;
 *   sat_underflow (nullable, [2]): |fl32(y r_y)| > F_max, and y != 0 cast to
 *   a zero code.
 * Operands, granularities and alignment as fp8_scaled_gemm; yq : [M x N]
 * codes (ldy).  Decode shapes (M <= 64, K a multiple of 128) run on the
 * decode kernel, row-major or on the weight image (FP8RT_B_PACKED16, not
 * with 1x32 scales; bit-identical results); the large-shape kernel
 * (per-tensor, per-row and 1x32 power-of-two scales) runs large shapes, a
 * ragged last wave of tiles split along K with the requantization in the
 * reduction kernel; other shapes run on the general kernel.  Limit:
 * ceil(M/128) ceil(N/128) <= 8192 (one per-block statistics partial per
 * output tile), and on the weight image ceil(N/16) times the decode
 * kernel's row-tile workgroups per column group <= 8192, else
 * FP8RT_EUNSUPPORTED.  FP8RT_EXACT_PRODUCTS is not accepted here
 * (FP8RT_EUNSUPPORTED): the FP8 matrix cores form the products. */
fp8rt_status fp8_scaled_gemm_fp8out(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                                    const float* scale_a, const uint8_t* b, fp8rt_format fb, int64_t ldb,
                                    fp8rt_gran gb, const float* scale_b, int64_t M, int64_t N, int64_t K,
                                    const void* bias, fp8rt_dtype bias_t, fp8rt_format fy,
                                    const float* scale_y, const float* inv_scale_y, uint8_t* yq,
                                    int64_t ldy, float* amax_y, uint64_t* sat_underflow, uint32_t flags,
                                    hipStream_t stream);

/* Weight-only FP8 GEMM ["FP8 formats and scaling for LLM inference", section
 * "Weight-only FP8 and W8A8 FP8": weights stored as FP8, activations kept in
 * BF16, the weight converted inside the kernel; section "Per-channel and
 * block scaling" for the weight's scale groups].
 *   Y[m,n] = sum_k x[m,k] s_w(n,k) dec(W[n,k]) + bias[n]
 *   x : [M x K] bf16 activations (ldx in elements); xt must be FP8RT_BF16
 *       (FP8RT_F32 returns FP8RT_EUNSUPPORTED)
 *   w : [N x K] FP8 codes (ldw bytes), format fw (E4M3 or E5M2)
 *   scale_w : fp32 [ceil(N/gw.rows)][ceil(K/gw.cols)]; gw.cols 0 / >= K
 *       (tensor, channel, row blocks) or a multiple of 128 (K groups), else
 *       FP8RT_EUNSUPPORTED
 *   bias : nullable [N] fp32 / bf16;  y : [M x N] fp32 / bf16 (ldy)
 * Every FP8 value is exactly a bf16 value: the products x dec(W) are exact,
 * accumulated in FP32; the scale multiplies each K group's partial sum in
 * FP32.  Built for decode shapes (W streamed once per 16 activation rows;
 * larger M re-reads W per 16 rows).  Limits: M <= 16 * 65535.
 * Alignment: K a multiple of 16, ldx a multiple of 8, ldw of 16; x and w
 * 16-byte aligned, scales and fp32 bias / y 4-byte aligned.
 * flags: 0 or FP8RT_B_PACKED16 (w is the fp8_pack_weights16 image of the
 * codes, ldw ignored, K a multiple of 128 else FP8RT_EALIGN; bit-identical to
 * the row-major call); other bits FP8RT_EINVAL. */
fp8rt_status fp8_weight_only_gemm(const void* x, fp8rt_dtype xt, int64_t ldx, const uint8_t* w,
                                  fp8rt_format fw, int64_t ldw, fp8rt_gran gw, const float* scale_w,
                                  int64_t M, int64_t N, int64_t K, const void* bias,
                                  fp8rt_dtype bias_t, void* y, fp8rt_dtype yt, int64_t ldy,
                                  uint32_t flags, hipStream_t stream);

/* Fragment-ordered weight image for the decode GEMMs [the layout is this
 * library's, not the sources': "FP8 formats and scaling for LLM inference",
 * section "Weight scale and activation scale lifetimes" -- a weight is
 * quantized and laid out once, offline, and reused by every call].  For a
 * decode GEMM (M <= 16) the work is streaming the weight; in row-major order
 * each load instruction of the matrix-core fragment touches 16 rows 64 bytes
 * apart, in this order 1 KB contiguous.
 *   q  : [N x K] codes (ldq bytes), K a multiple of 128
 *   qp : fp8_packed16_bytes(N, K) bytes (caller-owned, not overlapping q):
 *        for 16-row group G, 128-byte step s, half h in {0,1}, lane l in
 *        [0,64), byte b in [0,16):
 *          qp[((G * K/128 + s) * 2 + h) * 1024 + 16 l + b]
 *            = q[16 G + l % 16][128 s + 32 (l / 16) + 16 h + b],
 *        0 for rows >= N.
 * One pass, codes copied unchanged.  Errors: null pointers, N or K <= 0,
 * ldq < K, N or K > 2^31: FP8RT_EINVAL; K or ldq not a multiple of 128 / 16,
 * pointers not 16-byte aligned: FP8RT_EALIGN. */
static inline int64_t fp8_packed16_bytes(int64_t N, int64_t K) { return (N + 15) / 16 * 16 * K; }
fp8rt_status fp8_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp,
                                hipStream_t stream);

/* fp8_quantize with the codes written straight into the fragment-ordered
 * weight image [as fp8_pack_weights16: the weight is quantized and laid out
 * once and reused by every call].  Arguments, scales, amax_out, counters
 * and statuses are those of fp8_quantize on x [rows x cols] (rows = N,
 * cols = K), with q replaced by
 *   qp : fp8_packed16_bytes(rows, cols) bytes, 16-byte aligned, caller-owned,
 *        not overlapping x or the scale arrays;
 * on return qp holds exactly what fp8_pack_weights16 makes of the codes
 * fp8_quantize would write (zeros in the rows past `rows` of a short last
 * 16-row group), without the row-major codes and the second pass.
 * Extra conditions: cols a multiple of 128 (else FP8RT_EALIGN), rows and
 * cols <= 2^31 (else FP8RT_EINVAL).  Every granularity of fp8_quantize. */
fp8rt_status fp8_quantize_packed16(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                                   int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                                   float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                                   uint8_t* qp, float* amax_out, uint64_t* sat_underflow,
                                   hipStream_t stream);

/* Quantization error of a weight, for the granularity ledger ["Quantization
 * W8A16" (datawhalechina llm-algo-leetcode): the granularity comparison
 * reports each granularity's restored-weight mean squared error and the layer
 * output's error against the unquantized weight].
 *   w : [N x K] fp32 / bf16 (ldw elements, a multiple of 8), the weight;
 *   q : [N x K] codes (ldq bytes, a multiple of 8) with scales [ceil(N/g.rows)]
 *       [ceil(K/g.cols)] (group widths a multiple of 8 or the whole row);
 *   x : nullable bf16 inputs [M x K] (ldx elements, a multiple of 8);
 *   stats : device double[7], OVERWRITTEN:
 *     {sum e^2, sum w^2, max |e|, sum d^2, sum y_ref^2, sum y_q^2, sum y_ref y_q}
 *     with w_hat = fl32(s dec(q)) (the dequantization), e = w_hat - w (exact),
 *     y_ref = x W^T, y_q = x W_hat^T, d = y_q - y_ref (each dot product an
 *     FP32 accumulation of exact products: e split exactly into three bf16
 *     parts on the matrix cores; squares and sums in binary64; 3..6 are 0
 *     when x is NULL).
 *     NaN propagates (max |e| is NaN when any e is).
 * K a multiple of 16; w and x 16-byte aligned, q and stats 8-byte aligned.
 * Scratch: the per-stream GEMM scratch buffer holds per-block partials. */
fp8rt_status fp8_quant_error(const void* w, fp8rt_dtype wt, int64_t N, int64_t K, int64_t ldw,
                             const uint8_t* q, fp8rt_format f, int64_t ldq, fp8rt_gran g,
                             const float* scale, const void* x, int64_t M, int64_t ldx,
                             double* stats, hipStream_t stream);

/* One granularity of the ledger: the scale groups and the power-of-two
 * round-up of the scales (MX-style 1x32 blocks use {1, 32} with 1). */
typedef struct fp8rt_ledger_spec {
  fp8rt_gran gran;
  int32_t pow2_round_up;
} fp8rt_ledger_spec;

/* One row of the ledger (host memory). */
typedef struct fp8rt_ledger_row {
  fp8rt_gran gran;
  int32_t pow2_round_up;
  int64_t qparam_count;            /* number of fp32 scales */
  int64_t qparam_bytes;            /* 4 * qparam_count */
  int64_t quantized_weight_bytes;  /* N * K code bytes */
  int64_t total_state_bytes;       /* codes + scales */
  double weight_mse;               /* sum e^2 / (N K) */
  double weight_max_abs_err;       /* max |e| */
  double output_mse;               /* sum d^2 / (M N); NaN without inputs */
  double output_cosine;            /* <y_ref, y_q> / max(|y_ref| |y_q|, 1e-8); NaN without inputs */
  uint64_t saturated, underflowed; /* the quantization's counters */
} fp8rt_ledger_row;

/* The FP8 granularity ledger ["Quantization W8A16", the granularity
 * comparison: for one weight and one set of inputs, each granularity's scale
 * count and bytes against the restored weight's and the output's error;
 * "FP8 formats and scaling for LLM inference", section "Per-channel and block
 * scaling": finer groups buy precision with scale metadata].  For each of
 * n_specs (1..64) specs: fp8_quantize(w, spec.gran, f, DYNAMIC, eps,
 * spec.pow2_round_up) into library scratch, then fp8_quant_error, and
 * rows[i] is filled on the host.  Synchronous: the stream is synchronized
 * once per spec.  Arguments as fp8_quant_error; a spec that fp8_quantize
 * rejects returns that status (rows before it are filled).  Scratch: the
 * per-stream GEMM scratch buffer holds the codes (N K bytes), the scales and
 * the partials. */
fp8rt_status fp8_granularity_ledger(const void* w, fp8rt_dtype wt, int64_t N, int64_t K, int64_t ldw,
                                    const void* x, int64_t M, int64_t ldx, fp8rt_format f, float eps,
                                    const fp8rt_ledger_spec* specs, int32_t n_specs,
                                    fp8rt_ledger_row* rows, hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char* fp8rt_status_string(fp8rt_status s);

#ifdef __cplusplus
}
#endif
#endif /* FP8RT_H */
