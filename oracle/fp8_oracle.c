/*
 * fp8_oracle.c -- TEST INFRASTRUCTURE ONLY: the CPU oracle for the FP8
 * runtime chain.  Plain C99, single-threaded, no blocking, no fusion, no
 * reordering beyond what each definition states.  Never linked into, and
 * never called by, the HIP library.
 *
 * Each function cites the passage of the pages it follows (page title and
 * section).  Where the pages leave a step open, the reading taken is stated
 * at the function.
 */
#include "fp8_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Formats.
 * "FP8 formats and scaling for LLM inference", section "How the 8 bits are
 * allocated": E4M3 = 1 sign + 4 exponent + 3 mantissa bits with max finite
 * 448; E5M2 = 1 + 5 + 2 bits with max finite 57344.
 * "FP8 inference: E4M3/E5M2 and the NVIDIA FP8 ecosystem", section "numeric
 * properties": exponent bias 7 (E4M3) and 15 (E5M2); E5M2 has full Inf/NaN,
 * E4M3 only a limited NaN.  Reading: E4M3 is the OCP "fn" variant, whose only
 * NaNs are S.1111.111 (0x7F / 0xFF) and which has no infinities. */

static int mant_bits(int fmt) { return fmt == ORC_E4M3 ? 3 : 2; }
static int exp_bias(int fmt) { return fmt == ORC_E4M3 ? 7 : 15; }
/* Smallest normal exponent: 1 - bias. */
static int min_exp(int fmt) { return 1 - exp_bias(fmt); }
static unsigned max_code(int fmt) { return fmt == ORC_E4M3 ? 0x7Eu : 0x7Bu; }

double orc_fmax(int fmt) { return fmt == ORC_E4M3 ? 448.0 : 57344.0; }

double orc_decode(unsigned code, int fmt) {
    code &= 0xFFu;
    const double sign = (code & 0x80u) ? -1.0 : 1.0;
    const int mb = mant_bits(fmt);
    const unsigned emask = fmt == ORC_E4M3 ? 0xFu : 0x1Fu;
    const unsigned e = (code >> mb) & emask;
    const unsigned m = code & ((1u << mb) - 1u);
    if (fmt == ORC_E4M3) {
        if (e == 15u && m == 7u) return NAN;
    } else {
        if (e == 31u) return m == 0u ? sign * INFINITY : NAN;
    }
    if (e == 0u) /* subnormal: m * 2^(1 - bias - mb) */
        return sign * ldexp((double)m, min_exp(fmt) - mb);
    /* normal: (1 + m / 2^mb) * 2^(e - bias) */
    return sign * ldexp((double)((1u << mb) + m), (int)e - exp_bias(fmt) - mb);
}

/* Saturating encode of an already-scaled binary32 value.
 * "FP8 formats and scaling for LLM inference", section "How a scale fits a
 * tensor into E4M3": X_fp8 = cast(clip(X / s)).  "FP8 production quantization
 * guide", dynamic quantize listing: clamp to +-F_max, then cast.
 * Readings: the clip is to +-F_max (so +-Inf saturate and never produce
 * Inf/NaN codes); the cast rounds to nearest with ties to even onto the full
 * OCP grid including subnormals; the sign of zero is kept; NaN -> 0x7F. */
unsigned orc_encode(float v, int fmt) {
    if (isnan(v)) return 0x7Fu;
    const unsigned sign = signbit(v) ? 0x80u : 0u;
    const double a = fabs((double)v);
    if (a > orc_fmax(fmt)) return sign | max_code(fmt);
    if (a == 0.0) return sign;
    const int mb = mant_bits(fmt);
    const int emin = min_exp(fmt);
    int e2;
    (void)frexp(a, &e2);           /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;                /* floor(log2 a) */
    if (E < emin) E = emin;        /* subnormal binade shares the quantum */
    const double quantum = ldexp(1.0, E - mb);
    const double n = nearbyint(a / quantum); /* exact divide; RNE */
    const double r = n * quantum;  /* a carry into the next binade is fine */
    if (r == 0.0) return sign;
    (void)frexp(r, &e2);
    const int Er = e2 - 1;
    if (Er < emin) /* subnormal code: exponent field 0, mantissa = r / 2^(emin-mb) */
        return sign | (unsigned)(r / ldexp(1.0, emin - mb));
    const unsigned mant = (unsigned)(r / ldexp(1.0, Er - mb)) - (1u << mb);
    return sign | ((unsigned)(Er + exp_bias(fmt)) << mb) | mant;
}

unsigned orc_encode_bruteforce(float v, int fmt) {
    if (isnan(v)) return 0x7Fu;
    const unsigned sign = signbit(v) ? 0x80u : 0u;
    double a = fabs((double)v);
    if (a > orc_fmax(fmt)) a = orc_fmax(fmt);
    unsigned best = 0;
    double best_d = INFINITY;
    for (unsigned c = 0; c < 0x80u; ++c) {
        const double d = orc_decode(c, fmt);
        if (!isfinite(d)) continue;
        const double dist = fabs(d - a);
        const int mant_even = (c & 1u) == 0u;
        if (dist < best_d || (dist == best_d && mant_even)) {
            best_d = dist;
            best = c;
        }
    }
    return sign | best;
}

/* ------------------------------------------------------------------------ */

float orc_load(const void* x, int dtype, int64_t i) {
    if (dtype == ORC_BF16) {
        uint16_t h;
        memcpy(&h, (const char*)x + 2 * i, 2);
        const uint32_t bits = (uint32_t)h << 16; /* bf16 is the top half of binary32 */
        float f;
        memcpy(&f, &bits, 4);
        return f;
    }
    float f;
    memcpy(&f, (const char*)x + 4 * i, 4);
    return f;
}

int64_t orc_ngroups(int64_t n, int64_t g) {
    if (g <= 0 || g >= n) return 1;
    return (n + g - 1) / g; /* the tail group is kept */
}

static int64_t eff(int64_t n, int64_t g) { return (g <= 0 || g > n) ? n : g; }

/* Per-group amax.
 * "FP8 formats and scaling for LLM inference", section "How a scale fits a
 * tensor into E4M3" (a_max = max|X|) and section "Per-channel and block
 * scaling" (a_g per block).  Groups tile the matrix with extents gr x gc;
 * the last row / column group may be short (tail groups are kept, as the
 * "Quantization W8A16" page's per-group granularity requires).
 * Reading: any NaN in a group makes its amax NaN. */
int orc_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
             int64_t gr, int64_t gc, float* amax) {
    if (!x || !amax || rows <= 0 || cols <= 0 || ldx < cols) return 1;
    const int64_t er = eff(rows, gr), ec = eff(cols, gc);
    const int64_t nR = orc_ngroups(rows, gr), nC = orc_ngroups(cols, gc);
    for (int64_t g = 0; g < nR * nC; ++g) amax[g] = 0.0f;
    char* has_nan = calloc((size_t)(nR * nC), 1);
    if (!has_nan) return 1;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            const int64_t g = (i / er) * nC + (j / ec);
            const float a = fabsf(orc_load(x, dtype, i * ldx + j));
            if (isnan(a)) has_nan[g] = 1;
            else if (a > amax[g]) amax[g] = a;
        }
    }
    for (int64_t g = 0; g < nR * nC; ++g)
        if (has_nan[g]) amax[g] = NAN;
    free(has_nan);
    return 0;
}

/* Scale from amax.
 * "FP8 formats and scaling for LLM inference", section "How a scale fits a
 * tensor into E4M3": s = a_max / F_max; the same section lists power-of-two
 * rounding among recipe options.  "FP8 production quantization guide",
 * dynamic quantize listing: amax is clamped from below by eps, then
 * scale = amax / F_max and inv_scale = F_max / amax.
 * Readings: a_c = max(a, eps); s and r are each the correctly rounded
 * binary32 quotient; pow2 rounds s up to 2^ceil(log2 s) and sets r = 1/s;
 * a non-finite amax gives NaN s and r. */
int orc_compute_scale(const float* amax, int64_t n, int fmt, float eps, int pow2,
                      float* s, float* r) {
    if (!amax || !s || n <= 0) return 1;
    const double F = orc_fmax(fmt);
    for (int64_t g = 0; g < n; ++g) {
        const float a = amax[g];
        float sg, rg;
        if (!isfinite(a)) {
            sg = NAN;
            rg = NAN;
        } else {
            const float ac = a < eps ? eps : a;
            sg = (float)((double)ac / F);
            rg = (float)(F / (double)ac);
            if (pow2) {
                int e2;
                const double f = frexp((double)sg, &e2); /* sg = f * 2^e2 */
                if (f != 0.5) sg = (float)ldexp(1.0, e2); /* not already 2^k: round up */
                rg = (float)(1.0 / (double)sg);
            }
        }
        s[g] = sg;
        if (r) r[g] = rg;
    }
    return 0;
}

/* Quantize with per-group scales and the saturation / underflow statistics.
 * "FP8 formats and scaling for LLM inference", sections "How a scale fits a
 * tensor into E4M3", "Current scaling" (reduce amax -> scale -> cast in the
 * same step), "Weight scale and activation scale lifetimes" (static scales
 * given from outside), "What numerical validation looks at" (saturation /
 * clipping rate and underflow / zero rate).  "FP8 production quantization
 * guide", dynamic quantize listing (multiply by inv_scale, clamp, cast).
 * Readings: v = fl32(x * r) with r = fl32(F_max / a_c) (or fl32(1/s) when only
 * s is given); saturated means |v| > F_max strictly (Inf included, NaN not);
 * underflowed means x != 0 but the code is +-0. */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                 int64_t gr, int64_t gc, int fmt, int mode, float eps, int pow2,
                 float* s, float* r, uint8_t* q, int64_t ldq,
                 float* amax_out, uint64_t* counts) {
    if (!x || !s || !q || rows <= 0 || cols <= 0 || ldx < cols || ldq < cols) return 1;
    const int64_t er = eff(rows, gr), ec = eff(cols, gc);
    const int64_t nR = orc_ngroups(rows, gr), nC = orc_ngroups(cols, gc);
    const int64_t G = nR * nC;
    float* amax = malloc((size_t)G * sizeof(float));
    float* rr = malloc((size_t)G * sizeof(float));
    if (!amax || !rr) { free(amax); free(rr); return 1; }
    orc_amax(x, dtype, rows, cols, ldx, gr, gc, amax);
    if (mode == ORC_DYNAMIC) {
        orc_compute_scale(amax, G, fmt, eps, pow2, s, rr);
        if (r) memcpy(r, rr, (size_t)G * sizeof(float));
    } else {
        for (int64_t g = 0; g < G; ++g)
            rr[g] = r ? r[g] : (float)(1.0 / (double)s[g]);
    }
    const double F = orc_fmax(fmt);
    uint64_t sat = 0, under = 0;
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            const int64_t g = (i / er) * nC + (j / ec);
            const float xv = orc_load(x, dtype, i * ldx + j);
            const float v = (float)((double)xv * (double)rr[g]);
            if (fabs((double)v) > F) ++sat;
            const unsigned c = orc_encode(v, fmt);
            if (xv != 0.0f && (c == 0x00u || c == 0x80u)) ++under;
            q[i * ldq + j] = (uint8_t)c;
        }
    }
    if (amax_out) memcpy(amax_out, amax, (size_t)G * sizeof(float));
    if (counts) { counts[0] = sat; counts[1] = under; }
    free(amax);
    free(rr);
    return 0;
}

/* Cast-transpose.  "FP8 formats and scaling for LLM inference", section "How
 * the 8 bits are allocated": the hybrid recipe keeps E4M3 for the forward
 * pass and E5M2 for the backward gradients, and a backward GEMM reads the
 * operand in the other orientation; "FP8 inference: E4M3/E5M2 and the NVIDIA
 * FP8 ecosystem", QAT section: forward and backward both run through FP8.
 * Definition: the quantize above (same groups, scales and counters), with
 * every code also written transposed, qt[j][i] = q[i][j]. */
int orc_quantize_transpose(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ldx,
                           int64_t gr, int64_t gc, int fmt, int mode, float eps, int pow2,
                           float* s, float* r, uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                           float* amax_out, uint64_t* counts) {
    if (!qt || ldqt < rows) return 1;
    const int rc = orc_quantize(x, dtype, rows, cols, ldx, gr, gc, fmt, mode, eps, pow2, s, r, q, ldq,
                                amax_out, counts);
    if (rc) return rc;
    for (int64_t i = 0; i < rows; ++i)
        for (int64_t j = 0; j < cols; ++j) qt[j * ldqt + i] = q[i * ldq + j];
    return 0;
}

/* Dequantize.  "FP8 formats and scaling for LLM inference", section "How a
 * scale fits a tensor into E4M3": X_hat = s * X_fp8.  "FP8 inference:
 * E4M3/E5M2 and the NVIDIA FP8 ecosystem", dequantization example.
 * Reading: the product is rounded once to binary32; a bf16 output rounds that
 * binary32 to nearest even. */
int orc_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                   int64_t gr, int64_t gc, const float* s, void* y, int out_dtype,
                   int64_t ldy) {
    if (!q || !s || !y || rows <= 0 || cols <= 0 || ldq < cols || ldy < cols) return 1;
    const int64_t er = eff(rows, gr), ec = eff(cols, gc);
    const int64_t nC = orc_ngroups(cols, gc);
    for (int64_t i = 0; i < rows; ++i) {
        for (int64_t j = 0; j < cols; ++j) {
            const int64_t g = (i / er) * nC + (j / ec);
            const float v = (float)((double)s[g] * orc_decode(q[i * ldq + j], fmt));
            if (out_dtype == ORC_BF16) {
                const uint16_t h = orc_round_bf16_from_f32(v);
                memcpy((char*)y + 2 * (i * ldy + j), &h, 2);
            } else {
                memcpy((char*)y + 4 * (i * ldy + j), &v, 4);
            }
        }
    }
    return 0;
}

/* Delayed scaling.  "FP8 formats and scaling for LLM inference", section
 * "Delayed scaling": step t quantizes with a scale from history up to t-1,
 * collects a_t, and s_{t+1} = f(a_t, ..., a_{t-h+1}) / F_max with f the most
 * recent value or the window maximum.
 * Readings: f = window maximum over a ring of h entries that starts at zero
 * (a partial window is the maximum over the entries seen so far, since amax
 * is never negative); the window includes a_t; the eps clamp and the optional
 * power-of-two rounding apply as for current scaling; NaN propagates. */
int orc_history_update(float* hist, int len, int* head, float amax_new, int fmt,
                       float eps, int pow2, float* s_next, float* r_next) {
    if (!hist || !head || len <= 0 || *head < 0 || *head >= len || !s_next) return 1;
    hist[*head] = amax_new;
    *head = (*head + 1) % len;
    float a = 0.0f;
    int nan = 0;
    for (int i = 0; i < len; ++i) {
        if (isnan(hist[i])) nan = 1;
        else if (hist[i] > a) a = hist[i];
    }
    if (nan) a = NAN;
    return orc_compute_scale(&a, 1, fmt, eps, pow2, s_next, r_next);
}

/* Delayed-scaling recipe variants (same section: the history function may be
 * the most recent value, the window maximum or another rule; real recipes add
 * a margin).  fn ORC_HIST_MAX is orc_history_update's window maximum;
 * ORC_HIST_LATEST uses a_t alone (a non-positive a_t counts as 0, NaN
 * propagates).  Reading of the margin m (0..16): the amax the scale is derived
 * from is a * 2^m, so s grows by exactly 2^m (an overflow to Inf gives NaN s
 * and r, as any non-finite amax does). */
int orc_history_update_recipe(float* hist, int len, int* head, float amax_new, int fmt, int fn,
                              int margin, float eps, int pow2, float* s_next, float* r_next) {
    if (!hist || !head || len <= 0 || *head < 0 || *head >= len || !s_next) return 1;
    if ((fn != ORC_HIST_MAX && fn != ORC_HIST_LATEST) || margin < 0 || margin > 16) return 1;
    hist[*head] = amax_new;
    *head = (*head + 1) % len;
    float a = 0.0f;
    if (fn == ORC_HIST_LATEST) {
        a = isnan(amax_new) ? NAN : (amax_new > 0.0f ? amax_new : 0.0f);
    } else {
        int nan = 0;
        for (int i = 0; i < len; ++i) {
            if (isnan(hist[i])) nan = 1;
            else if (hist[i] > a) a = hist[i];
        }
        if (nan) a = NAN;
    }
    a = (float)ldexp((double)a, margin);
    return orc_compute_scale(&a, 1, fmt, eps, pow2, s_next, r_next);
}

/* ------------------------------------------------------------------------ */
/* Scaled GEMM.  "FP8 formats and scaling for LLM inference", section "The full
 * precision contract of one FP8 GEMM": X ~ s_x X8, W ~ s_w W8,
 * Y ~ s_x s_w (X8 W8), accumulated in higher precision, with bias fusion and
 * a BF16/FP32 output.  "FP8 production quantization guide", GEMM listing
 * (scale_a, scale_b, out_dtype, bias).  Per-block scales ("Per-channel and
 * block scaling") enter per element: s_a(m,k) s_b(n,k).
 * Orientation: A is [M x K], B is [N x K] (the nn.Linear weight layout), both
 * K-contiguous, Y = A B^T. */

static float scale_at(const float* s, int64_t rows, int64_t cols, int64_t gr, int64_t gc,
                      int64_t i, int64_t k) {
    const int64_t er = eff(rows, gr), ec = eff(cols, gc);
    const int64_t nC = orc_ngroups(cols, gc);
    return s[(i / er) * nC + (k / ec)];
}

static double bias_at(const void* bias, int dt, int64_t n) {
    if (!bias) return 0.0;
    return (double)orc_load(bias, dt == ORC_BF16 ? ORC_BF16 : ORC_F32, n);
}

/* orc_decode of every code, memoized (the same values, looked up). */
static const double* decode_table(int fmt) {
    static double tab[2][256];
    static int ready[2] = {0, 0};
    const int f = fmt == ORC_E4M3 ? 0 : 1;
    if (!ready[f]) {
        for (unsigned c = 0; c < 256; ++c) tab[f][c] = orc_decode(c, fmt);
        ready[f] = 1;
    }
    return tab[f];
}

int orc_gemm_points(const uint8_t* a, int fa, int64_t lda, int64_t gra, int64_t gca,
                    const float* sa, const uint8_t* b, int fb, int64_t ldb,
                    int64_t grb, int64_t gcb, const float* sb, int64_t M, int64_t N,
                    int64_t K, const void* bias, int bias_dtype, const int64_t* m,
                    const int64_t* n, int64_t npts, double* y, double* S) {
    if (!a || !b || !sa || !sb || !m || !n || !y || M <= 0 || N <= 0 || K <= 0) return 1;
    const double* da = decode_table(fa);
    const double* db = decode_table(fb);
    const int64_t ca = eff(K, gca), cb = eff(K, gcb);
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t mi = m[p], ni = n[p];
        if (mi < 0 || mi >= M || ni < 0 || ni >= N) return 1;
        const uint8_t* ar = a + mi * lda;
        const uint8_t* br = b + ni * ldb;
        double acc = 0.0, absacc = 0.0;
        int64_t k = 0;
        while (k < K) {
            /* scales are constant up to the next K-block boundary of either operand */
            int64_t end = (k / ca + 1) * ca;
            const int64_t end_b = (k / cb + 1) * cb;
            if (end_b < end) end = end_b;
            if (K < end) end = K;
            const double s1 = (double)scale_at(sa, M, K, gra, gca, mi, k);
            const double s2 = (double)scale_at(sb, N, K, grb, gcb, ni, k);
            for (; k < end; ++k) {
                const double t = s1 * s2 * da[ar[k]] * db[br[k]];
                acc += t;
                absacc += fabs(t);
            }
        }
        y[p] = acc + bias_at(bias, bias_dtype, ni);
        if (S) S[p] = absacc;
    }
    return 0;
}

/* Weight-only FP8 ("FP8 formats and scaling for LLM inference", section
 * "Weight-only FP8 and W8A8 FP8": weights stored as FP8 with their scales,
 * activations kept in BF16, the weight restored inside the GEMM).  The
 * restored weight is the exact real value s_w * dec(code); every product
 * x * s_w * dec is exact in binary64 (8 + 24 + 4 significant bits), and the
 * products are summed in k order. */
int orc_wonly_gemm_points(const void* x, int xdtype, int64_t ldx, const uint8_t* w, int fw,
                          int64_t ldw, int64_t grw, int64_t gcw, const float* sw, int64_t M,
                          int64_t N, int64_t K, const void* bias, int bias_dtype,
                          const int64_t* m, const int64_t* n, int64_t npts, double* y,
                          double* S) {
    if (!x || !w || !sw || !m || !n || !y || M <= 0 || N <= 0 || K <= 0) return 1;
    const double* dw = decode_table(fw);
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t mi = m[p], ni = n[p];
        if (mi < 0 || mi >= M || ni < 0 || ni >= N) return 1;
        double acc = 0.0, absacc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double xv = (double)orc_load(x, xdtype, mi * ldx + k);
            const double t = xv * (double)scale_at(sw, N, K, grw, gcw, ni, k) * dw[w[ni * ldw + k]];
            acc += t;
            absacc += fabs(t);
        }
        y[p] = acc + bias_at(bias, bias_dtype, ni);
        if (S) S[p] = absacc;
    }
    return 0;
}

/* Reconstruction error of a quantized weight, for the granularity ledger
 * ("Quantization W8A16", the granularity comparison: per granularity the
 * scale count and bytes, the restored weight's mean squared error, and the
 * layer output's squared error and cosine against the unquantized weight).
 * The restored weight is the dequantization fl32(s * dec(q)); e = w_hat - w
 * exactly (binary64).  With inputs x [M x K]: y_ref = x W^T and
 * y_q = x W_hat^T in binary64, d = y_q - y_ref = x e^T.
 * stats[0] = sum e^2, [1] = sum w^2, [2] = max |e|, [3] = sum d^2,
 * [4] = sum y_ref^2, [5] = sum y_q^2, [6] = sum y_ref y_q (3..6 zero when
 * x is NULL). */
int orc_quant_error(const void* w, int wdtype, int64_t N, int64_t K, int64_t ldw, const uint8_t* q,
                    int fmt, int64_t ldq, int64_t gr, int64_t gc, const float* scale, const void* x,
                    int64_t M, int64_t ldx, double* stats) {
    if (!w || !q || !scale || !stats || N <= 0 || K <= 0 || ldw < K || ldq < K) return 1;
    if (x && (M <= 0 || ldx < K)) return 1;
    const int64_t er = eff(N, gr), ec = eff(K, gc);
    const int64_t nC = orc_ngroups(K, gc);
    double* e = (double*)malloc(sizeof(double) * (size_t)K);
    double* wv = (double*)malloc(sizeof(double) * (size_t)K);
    if (!e || !wv) { free(e); free(wv); return 1; }
    for (int i = 0; i < 7; ++i) stats[i] = 0.0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            const double sv = (double)scale[(n / er) * nC + (k / ec)];
            const float wh = (float)(sv * orc_decode(q[n * ldq + k], fmt));
            wv[k] = (double)orc_load(w, wdtype, n * ldw + k);
            e[k] = (double)wh - wv[k];
            stats[0] += e[k] * e[k];
            stats[1] += wv[k] * wv[k];
            const double ae = fabs(e[k]);
            if (isnan(ae)) stats[2] = NAN;                 /* NaN propagates */
            else if (ae > stats[2]) stats[2] = ae;         /* false once stats[2] is NaN */
        }
        if (!x) continue;
        for (int64_t m = 0; m < M; ++m) {
            double d = 0.0, yr = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double xv = (double)orc_load(x, ORC_BF16, m * ldx + k);
                d += xv * e[k];
                yr += xv * wv[k];
            }
            const double yq = yr + d;
            stats[3] += d * d;
            stats[4] += yr * yr;
            stats[5] += yq * yq;
            stats[6] += yr * yq;
        }
    }
    free(e);
    free(wv);
    return 0;
}

/* Fragment-ordered weight codes (a layout of the same codes, no arithmetic):
 * rows in groups of 16, K in steps of 128; the 2048 bytes of (group G, step s)
 * hold at byte h * 1024 + l * 16 + b (h in {0,1}, lane l in 0..63, b in 0..15)
 * the code W[16 G + l % 16][128 s + 32 (l / 16) + 16 h + b], or 0 past the
 * last row.  Requires K % 128 == 0; qp holds ceil(N/16) * 16 * K bytes. */
int orc_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp) {
    if (!q || !qp || N <= 0 || K <= 0 || K % 128 != 0 || ldq < K) return 1;
    const int64_t steps = K / 128, groups = (N + 15) / 16;
    for (int64_t G = 0; G < groups; ++G)
        for (int64_t st = 0; st < steps; ++st)
            for (int h = 0; h < 2; ++h)
                for (int l = 0; l < 64; ++l)
                    for (int b = 0; b < 16; ++b) {
                        const int64_t row = 16 * G + l % 16;
                        const int64_t col = 128 * st + 32 * (l / 16) + 16 * h + b;
                        qp[(G * steps + st) * 2048 + h * 1024 + l * 16 + b] = row < N ? q[row * ldq + col] : 0;
                    }
    return 0;
}

/* Integer value of a code in units of the format's smallest subnormal
 * (2^-9 for E4M3, 2^-16 for E5M2); returns 0 and sets *bad for NaN/Inf. */
static int64_t code_units(unsigned code, int fmt, int* bad) {
    const double d = orc_decode(code, fmt);
    if (!isfinite(d)) { *bad = 1; return 0; }
    return (int64_t)ldexp(d, fmt == ORC_E4M3 ? 9 : 16);
}

int orc_gemm_points_exact(const uint8_t* a, int fa, int64_t lda, int64_t gra, int64_t gca,
                          const float* sa, const uint8_t* b, int fb, int64_t ldb,
                          int64_t grb, int64_t gcb, const float* sb, int64_t M,
                          int64_t N, int64_t K, const void* bias, int bias_dtype,
                          const int64_t* m, const int64_t* n, int64_t npts, double* y) {
    if (!a || !b || !sa || !sb || !m || !n || !y || M <= 0 || N <= 0 || K <= 0) return 1;
    const int qexp = -((fa == ORC_E4M3 ? 9 : 16) + (fb == ORC_E4M3 ? 9 : 16));
    for (int64_t p = 0; p < npts; ++p) {
        const int64_t mi = m[p], ni = n[p];
        if (mi < 0 || mi >= M || ni < 0 || ni >= N) return 1;
        double acc = 0.0;
        int bad = 0;
        const int64_t ca = eff(K, gca), cb = eff(K, gcb);
        int64_t k = 0;
        while (k < K) {
            /* a run ends at the next K-block boundary of either operand */
            int64_t end = (k / ca + 1) * ca;
            const int64_t end_b = (k / cb + 1) * cb;
            if (end_b < end) end = end_b;
            if (K < end) end = K;
            __int128 run = 0;
            for (int64_t k2 = k; k2 < end; ++k2)
                run += (__int128)code_units(a[mi * lda + k2], fa, &bad) *
                       (__int128)code_units(b[ni * ldb + k2], fb, &bad);
            acc += (double)scale_at(sa, M, K, gra, gca, mi, k) *
                   (double)scale_at(sb, N, K, grb, gcb, ni, k) * ldexp((double)run, qexp);
            k = end;
        }
        y[p] = bad ? NAN : acc + bias_at(bias, bias_dtype, ni);
    }
    return 0;
}

/* Round to bfloat16 (8 significant bits, exponent range of binary32), nearest
 * with ties to even; overflow past the largest finite value rounds to Inf. */
uint16_t orc_round_bf16(double v) {
    if (isnan(v)) return 0x7FC0u;
    const uint16_t sign = signbit(v) ? 0x8000u : 0u;
    if (isinf(v)) return sign | 0x7F80u;
    const double a = fabs(v);
    if (a == 0.0) return sign;
    int e2;
    (void)frexp(a, &e2);
    int E = e2 - 1;
    if (E < -126) E = -126;
    const double quantum = ldexp(1.0, E - 7);
    const double r = nearbyint(a / quantum) * quantum;
    if (r >= 0x1p128) return sign | 0x7F80u;
    const float f = (float)r; /* exact: r has at most 8 significant bits */
    uint32_t bits;
    memcpy(&bits, &f, 4);
    return sign | (uint16_t)(bits >> 16);
}

uint16_t orc_round_bf16_from_f32(float v) { return orc_round_bf16((double)v); }
