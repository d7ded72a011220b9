// api.hip -- the C ABI of include/fp8rt.h: host-side argument validation and
// dispatch to the gfx950 kernels.  Every check runs before anything is
// enqueued; on an error nothing is written.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <cmath>
#include <limits>

#include "fp8rt.h"
#include "internal.h"

using namespace fp8rt;

namespace {

constexpr float kMinEps = 0x1p-96f;  // keeps r = F_max / eps finite for both formats

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }
bool valid_fmt(int f) { return f == FP8RT_E4M3 || f == FP8RT_E5M2; }
bool valid_dtype(int d) { return d == FP8RT_F32 || d == FP8RT_BF16; }
bool valid_eps(float e) { return isfinite(e) && e >= kMinEps; }

fp8rt_status from_hip(hipError_t e) { return e == hipSuccess ? FP8RT_OK : FP8RT_EHIP; }

// Common checks of a [rows x cols] row-major operand with group extents g.
fp8rt_status check_matrix(const void* p, int64_t rows, int64_t cols, int64_t ld, fp8rt_gran g) {
  if (!p) return FP8RT_EINVAL;
  if (rows <= 0 || cols <= 0 || ld < cols) return FP8RT_EINVAL;
  if (g.rows < 0 || g.cols < 0) return FP8RT_EINVAL;
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (cols % 16 != 0 || ld % 16 != 0) return FP8RT_EALIGN;
  const int64_t ec = group_extent(cols, g.cols);
  if (ec != cols && ec % 16 != 0) return FP8RT_EALIGN;
  if (!aligned16(p)) return FP8RT_EALIGN;
  return FP8RT_OK;
}

// fp8_quantize and fp8_quantize_packed16: q row-major with pitch ldq
// (img == 0), or the weight image of a matrix of cols = 128 img columns.
fp8rt_status quantize_to(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                         fp8rt_gran g, fp8rt_format f, fp8rt_mode mode, float eps, int32_t pow2_round_up,
                         float* scale, float* inv_scale, uint8_t* q, int64_t ldq, int64_t img,
                         float* amax_out, uint64_t* sat_underflow, hipStream_t stream) {
  if (!valid_dtype(xt) || !valid_fmt(f) || !scale || !q) return FP8RT_EINVAL;
  if (mode != FP8RT_DYNAMIC && mode != FP8RT_GIVEN) return FP8RT_EINVAL;
  if (mode == FP8RT_DYNAMIC && !valid_eps(eps)) return FP8RT_EINVAL;
  fp8rt_status st = check_matrix(x, rows, cols, ldx, g);
  if (st != FP8RT_OK) return st;
  if (ldq < cols) return FP8RT_EINVAL;
  if (ldq % 16 != 0 || !aligned16(q)) return FP8RT_EALIGN;
  if (!aligned4(scale) || (inv_scale && !aligned4(inv_scale)) || (amax_out && !aligned4(amax_out)) ||
      (sat_underflow && (reinterpret_cast<uintptr_t>(sat_underflow) & 7u)))
    return FP8RT_EALIGN;
  QuantArgs a{};
  a.x = x;
  a.xt = xt;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.er = group_extent(rows, g.rows);
  a.ec = group_extent(cols, g.cols);
  a.fmt = f;
  a.mode = mode;
  a.eps = mode == FP8RT_DYNAMIC ? eps : 1.0f;
  a.pow2 = pow2_round_up != 0;
  a.scale = scale;
  a.inv_scale = inv_scale;
  a.q = q;
  a.ldq = ldq;
  a.img = img;
  a.amax_out = amax_out;
  a.counts = reinterpret_cast<unsigned long long*>(sat_underflow);
  a.amax_only = false;
  return from_hip(launch_quantize(a, stream));
}

}  // namespace

extern "C" {

const char* fp8rt_status_string(fp8rt_status s) {
  switch (s) {
    case FP8RT_OK: return "ok";
    case FP8RT_EINVAL: return "invalid argument";
    case FP8RT_EALIGN: return "misaligned size, leading dimension or pointer (16 required)";
    case FP8RT_EUNSUPPORTED: return "unsupported format or scale-granularity combination";
    case FP8RT_EHIP: return "HIP launch error";
    case FP8RT_ESCRATCH: return "the call needs more scratch than the allocation-free entry point's fixed 16 MiB";
  }
  return "unknown status";
}

fp8rt_status fp8_amax(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols, int64_t ldx,
                      fp8rt_gran g, float* amax, hipStream_t stream) {
  if (!valid_dtype(xt) || !amax) return FP8RT_EINVAL;
  fp8rt_status st = check_matrix(x, rows, cols, ldx, g);
  if (st != FP8RT_OK) return st;
  if (!aligned4(amax)) return FP8RT_EALIGN;
  QuantArgs a{};
  a.x = x;
  a.xt = xt;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.er = group_extent(rows, g.rows);
  a.ec = group_extent(cols, g.cols);
  a.fmt = FP8RT_E4M3;
  a.mode = FP8RT_DYNAMIC;
  a.eps = 1.0f;
  a.ldq = cols;
  a.amax_out = amax;
  a.amax_only = true;
  return from_hip(launch_quantize(a, stream));
}

fp8rt_status fp8_compute_scale(const float* amax, int64_t n, fp8rt_format f, float eps,
                               int32_t pow2_round_up, float* scale, float* inv_scale,
                               hipStream_t stream) {
  if (!amax || !scale || n <= 0 || !valid_fmt(f) || !valid_eps(eps)) return FP8RT_EINVAL;
  if (!aligned4(amax) || !aligned4(scale) || (inv_scale && !aligned4(inv_scale))) return FP8RT_EALIGN;
  return from_hip(launch_compute_scale(amax, n, f, eps, pow2_round_up != 0, scale, inv_scale, stream));
}

fp8rt_status fp8_quantize(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                          int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                          float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                          uint8_t* q, int64_t ldq, float* amax_out, uint64_t* sat_underflow,
                          hipStream_t stream) {
  return quantize_to(x, xt, rows, cols, ldx, g, f, mode, eps, pow2_round_up, scale, inv_scale, q, ldq, 0,
                     amax_out, sat_underflow, stream);
}

fp8rt_status fp8_quantize_packed16(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                                   int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                                   float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                                   uint8_t* qp, float* amax_out, uint64_t* sat_underflow,
                                   hipStream_t stream) {
  // the limits of fp8_pack_weights16; the rest is fp8_quantize's validation
  if (rows > (int64_t(1) << 31) || cols > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (cols > 0 && cols % 128 != 0) return FP8RT_EALIGN;
  return quantize_to(x, xt, rows, cols, ldx, g, f, mode, eps, pow2_round_up, scale, inv_scale, qp, cols,
                     cols / 128, amax_out, sat_underflow, stream);
}

fp8rt_status fp8_quantize_transpose(const void* x, fp8rt_dtype xt, int64_t rows, int64_t cols,
                                    int64_t ldx, fp8rt_gran g, fp8rt_format f, fp8rt_mode mode,
                                    float eps, int32_t pow2_round_up, float* scale, float* inv_scale,
                                    uint8_t* q, int64_t ldq, uint8_t* qt, int64_t ldqt,
                                    float* amax_out, uint64_t* sat_underflow, hipStream_t stream) {
  if (!valid_dtype(xt) || !valid_fmt(f) || !scale || !q || !qt) return FP8RT_EINVAL;
  if (mode != FP8RT_DYNAMIC && mode != FP8RT_GIVEN) return FP8RT_EINVAL;
  if (mode == FP8RT_DYNAMIC && !valid_eps(eps)) return FP8RT_EINVAL;
  // one-column groups are read whole by this kernel: the 16-wide group rule
  // of the quantize kernels does not apply to them
  fp8rt_gran gc = g;
  if (g.cols == 1 && group_extent(rows, g.rows) == rows) gc.cols = 0;
  fp8rt_status st = check_matrix(x, rows, cols, ldx, gc);
  if (st != FP8RT_OK) return st;
  if (ldq < cols || ldqt < rows) return FP8RT_EINVAL;
  if (rows % 16 != 0 || ldq % 16 != 0 || ldqt % 16 != 0 || !aligned16(q) || !aligned16(qt))
    return FP8RT_EALIGN;
  if (!aligned4(scale) || (inv_scale && !aligned4(inv_scale)) || (amax_out && !aligned4(amax_out)) ||
      (sat_underflow && (reinterpret_cast<uintptr_t>(sat_underflow) & 7u)))
    return FP8RT_EALIGN;
  const int64_t er = group_extent(rows, g.rows), ec = group_extent(cols, g.cols);
  const bool tensor = er == rows && ec == cols, row = er == 1 && ec == cols, col = er == rows && ec == 1;
  if (!tensor && !row && !col) return FP8RT_EUNSUPPORTED;
  QuantArgs a{};
  a.x = x;
  a.xt = xt;
  a.rows = rows;
  a.cols = cols;
  a.ldx = ldx;
  a.er = er;
  a.ec = ec;
  a.fmt = f;
  a.mode = mode;
  a.eps = mode == FP8RT_DYNAMIC ? eps : 1.0f;
  a.pow2 = pow2_round_up != 0;
  a.scale = scale;
  a.inv_scale = inv_scale;
  a.q = q;
  a.ldq = ldq;
  a.amax_out = amax_out;
  a.counts = reinterpret_cast<unsigned long long*>(sat_underflow);
  a.amax_only = false;
  return from_hip(launch_quantize_transpose(a, qt, ldqt, stream));
}

fp8rt_status fp8_dequantize(const uint8_t* q, fp8rt_format f, int64_t rows, int64_t cols,
                            int64_t ldq, fp8rt_gran g, const float* scale, void* y,
                            fp8rt_dtype yt, int64_t ldy, hipStream_t stream) {
  if (!valid_fmt(f) || !valid_dtype(yt) || !scale || !y) return FP8RT_EINVAL;
  fp8rt_status st = check_matrix(q, rows, cols, ldq, g);
  if (st != FP8RT_OK) return st;
  if (ldy < cols) return FP8RT_EINVAL;
  if (ldy % 16 != 0 || !aligned16(y) || !aligned4(scale)) return FP8RT_EALIGN;
  return from_hip(launch_dequantize(q, f, rows, cols, ldq, group_extent(rows, g.rows),
                                    group_extent(cols, g.cols), scale, y, yt, ldy, stream));
}

fp8rt_status fp8_amax_history_update(float* history, int32_t len, int32_t* head,
                                     const float* amax_new, fp8rt_format f, float eps,
                                     int32_t pow2_round_up, float* scale_next,
                                     float* inv_scale_next, hipStream_t stream) {
  if (!history || !head || !amax_new || !scale_next || !valid_fmt(f) || !valid_eps(eps))
    return FP8RT_EINVAL;
  if (len < 1 || len > 1024) return FP8RT_EINVAL;
  if (!aligned4(history) || !aligned4(head) || !aligned4(amax_new) || !aligned4(scale_next) ||
      (inv_scale_next && !aligned4(inv_scale_next)))
    return FP8RT_EALIGN;
  return from_hip(launch_history_update(history, len, head, amax_new, f, eps, pow2_round_up != 0, 0, 0,
                                        scale_next, inv_scale_next, stream));
}

fp8rt_status fp8_delayed_scale_update(float* history, int32_t len, int32_t* head, const float* amax_new,
                                      fp8rt_format f, fp8rt_history_fn fn, int32_t margin, float eps,
                                      int32_t pow2_round_up, float* scale_next, float* inv_scale_next,
                                      hipStream_t stream) {
  if (!history || !head || !amax_new || !scale_next || !valid_fmt(f) || !valid_eps(eps))
    return FP8RT_EINVAL;
  if (len < 1 || len > 1024) return FP8RT_EINVAL;
  if ((fn != FP8RT_HIST_MAX && fn != FP8RT_HIST_LATEST) || margin < 0 || margin > 16) return FP8RT_EINVAL;
  if (!aligned4(history) || !aligned4(head) || !aligned4(amax_new) || !aligned4(scale_next) ||
      (inv_scale_next && !aligned4(inv_scale_next)))
    return FP8RT_EALIGN;
  return from_hip(launch_history_update(history, len, head, amax_new, f, eps, pow2_round_up != 0,
                                        fn == FP8RT_HIST_LATEST ? 1 : 0, margin, scale_next, inv_scale_next,
                                        stream));
}

namespace {

// Validation shared by the two GEMM entry points; fills g (output fields
// excepted) and returns FP8RT_OK, or the status to return.
fp8rt_status gemm_setup(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga, const float* scale_a,
                        const uint8_t* b, fp8rt_format fb, int64_t ldb, fp8rt_gran gb, const float* scale_b,
                        int64_t M, int64_t N, int64_t K, const void* bias, fp8rt_dtype bias_t, int64_t ldy,
                        uint32_t flags, GemmArgs& g) {
  if (!a || !b || !scale_a || !scale_b) return FP8RT_EINVAL;
  if (!valid_fmt(fa) || !valid_fmt(fb) || (bias && !valid_dtype(bias_t))) return FP8RT_EINVAL;
  if ((flags & ~(FP8RT_POW2_SCALES | FP8RT_B_PACKED16 | FP8RT_EXACT_PRODUCTS)) != 0) return FP8RT_EINVAL;
  const bool packed = (flags & FP8RT_B_PACKED16) != 0;
  if (packed) ldb = K;  // ignored: the packed image has no leading dimension
  if (M <= 0 || N <= 0 || K <= 0 || lda < K || ldb < K || ldy < N) return FP8RT_EINVAL;
  if (M > (int64_t(1) << 31) || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (ga.rows < 0 || ga.cols < 0 || gb.rows < 0 || gb.cols < 0) return FP8RT_EINVAL;
  if (K % 16 != 0 || lda % 16 != 0 || ldb % 16 != 0) return FP8RT_EALIGN;
  if (!aligned16(a) || !aligned16(b) || !aligned4(scale_a) || !aligned4(scale_b)) return FP8RT_EALIGN;
  if (bias && !aligned4(bias)) return FP8RT_EALIGN;
  if (!((fa == FP8RT_E4M3 && fb == FP8RT_E4M3) || (fa == FP8RT_E5M2 && fb == FP8RT_E4M3)))
    return FP8RT_EUNSUPPORTED;
  g.a = a;
  g.fa = fa;
  g.lda = lda;
  g.era = group_extent(M, ga.rows);
  g.eca = group_extent(K, ga.cols);
  g.sa = scale_a;
  g.b = b;
  g.fb = fb;
  g.ldb = ldb;
  g.erb = group_extent(N, gb.rows);
  g.ecb = group_extent(K, gb.cols);
  g.sb = scale_b;
  g.M = M;
  g.N = N;
  g.K = K;
  g.bias = bias;
  g.bias_t = bias_t;
  g.ldy = ldy;
  g.pow2_mx = false;
  // Scale granularities the kernels implement.
  const bool a_kblk = g.eca < K, b_kblk = g.ecb < K;
  if (a_kblk && g.era != 1) return FP8RT_EUNSUPPORTED;  // A: tensor, row or {1, g}
  // 1x32 blocks only when both operands are split along K into 32-wide blocks
  // (at K = 32 a {1, 32} group is the whole row: per-row scales)
  if (a_kblk && b_kblk && g.eca == 32 && g.ecb == 32 && g.era == 1 && g.erb == 1) {
    if (!(flags & FP8RT_POW2_SCALES)) return FP8RT_EUNSUPPORTED;
    g.pow2_mx = true;
  } else {
    if (a_kblk && g.eca % 128 != 0) return FP8RT_EUNSUPPORTED;
    if (b_kblk && g.ecb % 128 != 0) return FP8RT_EUNSUPPORTED;
    if (a_kblk && b_kblk && g.eca != g.ecb) return FP8RT_EUNSUPPORTED;
  }
  // the packed weight image is read by the decode kernel only
  g.b_packed = packed;
  const bool decode = gemm_skinny_eligible(g);
  if (packed && !decode) return FP8RT_EUNSUPPORTED;
  // exact products: asked for, or free where the decode kernel is latency bound
  const bool exact = (flags & FP8RT_EXACT_PRODUCTS) != 0;
  if (exact && (!decode || g.pow2_mx)) return FP8RT_EUNSUPPORTED;
  g.exact_products = decode && !g.pow2_mx && (exact || N * K <= int64_t(FP8RT_EXACT_AUTO_BYTES));
  return FP8RT_OK;
}

}  // namespace

fp8rt_status fp8_scaled_gemm(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                             const float* scale_a, const uint8_t* b, fp8rt_format fb,
                             int64_t ldb, fp8rt_gran gb, const float* scale_b, int64_t M,
                             int64_t N, int64_t K, const void* bias, fp8rt_dtype bias_t,
                             void* y, fp8rt_dtype yt, int64_t ldy, uint32_t flags,
                             hipStream_t stream) {
  if (!y || !valid_dtype(yt)) return FP8RT_EINVAL;
  GemmArgs g{};
  const fp8rt_status st =
      gemm_setup(a, fa, lda, ga, scale_a, b, fb, ldb, gb, scale_b, M, N, K, bias, bias_t, ldy, flags, g);
  if (st != FP8RT_OK) return st;
  if ((yt == FP8RT_F32 && !aligned4(y)) || (yt == FP8RT_BF16 && (reinterpret_cast<uintptr_t>(y) & 1u)))
    return FP8RT_EALIGN;
  g.y = y;
  g.yt = yt;
  return from_hip(launch_gemm(g, stream));
}

fp8rt_status fp8_scaled_gemm_noalloc(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                                     const float* scale_a, const uint8_t* b, fp8rt_format fb,
                                     int64_t ldb, fp8rt_gran gb, const float* scale_b, int64_t M,
                                     int64_t N, int64_t K, const void* bias, fp8rt_dtype bias_t,
                                     void* y, fp8rt_dtype yt, int64_t ldy, uint32_t flags,
                                     hipStream_t stream) {
  if (!y || !valid_dtype(yt)) return FP8RT_EINVAL;
  GemmArgs g{};
  const fp8rt_status st =
      gemm_setup(a, fa, lda, ga, scale_a, b, fb, ldb, gb, scale_b, M, N, K, bias, bias_t, ldy, flags, g);
  if (st != FP8RT_OK) return st;
  if ((yt == FP8RT_F32 && !aligned4(y)) || (yt == FP8RT_BF16 && (reinterpret_cast<uintptr_t>(y) & 1u)))
    return FP8RT_EALIGN;
  g.y = y;
  g.yt = yt;
  if (gemm_required_scratch(g) > kNoAllocScratchBytes) return FP8RT_ESCRATCH;
  void* p = nullptr;
  if (noalloc_scratch(&p) != hipSuccess) return FP8RT_EHIP;
  g.fixed_scratch = p;
  g.fixed_scratch_bytes = kNoAllocScratchBytes;
  return from_hip(launch_gemm(g, stream));
}

fp8rt_status fp8_scaled_gemm_fp8out(const uint8_t* a, fp8rt_format fa, int64_t lda, fp8rt_gran ga,
                                    const float* scale_a, const uint8_t* b, fp8rt_format fb, int64_t ldb,
                                    fp8rt_gran gb, const float* scale_b, int64_t M, int64_t N, int64_t K,
                                    const void* bias, fp8rt_dtype bias_t, fp8rt_format fy,
                                    const float* scale_y, const float* inv_scale_y, uint8_t* yq,
                                    int64_t ldy, float* amax_y, uint64_t* sat_underflow, uint32_t flags,
                                    hipStream_t stream) {
  if (!yq || !scale_y || !valid_fmt(fy)) return FP8RT_EINVAL;
  if (flags & FP8RT_EXACT_PRODUCTS) return FP8RT_EUNSUPPORTED;
  GemmArgs g{};
  const fp8rt_status st =
      gemm_setup(a, fa, lda, ga, scale_a, b, fb, ldb, gb, scale_b, M, N, K, bias, bias_t, ldy, flags, g);
  if (st != FP8RT_OK) return st;
  g.exact_products = false;  // the FP8 matrix cores form the products here
  // the weight image: the decode kernel, one statistics partial per workgroup
  if (g.b_packed && skinny_blocks(g) > kMaxBlocks) return FP8RT_EUNSUPPORTED;
  if (!aligned4(scale_y) || (inv_scale_y && !aligned4(inv_scale_y)) || (amax_y && !aligned4(amax_y)) ||
      (sat_underflow && (reinterpret_cast<uintptr_t>(sat_underflow) & 7u)))
    return FP8RT_EALIGN;
  // one per-block partial per 128 x 128 output tile at most
  if (ceil_div(M, 128) * ceil_div(N, 128) > kMaxBlocks) return FP8RT_EUNSUPPORTED;
  DevWorkspace* ws = nullptr;
  if (get_workspace(stream, &ws) != hipSuccess) return FP8RT_EHIP;
  g.y = yq;
  g.yt = FP8RT_F32;  // unused with yq_fmt set
  g.yq_fmt = fy;
  g.sy = scale_y;
  g.ry = inv_scale_y;
  g.amax_y = amax_y;
  g.counts_y = reinterpret_cast<unsigned long long*>(sat_underflow);
  g.part = ws->pass2;
  return from_hip(launch_gemm(g, stream));
}

fp8rt_status fp8_weight_only_gemm(const void* x, fp8rt_dtype xt, int64_t ldx, const uint8_t* w, fp8rt_format fw,
                                  int64_t ldw, fp8rt_gran gw, const float* scale_w, int64_t M, int64_t N,
                                  int64_t K, const void* bias, fp8rt_dtype bias_t, void* y, fp8rt_dtype yt,
                                  int64_t ldy, uint32_t flags, hipStream_t stream) {
  if (!x || !w || !scale_w || !y) return FP8RT_EINVAL;
  if (!valid_dtype(xt) || !valid_fmt(fw) || !valid_dtype(yt) || (bias && !valid_dtype(bias_t)))
    return FP8RT_EINVAL;
  if ((flags & ~FP8RT_B_PACKED16) != 0) return FP8RT_EINVAL;
  const bool packed = (flags & FP8RT_B_PACKED16) != 0;
  if (packed) ldw = K;  // ignored: the packed image has no leading dimension
  if (M <= 0 || N <= 0 || K <= 0 || ldx < K || ldw < K || ldy < N || gw.rows < 0 || gw.cols < 0)
    return FP8RT_EINVAL;
  if (M > int64_t(16) * 65535 || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (xt != FP8RT_BF16) return FP8RT_EUNSUPPORTED;  // activations stay BF16
  if (K % 16 != 0 || ldx % 8 != 0 || ldw % 16 != 0 || (packed && K % 128 != 0)) return FP8RT_EALIGN;
  if (!aligned16(x) || !aligned16(w) || !aligned4(scale_w) || (bias && !aligned4(bias))) return FP8RT_EALIGN;
  if ((yt == FP8RT_F32 && !aligned4(y)) || (yt == FP8RT_BF16 && (reinterpret_cast<uintptr_t>(y) & 1u)))
    return FP8RT_EALIGN;
  WonlyArgs g;
  g.erw = group_extent(N, gw.rows);
  g.ecw = group_extent(K, gw.cols);
  if (g.ecw < K && g.ecw % 128 != 0) return FP8RT_EUNSUPPORTED;  // K groups: whole 128-deep steps
  if (ceil_div(N, g.erw) * ceil_div(K, g.ecw) >= (int64_t(1) << 31)) return FP8RT_EUNSUPPORTED;
  g.x = static_cast<const uint16_t*>(x);
  g.ldx = ldx;
  g.w = w;
  g.fw = fw;
  g.ldw = ldw;
  g.sw = scale_w;
  g.M = M;
  g.N = N;
  g.K = K;
  g.bias = bias;
  g.bias_t = bias_t;
  g.y = y;
  g.yt = yt;
  g.ldy = ldy;
  g.w_packed = packed;
  return from_hip(launch_gemm_wonly(g, stream));
}

fp8rt_status fp8_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp,
                                hipStream_t stream) {
  if (!q || !qp || N <= 0 || K <= 0 || ldq < K) return FP8RT_EINVAL;
  if (N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (K % 128 != 0 || ldq % 16 != 0 || !aligned16(q) || !aligned16(qp)) return FP8RT_EALIGN;
  return from_hip(launch_pack_weights16(q, N, K, ldq, qp, stream));
}

namespace {

// Validation shared by the two ledger entry points; fills g (q / scale /
// stats excepted).
fp8rt_status quant_error_setup(const void* w, fp8rt_dtype wt, int64_t N, int64_t K, int64_t ldw, const void* x,
                               int64_t M, int64_t ldx, fp8rt_format f, QuantErrorArgs& g) {
  if (!w || !valid_dtype(wt) || !valid_fmt(f)) return FP8RT_EINVAL;
  if (N <= 0 || K <= 0 || ldw < K || N > (int64_t(1) << 31) || K > (int64_t(1) << 31)) return FP8RT_EINVAL;
  if (x && (M <= 0 || ldx < K)) return FP8RT_EINVAL;
  if (K % 16 != 0 || ldw % 8 != 0 || (x && ldx % 8 != 0)) return FP8RT_EALIGN;
  if (!aligned16(w) || (x && !aligned16(x))) return FP8RT_EALIGN;
  g.w = w;
  g.wt = wt;
  g.ldw = ldw;
  g.f = f;
  g.N = N;
  g.K = K;
  g.x = static_cast<const uint16_t*>(x);
  g.M = x ? M : 0;
  g.ldx = ldx;
  return FP8RT_OK;
}

}  // namespace

fp8rt_status fp8_quant_error(const void* w, fp8rt_dtype wt, int64_t N, int64_t K, int64_t ldw, const uint8_t* q,
                             fp8rt_format f, int64_t ldq, fp8rt_gran g, const float* scale, const void* x,
                             int64_t M, int64_t ldx, double* stats, hipStream_t stream) {
  QuantErrorArgs a;
  fp8rt_status st = quant_error_setup(w, wt, N, K, ldw, x, M, ldx, f, a);
  if (st != FP8RT_OK) return st;
  if (!q || !scale || !stats || ldq < K || g.rows < 0 || g.cols < 0) return FP8RT_EINVAL;
  if (ldq % 8 != 0 || (reinterpret_cast<uintptr_t>(q) & 7u) || !aligned4(scale) ||
      (reinterpret_cast<uintptr_t>(stats) & 7u))
    return FP8RT_EALIGN;
  a.q = q;
  a.ldq = ldq;
  a.scale = scale;
  a.er = group_extent(N, g.rows);
  a.ec = group_extent(K, g.cols);
  if (a.ec < K && a.ec % 8 != 0) return FP8RT_EUNSUPPORTED;  // a lane's 8 elements share one scale
  a.stats = stats;
  void* part = nullptr;
  if (get_scratch(stream, quant_error_partials_bytes(N), &part) != hipSuccess) return FP8RT_EHIP;
  return from_hip(launch_quant_error(a, part, stream));
}

fp8rt_status fp8_granularity_ledger(const void* w, fp8rt_dtype wt, int64_t N, int64_t K, int64_t ldw,
                                    const void* x, int64_t M, int64_t ldx, fp8rt_format f, float eps,
                                    const fp8rt_ledger_spec* specs, int32_t n_specs, fp8rt_ledger_row* rows,
                                    hipStream_t stream) {
  QuantErrorArgs a;
  fp8rt_status st = quant_error_setup(w, wt, N, K, ldw, x, M, ldx, f, a);
  if (st != FP8RT_OK) return st;
  if (!specs || !rows || n_specs < 1 || n_specs > 64 || !valid_eps(eps)) return FP8RT_EINVAL;
  // one scratch buffer: codes [N x K], the largest scale array, 7 stats, 2 counters, partials
  int64_t max_scales = 1;
  for (int i = 0; i < n_specs; ++i) {
    if (specs[i].gran.rows < 0 || specs[i].gran.cols < 0) return FP8RT_EINVAL;
    max_scales = std::max(max_scales, ceil_div(N, group_extent(N, specs[i].gran.rows)) *
                                          ceil_div(K, group_extent(K, specs[i].gran.cols)));
  }
  auto up = [](int64_t b) { return (b + 255) / 256 * 256; };
  const int64_t off_s = up(N * K), off_st = off_s + up(max_scales * 4), off_c = off_st + 256,
                off_p = off_c + 256;
  void* scr = nullptr;
  if (get_scratch(stream, static_cast<size_t>(off_p) + quant_error_partials_bytes(N), &scr) != hipSuccess)
    return FP8RT_EHIP;
  uint8_t* base = static_cast<uint8_t*>(scr);
  uint8_t* codes = base;
  float* scales = reinterpret_cast<float*>(base + off_s);
  double* stats = reinterpret_cast<double*>(base + off_st);
  uint64_t* counts = reinterpret_cast<uint64_t*>(base + off_c);
  for (int i = 0; i < n_specs; ++i) {
    const fp8rt_gran gr = specs[i].gran;
    st = fp8_quantize(w, wt, N, K, ldw, gr, f, FP8RT_DYNAMIC, eps, specs[i].pow2_round_up, scales, nullptr,
                      codes, K, nullptr, counts, stream);
    if (st != FP8RT_OK) return st;
    a.q = codes;
    a.ldq = K;
    a.scale = scales;
    a.er = group_extent(N, gr.rows);
    a.ec = group_extent(K, gr.cols);
    a.stats = stats;
    if (launch_quant_error(a, base + off_p, stream) != hipSuccess) return FP8RT_EHIP;
    double hs[7];
    uint64_t hc[2];
    if (hipMemcpyAsync(hs, stats, sizeof(hs), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(hc, counts, sizeof(hc), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
      return FP8RT_EHIP;
    fp8rt_ledger_row& r = rows[i];
    r.gran = gr;
    r.pow2_round_up = specs[i].pow2_round_up;
    r.qparam_count = ceil_div(N, a.er) * ceil_div(K, a.ec);
    r.qparam_bytes = r.qparam_count * static_cast<int64_t>(sizeof(float));
    r.quantized_weight_bytes = N * K;
    r.total_state_bytes = r.quantized_weight_bytes + r.qparam_bytes;
    r.weight_mse = hs[0] / static_cast<double>(N * K);
    r.weight_max_abs_err = hs[2];
    const double nan = std::numeric_limits<double>::quiet_NaN();
    r.output_mse = x ? hs[3] / (static_cast<double>(M) * static_cast<double>(N)) : nan;
    r.output_cosine = x ? hs[6] / std::max(std::sqrt(hs[4]) * std::sqrt(hs[5]), 1e-8) : nan;
    r.saturated = hc[0];
    r.underflowed = hc[1];
  }
  return FP8RT_OK;
}

}  // extern "C"
