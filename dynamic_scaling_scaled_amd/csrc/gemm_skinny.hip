// gemm_skinny.hip -- scaled FP8 GEMM for a few rows of A (decode-shaped
// layers, M <= 64): streaming B at HBM speed is the whole job.
//
// Method: "FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM" (Y ~ s_x s_w X8 W8, FP32 accumulation,
// BF16/FP32 output, bias) and section "Per-channel and block scaling"
// (per-token and per-output-channel scales, and scales per block):
//   Y[m,n] = sum_g s_a(m,g) s_b(n,g) sum_{k in g} dec(A[m,k]) dec(B[n,k]) + bias[n]
// with g over the 128-deep K steps (one group of each operand per step).
//
// Design for MI355X: with M <= 64 the arithmetic intensity is at most 2M
// FLOP per byte of B, far below the MFMA ridge, so the kernel is built
// around keeping enough of B in flight: many small waves instead of deep
// per-wave prefetch.
//  - One workgroup of 16 waves owns 16 rows of B; wave w takes the w-th
//    sixteenth of the 128-deep K steps and runs a plain load -> MFMA loop
//    (global loads straight into the MFMA operand layout, no LDS staging: B
//    is read exactly once, nontemporally).  Two workgroups per CU (64
//    VGPRs per lane, where the variant fits) keep 32 waves' loads in flight,
//    which hides the HBM latency.
//  - v_mfma_f32_16x16x128 with B as the first operand: the 16 x 16 result
//    holds 16 rows of B (output columns) by 16 rows of A (one MFMA per 16-row
//    tile of A, up to 4 per workgroup; with fewer 16-row groups of B than
//    CUs each tile of A gets a workgroup of its own); each lane ends with 4
//    consecutive output columns of one output row per tile.  Lane quarter g loads
//    bytes [32 g, 32 g + 32) of every 128-byte K step of both operands, the
//    same K permutation on both sides, which the per-row scales (applied
//    after the sum) do not see.
//  - The 16 partial sums meet in LDS; wave 0 applies the scales and the bias,
//    rounds and stores 8- or 16-byte pieces, or (FP8 output) casts y * r_y as
//    the quantize kernels do and writes the workgroup's max |y| and
//    saturation / underflow counts for the finisher.
//  - Scales that change along K (1 x g token groups, g_r x g weight blocks,
//    g a multiple of 128): each step's MFMAs start from zero and the partial
//    is added to the accumulator times s_a(m, step) s_b(n, step) (one FMA
//    per element; the step's scales are cached loads), so the epilogue only
//    adds the bias.  The stream of B is the same, so such decode GEMMs cost
//    what per-channel ones do.
//  - 1 x 32 power-of-two scales ("Per-channel and block scaling", with
//    the scales' exponents as E8M0): v_mfma_scale_f32_16x16x128_f8f6f4 takes
//    one exponent per lane and operand, its row's scale for the 32-deep K
//    block of its lane quarter; the lanes then load bytes [16 g, +16) and
//    [64 + 16 g, +16) of each step, the matrix core's own K order, so those
//    blocks are the memory's.  Row-major B only.
//  - Exact products (a template flag): each 128-deep step becomes four
//    v_mfma_f32_16x16x32_bf16, instruction j taking bytes [8 j, 8 j + 8) of
//    every lane's 32 on both operands, widened exactly to bf16 in registers
//    (v_cvt_scalef32_pk_bf16_fp8 / _bf8 with scale 1: two codes each).  The
//    bf16 matrix cores multiply exactly, so only the FP32 accumulation
//    rounds, where the FP8 ones align each 8-deep run's products to the
//    largest and drop the bits below 2^-13 of it.  Four times the matrix-core
//    instructions and one VALU op per two codes: free where the launch is
//    latency bound.
//  - Fragment-ordered B (fp8_pack_weights16): each 16-row x 128-byte step of
//    B is one 2 KB tile whose first KB holds every lane's first 16 bytes in
//    lane order and whose second KB their last 16 bytes, so each load
//    instruction reads 1 KB contiguous instead of 64 bytes of 16 rows (a
//    timing copy with contiguous loads ran 22% faster).  The MFMA receives
//    the same bytes as from row-major B: the results are identical.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Exact products: every E4M3 / E5M2 value is a bf16 value, and the bf16
// matrix cores multiply bf16 exactly into FP32.  One conversion turns two
// codes of a dword half into two bf16 (element order kept; the conversion's
// scale operand is 1.0, so nothing is rounded); 8 codes -> 8 bf16.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int F, bool HI>
__device__ __forceinline__ uint32_t widen2(int w) {
  bf16x2 h;
  if constexpr (F == kE4M3) {
    h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI);
  } else {
    h = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w, 1.0f, HI);
  }
  return __builtin_bit_cast(uint32_t, h);
}
template <int F>
__device__ __forceinline__ bf16x8 widen8(int w0, int w1) {
  return __builtin_bit_cast(bf16x8, u32x4{widen2<F, false>(w0), widen2<F, true>(w0), widen2<F, false>(w1),
                                          widen2<F, true>(w1)});
}

constexpr int kSkWaves = 16;
constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkMaxM = 64;  // up to 4 MFMA row tiles of A

// Waves per SIMD the register budget is sized for: 8 (two workgroups per CU,
// 64 VGPRs) for one or two row tiles of A, or one with exact products; 4 (one
// workgroup, 128 VGPRs) for four row tiles, whose A fragments alone fill 64
// VGPRs, and for two with exact products (their widened operands) or with
// scales read per step (sm 1 or 2).
constexpr int sk_waves_per_simd(int mt, bool exact, int sm) {
  return (mt >= 4 || (mt >= 2 && (exact || sm != 0)) || (exact && sm == 1)) ? 4 : 8;
}

// SM, where the scales apply: 0 in the epilogue (per tensor or per row, whole
// K); 1 per 128-deep step (1 x g groups on A, g_r x g blocks on B, g a
// multiple of 128, or row groups that are neither one row nor all rows):
// the step's partial comes out of MFMAs started from zero and is added to
// the accumulator times s_a(m, step) s_b(n, step); 2 inside the MFMA (1 x 32
// power-of-two scales passed as E8M0 exponents, one per lane: its row and
// its 32-deep K block).  With 1 or 2 the epilogue adds only the bias.
// OUT: kOutF32 / kOutBF16, or FP8 codes (kOutE4M3 / kOutE5M2) of y * r_y,
// r_y = ry[0] or fl32(1 / sy[0]), with the workgroup's max |y| and
// saturation / underflow counts in ypart[workgroup] (combined by k_finish).
template <int FA, int FB, int MT, int OUT, bool PACKED, bool EXACT, int SM>
__global__ __launch_bounds__(kSkThreads, sk_waves_per_simd(MT, EXACT, SM)) void k_gemm_skinny(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sa, int64_t era, int64_t eca, const float* __restrict__ sb,
    int64_t erb, int64_t ecb, const void* __restrict__ bias, int bias_bf16, void* __restrict__ Y, int64_t ldy,
    int vec_store, const float* __restrict__ sy, const float* __restrict__ ry, BlockPartial* __restrict__ ypart) {
  constexpr bool KB = SM == 1, MX = SM == 2;
  __shared__ f32x4 red[kSkWaves - 1][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const int64_t mb = static_cast<int64_t>(blockIdx.y) * (16 * MT);  // first row of A
  // row-major: row n0 + r, bytes [32 g, +32) of each step, or (MX) bytes
  // [16 g, +16) and [64 + 16 g, +16): the matrix core's own K order, so its
  // 32-deep scale blocks are the memory's; packed: the lane's 16-byte slots
  // of its group's 2 KB tiles
  constexpr int kLane = MX ? 16 : 32;
  const uint8_t* brow = PACKED ? B + static_cast<int64_t>(blockIdx.x) * (K / 128) * 2048 + lane * 16
                               : B + min(n0 + r, N - 1) * ldb + kLane * g;
  const int64_t bstep = PACKED ? 2048 : 128, bhalf = PACKED ? 1024 : (MX ? 64 : 16);
  constexpr int ahalf = MX ? 64 : 16;
  const uint8_t* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = A + min<int64_t>(mb + 16 * t + r, M - 1) * lda + kLane * g;
  // MX: the lane's scale rows (one float per 32 K)
  const float* sbx = MX ? sb + min(n0 + r, N - 1) * (K / 32) + g : nullptr;
  const float* sax[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) sax[t] = MX ? sa + min<int64_t>(mb + 16 * t + r, M - 1) * (K / 32) + g : nullptr;

  // this wave's K steps: [s0, s1)
  const int nk = static_cast<int>(K / 128);
  const int s0 = (nk * wave) / kSkWaves, s1 = (nk * (wave + 1)) / kSkWaves;
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // KB: offsets of the scale rows of the lane's output row (per row tile)
  // and of its 4 output columns n0 + 4 g + e
  int64_t aoff[KB ? MT : 1], boff[KB ? 4 : 1];
  int spa = 1, spb = 1;  // 128-deep steps per scale group along K
  if constexpr (KB) {
    const int64_t nga = (K + eca - 1) / eca, ngb = (K + ecb - 1) / ecb;
    spa = static_cast<int>(min(eca, K) / 128);
    spb = static_cast<int>(min(ecb, K) / 128);
#pragma unroll
    for (int t = 0; t < MT; ++t) aoff[t] = (min<int64_t>(mb + 16 * t + r, M - 1) / era) * nga;
#pragma unroll
    for (int e = 0; e < 4; ++e) boff[e] = (min<int64_t>(n0 + 4 * g + e, N - 1) / erb) * ngb;
  }
  // Two steps per iteration (loads of both first, then both MFMAs): twice
  // the bytes in flight per wave.  An odd last step loads step s1 - 1 again
  // (a cache hit), runs its MFMAs and keeps the accumulator as it was (a
  // select, not a branch: loads used only under a branch are sunk into it,
  // after the first step's MFMAs, which leaves one step in flight).
  auto mma = [&](const u32x4& b0, const u32x4& b1, const u32x4 (&a0)[MT], const u32x4 (&a1)[MT], bool on,
                 int step) {
    i32x8 bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
    // the step's scale factors (KB); a skipped tail step adds exactly zero
    float fb[4] = {1.f, 1.f, 1.f, 1.f};
    int ka = 0;
    if constexpr (KB) {
      ka = step / spa;
      const int kb = step / spb;
#pragma unroll
      for (int e = 0; e < 4; ++e) fb[e] = sb[boff[e] + kb];
    }
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      f32x4 c = KB ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[t];
      i32x8 af = i32x8{(int)a0[t][0], (int)a0[t][1], (int)a0[t][2], (int)a0[t][3],
                       (int)a1[t][0], (int)a1[t][1], (int)a1[t][2], (int)a1[t][3]};
      if constexpr (EXACT) {
        // the step's 128 K as 4 bf16 MFMAs of 32: instruction j takes codes
        // [8 j, +8) of every lane's 32 on both operands (the same K set in
        // the same order, a permutation of the step that the per-row scales
        // do not see); products exact, FP32 accumulation
#pragma unroll
        for (int j = 0; j < 4; ++j)
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(widen8<FB>(bf[2 * j], bf[2 * j + 1]),
                                                      widen8<FA>(af[2 * j], af[2 * j + 1]), c, 0, 0, 0);
      } else if constexpr (MX) {
        // E8M0 exponents of the power-of-two scales of the lane's rows and K block
        const int xb = static_cast<int>((__float_as_uint(sbx[step * 4]) >> 23) & 0xFFu);
        const int xa = static_cast<int>((__float_as_uint(sax[t][step * 4]) >> 23) & 0xFFu);
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, c, FB, FA, 0, xb, 0, xa);
      } else {
        c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, c, FB, FA, 0, 0, 0, 0);
      }
      if constexpr (KB) {
        const float fa = sa[aoff[t] + ka];
#pragma unroll
        for (int e = 0; e < 4; ++e) c[e] = fmaf(fa * fb[e], c[e], acc[t][e]);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = on ? c[e] : acc[t][e];
    }
  };
  for (int st = s0; st < s1; st += 2) {
    const int st2 = min(st + 1, s1 - 1);
    const int64_t ko = static_cast<int64_t>(st) * 128, ko2 = static_cast<int64_t>(st2) * 128;
    const int64_t bo = static_cast<int64_t>(st) * bstep, bo2 = static_cast<int64_t>(st2) * bstep;
    const u32x4 b0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo));
    const u32x4 b1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo + bhalf));
    const u32x4 c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo2));
    const u32x4 c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo2 + bhalf));
    u32x4 a0[MT], a1[MT], d0[MT], d1[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      a0[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko);
      a1[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko + ahalf);
      d0[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko2);
      d1[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko2 + ahalf);
    }
    mma(b0, b1, a0, a1, true, st);
    mma(c0, c1, d0, d1, st + 1 < s1, st2);
  }

  // The partial sums meet in LDS; wave 0 finishes.
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll 5  // 15 partials: three batches of 5 reads in flight
    for (int w = 0; w < kSkWaves - 1; ++w) acc[t] += red[w][t][lane];

  // lane: output row m = mb + 16 t + r, columns n0 + 4 g + (0..3)
  const int64_t nb = n0 + 4 * g;
  float sbv[4], bv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t n = min(nb + e, N - 1);
    sbv[e] = SM != 0 ? 1.0f : sb[erb == 1 ? n : 0];
    bv[e] = 0.0f;
    if (bias)
      bv[e] = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[n]) << 16)
                        : static_cast<const float*>(bias)[n];
  }
  float rq = 1.0f;
  uint32_t ymax = 0, sat_l = 0, under_l = 0;  // FP8 output: this lane's statistics
  if constexpr (OUT >= kOutE4M3) rq = ry ? ry[0] : 1.0f / sy[0];
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = mb + 16 * t + r;
    if (m >= M) continue;
    const float sav = SM != 0 ? 1.0f : sa[era == 1 ? m : 0];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[t][e] * (sav * sbv[e]) + bv[e];
    if constexpr (OUT >= kOutE4M3) {
      // the GIVEN-mode cast of the quantize kernels on y * r_y; statistics of
      // stored elements only (columns past N are clamped repeats)
      constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = v[e] * rq;
        const uint32_t ab = nb + e < N ? (__float_as_uint(v[e]) & kAbsMask) : 0u;  // 0: not counted
        ymax = max(ymax, ab);
        sat_l += (ab != 0u && fabsf(f[e]) > Fmt<F>::kMax) ? 1u : 0u;
        under_l += (ab != 0u && fabsf(f[e]) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
      }
      uint32_t w = cvt4<F>(f[0], f[1], f[2], f[3]);
      if (__builtin_isunordered(f[0], f[1]) || __builtin_isunordered(f[2], f[3])) w = cvt4_nan<F>(f[0], f[1], f[2], f[3]);
      uint8_t* dst = static_cast<uint8_t*>(Y) + m * ldy + nb;
      if (vec_store && nb + 4 <= N) {
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        for (int e = 0; e < 4 && nb + e < N; ++e) dst[e] = static_cast<uint8_t>(w >> (8 * e));
      }
    } else if constexpr (OUT == kOutBF16) {
      uint16_t* dst = static_cast<uint16_t*>(Y) + m * ldy + nb;
      const bf16x4 h = __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4);
      if (vec_store && nb + 4 <= N) {
        *reinterpret_cast<bf16x4*>(dst) = h;
      } else {
        const u32x2 hb = __builtin_bit_cast(u32x2, h);  // 4 bf16 as 2 words
        for (int e = 0; e < 4 && nb + e < N; ++e) dst[e] = static_cast<uint16_t>(hb[e >> 1] >> (16 * (e & 1)));
      }
    } else {
      float* dst = static_cast<float*>(Y) + m * ldy + nb;
      if (vec_store && nb + 4 <= N) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        for (int e = 0; e < 4 && nb + e < N; ++e) dst[e] = v[e];
      }
    }
  }
  if constexpr (OUT >= kOutE4M3) {
    ymax = wave_max_u32(ymax);
    const uint32_t s_w = static_cast<uint32_t>(wave_sum_u64(sat_l));
    const uint32_t u_w = static_cast<uint32_t>(wave_sum_u64(under_l));
    if (lane == 0)
      *reinterpret_cast<u32x4*>(&ypart[static_cast<int64_t>(blockIdx.y) * gridDim.x + blockIdx.x]) =
          u32x4{ymax, s_w, u_w, 0u};
  }
}

// Scales the epilogue applies: per tensor or per row on both sides, whole K.
bool skinny_epilogue_scales(const GemmArgs& g) {
  return (g.era == 1 || g.era >= g.M) && (g.erb == 1 || g.erb >= g.N) && g.eca >= g.K && g.ecb >= g.K;
}

template <int FA, int FB, int MT, bool PACKED, bool EXACT, int SM>
void launch_mt_k(const GemmArgs& g, hipStream_t st, int vec) {
  const dim3 grid(static_cast<unsigned>((g.N + 15) / 16), static_cast<unsigned>((g.M + 16 * MT - 1) / (16 * MT)));
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
#define FP8RT_SK(OUT)                                                                                            \
  hipLaunchKernelGGL((k_gemm_skinny<FA, FB, MT, OUT, PACKED, EXACT, SM>), grid, dim3(kSkThreads), 0, st, g.a,   \
                     g.lda, g.b, g.ldb, g.M, g.N, g.K, g.sa, g.era, g.eca, g.sb, g.erb, g.ecb, g.bias, bb, g.y, \
                     g.ldy, vec, g.sy, g.ry, g.part)
  switch (gemm_out_kind(g)) {
    case kOutBF16: FP8RT_SK(kOutBF16); break;
    case kOutF32: FP8RT_SK(kOutF32); break;
    default:
      // FP8 output: FP8 matrix cores only
      if constexpr (!EXACT) {
        if (gemm_out_kind(g) == kOutE4M3) FP8RT_SK(kOutE4M3);
        else FP8RT_SK(kOutE5M2);
      }
      break;
  }
#undef FP8RT_SK
}

template <int FA, int FB, int MT, bool PACKED, bool EXACT>
void launch_mt_e(const GemmArgs& g, hipStream_t st, int vec) {
  if (g.pow2_mx) {
    // 1 x 32 scales: FP8 matrix cores on a row-major B (the eligibility test)
    if constexpr (!PACKED && !EXACT) launch_mt_k<FA, FB, MT, PACKED, EXACT, 2>(g, st, vec);
  } else if (skinny_epilogue_scales(g)) {
    launch_mt_k<FA, FB, MT, PACKED, EXACT, 0>(g, st, vec);
  } else {
    if constexpr (!(MT == 4 && EXACT)) launch_mt_k<FA, FB, MT, PACKED, EXACT, 1>(g, st, vec);  // see skinny_row_tiles
  }
}

template <int FA, int FB, int MT, bool PACKED>
void launch_mt(const GemmArgs& g, hipStream_t st, int vec) {
  if (g.exact_products) launch_mt_e<FA, FB, MT, PACKED, true>(g, st, vec);
  else launch_mt_e<FA, FB, MT, PACKED, false>(g, st, vec);
}

// Row tiles of A per workgroup.  All of M in one workgroup reads B once,
// which is what counts when the 16-row groups of B alone give every CU a
// workgroup; with fewer groups of B each 16-row tile of A gets a workgroup of
// its own (B re-read per tile, mostly from L2): up to four times the CUs and
// a quarter of the matrix-core work per SIMD (64 x 2048 x 2048: 18.1 -> 14.2
// us per call; 64 x 4096 x 4096, 256 groups: 21.2 with one workgroup per
// group, 23.2 split).
int skinny_row_tiles(const GemmArgs& g) {
  if ((g.N + 15) / 16 < static_cast<int64_t>(device_cus())) return 1;
  const int mt = g.M <= 16 ? 1 : g.M <= 32 ? 2 : 4;
  // four tiles with exact products and per-step scales exceed 128 VGPRs
  return (mt == 4 && g.exact_products && !g.pow2_mx && !skinny_epilogue_scales(g)) ? 2 : mt;
}

template <int FA, int FB, bool PACKED>
void launch_rows(const GemmArgs& g, hipStream_t st, int vec) {
  const int mt = skinny_row_tiles(g);
  if (mt == 1) launch_mt<FA, FB, 1, PACKED>(g, st, vec);
  else if (mt == 2) launch_mt<FA, FB, 2, PACKED>(g, st, vec);
  else launch_mt<FA, FB, 4, PACKED>(g, st, vec);
}

template <int FA, int FB>
void launch_fmt(const GemmArgs& g, hipStream_t st, int vec) {
  if (g.b_packed) launch_rows<FA, FB, true>(g, st, vec);
  else launch_rows<FA, FB, false>(g, st, vec);
}

// Fragment-ordered copy of row-major codes: 16-byte piece c of qp is tile
// c / 128 (group G, step s), half (c / 64) % 2, lane c % 64 (zeros past row
// N).  Grid-stride; consecutive threads write consecutive pieces.
__global__ __launch_bounds__(256) void k_pack_weights16(const uint8_t* __restrict__ q, int64_t N, int64_t K,
                                                        int64_t ldq, uint8_t* __restrict__ qp, int64_t nchunks) {
  const int64_t steps = K / 128;
  for (int64_t c = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; c < nchunks;
       c += static_cast<int64_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(c & 63), h = static_cast<int>((c >> 6) & 1);
    const int64_t tile = c >> 7;
    const int64_t grp = tile / steps, st = tile - grp * steps;
    const int64_t row = 16 * grp + (l & 15);
    const int64_t col = 128 * st + 32 * (l >> 4) + 16 * h;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (row < N) v = *reinterpret_cast<const u32x4*>(q + row * ldq + col);
    *reinterpret_cast<u32x4*>(qp + c * 16) = v;
  }
}

}  // namespace

bool gemm_skinny_eligible(const GemmArgs& g) {
  // whole 128-deep K steps, each inside one scale group of either operand,
  // or 1 x 32 scales (inside the MFMA) on a row-major B
  const bool k_ok = g.pow2_mx ? !g.b_packed
                              : (g.eca >= g.K || g.eca % 128 == 0) && (g.ecb >= g.K || g.ecb % 128 == 0);
  return k_ok && g.M <= kSkMaxM && g.K % 128 == 0;
}

hipError_t launch_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp,
                                 hipStream_t st) {
  const int64_t nchunks = (N + 15) / 16 * (K / 128) * 128;  // 16-byte pieces
  const int64_t nb = std::min<int64_t>((nchunks + 255) / 256, int64_t(1) << 20);
  hipLaunchKernelGGL(k_pack_weights16, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st, q, N, K, ldq, qp, nchunks);
  return hipGetLastError();
}

int64_t skinny_blocks(const GemmArgs& g) {
  const int mt = skinny_row_tiles(g);
  return (g.N + 15) / 16 * ((g.M + 16 * mt - 1) / (16 * mt));
}

hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t st) {
  const int kind = gemm_out_kind(g);
  // FP8 codes out: built for the FP8 matrix cores only
  if (kind >= kOutE4M3 && g.exact_products) return hipErrorInvalidValue;
  const int esz = kind == kOutF32 ? 4 : kind == kOutBF16 ? 2 : 1;
  const int vec = ((g.ldy * esz) % (4 * esz) == 0) && ((reinterpret_cast<uintptr_t>(g.y) & (4 * esz - 1)) == 0);
  if (g.fa == FP8RT_E4M3) launch_fmt<0, 0>(g, st, vec);
  else launch_fmt<1, 0>(g, st, vec);
  return hipGetLastError();
}

}  // namespace fp8rt
