// gemm_kernels.hip -- scaled FP8 GEMM on gfx950 matrix cores.
//
// Method ("FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM"): X ~ s_x X8, W ~ s_w W8, so
// Y ~ s_x s_w (X8 W8) with higher-precision accumulation, a BF16/FP32 output
// and bias fusion; section "Per-channel and block scaling": per-row and
// per-block scales.  "FP8 production quantization guide", GEMM listing:
// (x_fp8, w_fp8, scale_a, scale_b, out_dtype, bias).
//
//   Y[m,n] = sum_k s_a(m,k) s_b(n,k) dec(A[m,k]) dec(B[n,k]) + bias[n]
//   A [M x K] and B [N x K] codes, both K-contiguous (B is the nn.Linear
//   weight layout), Y row-major.
//
// Design: a workgroup of 4 waves owns a BM x BN = 128 x 128 output tile and
// walks K in 128-deep steps.  Each step stages A and B (16 KB each) from HBM
// through registers into a double-buffered, XOR-swizzled LDS tile; each wave
// computes a 64 x 64 sub-tile with 16 v_mfma_f32_16x16x128_f8f6f4 per step
// (operand formats selected per operand: E4M3 / E5M2).  Scales:
//   - per-tensor / per-row on both operands: applied once in the epilogue;
//   - K-blocked (block size a multiple of 128): each step's MFMA result is
//     promoted into the FP32 accumulator with s_a(m,kb) s_b(n,kb);
//   - 1x32 power-of-two scales: passed to the scaled MFMA as E8M0 exponents.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 128;
constexpr int kGemmThreads = 256;
constexpr int kTileBytes = BM * BK;  // one operand tile in LDS (bytes)

enum ScaleMode { kScaleEpilogue = 0, kScaleKBlock = 1, kScaleMX32 = 2 };

// Byte offset of 16-byte chunk c (0..7) of tile row r in the swizzled LDS tile.
__device__ __forceinline__ int lds_off(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

template <int FA, int FB, int MODE, int OUT>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ sa, int64_t era, int64_t nKa,
    int64_t eca, const float* __restrict__ sb, int64_t erb, int64_t nKb, int64_t ecb,
    const void* __restrict__ bias, int bias_bf16, void* __restrict__ Y, int64_t ldy,
    int tiles_n, const float* __restrict__ sy, const float* __restrict__ ry, BlockPartial* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];  // [buf][A|B]
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x - tile_m * tiles_n;
  const int64_t m0 = static_cast<int64_t>(tile_m) * BM, n0 = static_cast<int64_t>(tile_n) * BN;
  const int nk = static_cast<int>((K + BK - 1) / BK);

  // Global staging: 4 chunks of A and 4 of B per thread per step.
  u32x4 ra[4], rb[4];
  int st_row[4], st_c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = t + kGemmThreads * j;
    st_row[j] = idx >> 3;
    st_c[j] = idx & 7;
  }
  auto load_step = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t kc = k0 + st_c[j] * 16;
      const int64_t ar = min(m0 + st_row[j], M - 1);
      const int64_t br = min(n0 + st_row[j], N - 1);
      if (kc < K) {
        ra[j] = *reinterpret_cast<const u32x4*>(A + ar * lda + kc);
        rb[j] = *reinterpret_cast<const u32x4*>(B + br * ldb + kc);
      } else {
        ra[j] = u32x4{0u, 0u, 0u, 0u};
        rb[j] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int off = lds_off(st_row[j], st_c[j]);
      *reinterpret_cast<u32x4*>(&lds[buf][0][off]) = ra[j];
      *reinterpret_cast<u32x4*>(&lds[buf][1][off]) = rb[j];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // MFMA operand lane layout (16x16x128): lane l holds row (l % 16) of the
  // 16-row sub-tile and the K bytes [16g, 16g+16) and [64+16g, 64+16g+16)
  // with g = l / 16.  The output lane l holds column (l % 16), rows
  // 4 (l / 16) + [0, 4).
  const int fr = lane & 15, fg = lane >> 4;

  load_step(0);
  store_step(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load_step(kt + 1);

    // Per-step scales.
    float sak[4][4], sbk[4];
    int exa[4], exb[4];
    if constexpr (MODE == kScaleKBlock) {
      const int64_t ka = (static_cast<int64_t>(kt) * BK) / eca;
      const int64_t kb = (static_cast<int64_t>(kt) * BK) / ecb;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int64_t row = min(m0 + wm * 64 + i * 16 + fg * 4 + r, M - 1);
          sak[i][r] = sa[(row / era) * nKa + ka];
        }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = min(n0 + wn * 64 + j * 16 + fr, N - 1);
        sbk[j] = sb[(col / erb) * nKb + kb];
      }
    } else if constexpr (MODE == kScaleMX32) {
      const int64_t kblk = static_cast<int64_t>(kt) * (BK / 32) + fg;  // hardware block fg
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t row = min(m0 + wm * 64 + i * 16 + fr, M - 1);
        const int64_t kk = min<int64_t>(kblk, nKa - 1);
        exa[i] = (__float_as_uint(sa[row * nKa + kk]) >> 23) & 0xFF;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = min(n0 + wn * 64 + j * 16 + fr, N - 1);
        const int64_t kk = min<int64_t>(kblk, nKb - 1);
        exb[j] = (__float_as_uint(sb[col * nKb + kk]) >> 23) & 0xFF;
      }
    }

    i32x8 bf[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = wn * 64 + j * 16 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&lds[buf][1][lds_off(r, fg)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&lds[buf][1][lds_off(r, 4 + fg)]);
      bf[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = wm * 64 + i * 16 + fr;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(&lds[buf][0][lds_off(r, fg)]);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(&lds[buf][0][lds_off(r, 4 + fg)]);
      const i32x8 af = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (MODE == kScaleEpilogue) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af, bf[j], acc[i][j], FA, FB,
                                                                       0, 0, 0, 0);
        } else if constexpr (MODE == kScaleMX32) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[j], acc[i][j], FA, FB, 0, exa[i], 0, exb[j]);
        } else {
          const f32x4 p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              af, bf[j], f32x4{0.f, 0.f, 0.f, 0.f}, FA, FB, 0, 0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sak[i][r] * sbk[j], p[r], acc[i][j][r]);
        }
      }
    }

    if (kt + 1 < nk) store_step(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: scales (per-tensor / per-row modes), bias, convert, store.
  // FP8 output: code = cast(y * r_y) with the quantize kernels' saturating
  // RNE cast; max |y| and the counters go to this block's partial.
  float rq = 1.0f;
  if constexpr (OUT >= kOutE4M3) rq = ry ? ry[0] : 1.0f / sy[0];
  uint32_t mb = 0, sat_l = 0, under_l = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t col = n0 + wn * 64 + j * 16 + fr;
    if (col >= N) continue;
    float sbv = 1.0f, bv = 0.0f;
    if constexpr (MODE == kScaleEpilogue) sbv = sb[(col / erb) * nKb];
    if (bias) {
      bv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col]) << 16)
                     : static_cast<const float*>(bias)[col];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 64 + i * 16 + fg * 4 + r;
        if (row >= M) continue;
        float v = acc[i][j][r];
        if constexpr (MODE == kScaleEpilogue) v = v * (sa[(row / era) * nKa] * sbv);
        v = v + bv;
        if constexpr (OUT == kOutBF16) {
          const uint32_t u = __float_as_uint(v);
          const uint16_t h = ((u & kAbsMask) > kInfBits) ? 0x7FC0u
                                                          : static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
          static_cast<uint16_t*>(Y)[row * ldy + col] = h;
        } else if constexpr (OUT == kOutF32) {
          static_cast<float*>(Y)[row * ldy + col] = v;
        } else {
          constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
          const float f = v * rq;
          mb = max(mb, __float_as_uint(v) & kAbsMask);
          sat_l += fabsf(f) > Fmt<F>::kMax ? 1u : 0u;
          under_l += (v != 0.0f && fabsf(f) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
          static_cast<uint8_t*>(Y)[row * ldy + col] = static_cast<uint8_t>(cvt4_nan<F>(f, 0.f, 0.f, 0.f));
        }
      }
    }
  }
  if constexpr (OUT >= kOutE4M3)
    block_stats_store<kGemmThreads / 64>(reinterpret_cast<u32x4*>(&part[blockIdx.x]), mb, sat_l, under_l);
}

template <int FA, int FB, int MODE>
static void launch_mode(const GemmArgs& g, hipStream_t st, int nKa, int nKb) {
  const int tiles_m = static_cast<int>((g.M + BM - 1) / BM);
  const int tiles_n = static_cast<int>((g.N + BN - 1) / BN);
  const dim3 grid(tiles_m * tiles_n);
#define FP8RT_GEN(OUT)                                                                                   \
  hipLaunchKernelGGL((k_gemm<FA, FB, MODE, OUT>), grid, dim3(kGemmThreads), 0, st, g.a, g.lda, g.b, g.ldb, \
                     g.M, g.N, g.K, g.sa, g.era, (int64_t)nKa, g.eca, g.sb, g.erb, (int64_t)nKb, g.ecb,   \
                     g.bias, g.bias_t == FP8RT_BF16 ? 1 : 0, g.y, g.ldy, tiles_n, g.sy, g.ry, g.part)
  switch (gemm_out_kind(g)) {
    case kOutBF16: FP8RT_GEN(kOutBF16); break;
    case kOutE4M3: FP8RT_GEN(kOutE4M3); break;
    case kOutE5M2: FP8RT_GEN(kOutE5M2); break;
    default: FP8RT_GEN(kOutF32); break;
  }
#undef FP8RT_GEN
}

template <int FA, int FB>
static void launch_formats(const GemmArgs& g, hipStream_t st) {
  const int nKa = static_cast<int>((g.K + g.eca - 1) / g.eca);
  const int nKb = static_cast<int>((g.K + g.ecb - 1) / g.ecb);
  if (g.pow2_mx) launch_mode<FA, FB, kScaleMX32>(g, st, nKa, nKb);
  else if (g.eca < g.K || g.ecb < g.K) launch_mode<FA, FB, kScaleKBlock>(g, st, nKa, nKb);
  else launch_mode<FA, FB, kScaleEpilogue>(g, st, nKa, nKb);
}

static hipError_t launch_generic(const GemmArgs& g, hipStream_t st) {
  if (g.fa == FP8RT_E4M3 && g.fb == FP8RT_E4M3) launch_formats<0, 0>(g, st);
  else if (g.fa == FP8RT_E5M2 && g.fb == FP8RT_E4M3) launch_formats<1, 0>(g, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t gemm_scratch(const GemmArgs& g, hipStream_t st, size_t bytes, void** ptr) {
  if (!g.fixed_scratch) return get_scratch(st, bytes, ptr);
  if (bytes > g.fixed_scratch_bytes) return hipErrorInvalidValue;  // checked by the caller first
  *ptr = g.fixed_scratch;
  return hipSuccess;
}

size_t gemm_required_scratch(const GemmArgs& g) {
  // the same order of choice as launch_gemm (BF16 / FP32 output)
  if (gemm_skinny_eligible(g)) return 0;
  if (gemm_big_eligible(g)) return gemm_big_required_scratch(g);
  if (gemm_kblock_eligible(g)) return gemm_kblock_required_scratch(g);
  return 0;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t st) {
  if (g.yq_fmt >= 0) {
    // FP8 output: the decode kernel, the large kernel or the general one,
    // then the partials of max |y| and the counters (one per workgroup or
    // tile, or per split-K reduce block).
    int nb = 0;
    hipError_t e;
    if (gemm_skinny_eligible(g) && !g.exact_products && skinny_blocks(g) <= kMaxBlocks) {
      e = launch_gemm_skinny(g, st);
      nb = static_cast<int>(skinny_blocks(g));
    } else if (g.b_packed) {
      return hipErrorInvalidValue;  // the weight image is read by the decode kernel only
    } else if (gemm_big_eligible(g)) {
      e = launch_gemm_big(g, st, &nb);
    } else {
      e = launch_generic(g, st);
      nb = static_cast<int>(ceil_div(g.M, BM) * ceil_div(g.N, BN));
    }
    if (e != hipSuccess) return e;
    if (g.amax_y || g.counts_y) return launch_finish(g.part, nb, g.amax_y, g.counts_y, st);
    return hipSuccess;
  }
  if (gemm_skinny_eligible(g)) return launch_gemm_skinny(g, st);
  if (gemm_big_eligible(g)) return launch_gemm_big(g, st);
  if (gemm_kblock_eligible(g)) return launch_gemm_kblock(g, st);
  return launch_generic(g, st);
}

}  // namespace fp8rt
