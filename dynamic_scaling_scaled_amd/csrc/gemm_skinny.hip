// gemm_skinny.hip -- scaled FP8 GEMM for a few rows of A (decode-shaped
// layers, M <= 16): streaming B at HBM speed is the whole job.
//
// Method: "FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM" (Y ~ s_x s_w X8 W8, FP32 accumulation,
// BF16/FP32 output, bias) and section "Per-channel and block scaling"
// (per-token and per-output-channel scales):
//   Y[m,n] = s_a(m) s_b(n) sum_k dec(A[m,k]) dec(B[n,k]) + bias[n].
//
// Design for MI355X: with M <= 16 the arithmetic intensity is at most 2M
// FLOP per byte of B, far below the MFMA ridge, so the kernel is built
// around keeping enough of B in flight: many small waves instead of deep
// per-wave prefetch.
//  - One workgroup of 16 waves owns 16 rows of B; wave w takes the w-th
//    sixteenth of the 128-deep K steps and runs a plain load -> MFMA loop
//    (global loads straight into the MFMA operand layout, no LDS staging: B
//    is read exactly once, nontemporally).  Two workgroups per CU (64
//    VGPRs per lane) keep 32 waves' loads in flight, which hides the HBM
//    latency.
//  - v_mfma_f32_16x16x128 with B as the first operand: the 16 x 16 result
//    holds 16 rows of B (output columns) by 16 rows of A; each lane ends with
//    4 consecutive output columns of one output row.  Lane quarter g loads
//    bytes [32 g, 32 g + 32) of every 128-byte K step of both operands, the
//    same K permutation on both sides, which the per-row scales (applied
//    after the sum) do not see.
//  - The 16 partial sums meet in LDS; wave 0 applies the scales and the bias,
//    rounds and stores 8- or 16-byte pieces.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kSkWaves = 16;
constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkMaxM = 16;

template <int FA, int FB, int MT, bool BF16OUT>
__global__ __launch_bounds__(kSkThreads, 8) void k_gemm_skinny(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sa, int64_t era, const float* __restrict__ sb,
    int64_t erb, const void* __restrict__ bias, int bias_bf16, void* __restrict__ Y, int64_t ldy,
    int vec_store) {
  __shared__ f32x4 red[kSkWaves - 1][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  const uint8_t* brow = B + min(n0 + r, N - 1) * ldb + 32 * g;
  const uint8_t* arow[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) arow[t] = A + min<int64_t>(16 * t + r, M - 1) * lda + 32 * g;

  // this wave's K steps: [s0, s1)
  const int nk = static_cast<int>(K / 128);
  const int s0 = (nk * wave) / kSkWaves, s1 = (nk * (wave + 1)) / kSkWaves;
  f32x4 acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Two steps per iteration (loads of both first, then both MFMAs): twice
  // the bytes in flight per wave.  An odd last step loads step s1 - 1 again
  // (a cache hit) and multiplies zeros in its place.
  auto mma = [&](const u32x4& b0, const u32x4& b1, const u32x4 (&a0)[MT], const u32x4 (&a1)[MT], bool on) {
    i32x8 bf = i32x8{(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
#pragma unroll
    for (int e = 0; e < 8; ++e) bf[e] = on ? bf[e] : 0;
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      const i32x8 af = i32x8{(int)a0[t][0], (int)a0[t][1], (int)a0[t][2], (int)a0[t][3],
                             (int)a1[t][0], (int)a1[t][1], (int)a1[t][2], (int)a1[t][3]};
      acc[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf, af, acc[t], FB, FA, 0, 0, 0, 0);
    }
  };
  for (int st = s0; st < s1; st += 2) {
    const int st2 = min(st + 1, s1 - 1);
    const int64_t ko = static_cast<int64_t>(st) * 128, ko2 = static_cast<int64_t>(st2) * 128;
    const u32x4 b0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + ko));
    const u32x4 b1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + ko + 16));
    const u32x4 c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + ko2));
    const u32x4 c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + ko2 + 16));
    u32x4 a0[MT], a1[MT], d0[MT], d1[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      a0[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko);
      a1[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko + 16);
      d0[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko2);
      d1[t] = *reinterpret_cast<const u32x4*>(arow[t] + ko2 + 16);
    }
    mma(b0, b1, a0, a1, true);
    mma(c0, c1, d0, d1, st + 1 < s1);
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
#pragma unroll 1
    for (int w = 0; w < kSkWaves - 1; ++w) acc[t] += red[w][t][lane];

  // lane: output row m = 16 t + r, columns n0 + 4 g + (0..3)
  const int64_t nb = n0 + 4 * g;
  float sbv[4], bv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t n = min(nb + e, N - 1);
    sbv[e] = sb[erb == 1 ? n : 0];
    bv[e] = 0.0f;
    if (bias)
      bv[e] = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[n]) << 16)
                        : static_cast<const float*>(bias)[n];
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) {
    const int64_t m = 16 * t + r;
    if (m >= M) continue;
    const float sav = sa[era == 1 ? m : 0];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = acc[t][e] * (sav * sbv[e]) + bv[e];
    if constexpr (BF16OUT) {
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
}

template <int FA, int FB, int MT>
void launch_mt(const GemmArgs& g, hipStream_t st, int vec) {
  const dim3 grid(static_cast<unsigned>((g.N + 15) / 16));
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
  if (g.yt == FP8RT_BF16)
    hipLaunchKernelGGL((k_gemm_skinny<FA, FB, MT, true>), grid, dim3(kSkThreads), 0, st, g.a, g.lda, g.b,
                       g.ldb, g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, vec);
  else
    hipLaunchKernelGGL((k_gemm_skinny<FA, FB, MT, false>), grid, dim3(kSkThreads), 0, st, g.a, g.lda, g.b,
                       g.ldb, g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, vec);
}

template <int FA, int FB>
void launch_fmt(const GemmArgs& g, hipStream_t st, int vec) {
  launch_mt<FA, FB, 1>(g, st, vec);
}

}  // namespace

bool gemm_skinny_eligible(const GemmArgs& g) {
  // per-tensor or per-row scales (selected, not divided); whole 128-deep K steps
  const bool rows_ok = (g.era == 1 || g.era >= g.M) && (g.erb == 1 || g.erb >= g.N);
  return rows_ok && !g.pow2_mx && g.eca >= g.K && g.ecb >= g.K && g.M <= kSkMaxM && g.K % 128 == 0;
}

hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t st) {
  const int esz = g.yt == FP8RT_BF16 ? 2 : 4;
  const int vec = ((g.ldy * esz) % (4 * esz) == 0) && ((reinterpret_cast<uintptr_t>(g.y) & (4 * esz - 1)) == 0);
  if (g.fa == FP8RT_E4M3) launch_fmt<0, 0>(g, st, vec);
  else launch_fmt<1, 0>(g, st, vec);
  return hipGetLastError();
}

}  // namespace fp8rt
