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
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kSkWaves = 16;
constexpr int kSkThreads = kSkWaves * 64;
constexpr int kSkMaxM = 16;

template <int FA, int FB, int MT, bool BF16OUT, bool PACKED>
__global__ __launch_bounds__(kSkThreads, 8) void k_gemm_skinny(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sa, int64_t era, const float* __restrict__ sb,
    int64_t erb, const void* __restrict__ bias, int bias_bf16, void* __restrict__ Y, int64_t ldy,
    int vec_store) {
  __shared__ f32x4 red[kSkWaves - 1][MT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * 16;
  // row-major: row n0 + r, bytes 32 g of each step; packed: the lane's
  // 16-byte slots of its group's 2 KB tiles
  const uint8_t* brow = PACKED ? B + static_cast<int64_t>(blockIdx.x) * (K / 128) * 2048 + lane * 16
                               : B + min(n0 + r, N - 1) * ldb + 32 * g;
  const int64_t bstep = PACKED ? 2048 : 128, bhalf = PACKED ? 1024 : 16;
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
    const int64_t bo = static_cast<int64_t>(st) * bstep, bo2 = static_cast<int64_t>(st2) * bstep;
    const u32x4 b0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo));
    const u32x4 b1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo + bhalf));
    const u32x4 c0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo2));
    const u32x4 c1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(brow + bo2 + bhalf));
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

template <int FA, int FB, int MT, bool PACKED>
void launch_mt(const GemmArgs& g, hipStream_t st, int vec) {
  const dim3 grid(static_cast<unsigned>((g.N + 15) / 16));
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
  if (g.yt == FP8RT_BF16)
    hipLaunchKernelGGL((k_gemm_skinny<FA, FB, MT, true, PACKED>), grid, dim3(kSkThreads), 0, st, g.a, g.lda, g.b,
                       g.ldb, g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, vec);
  else
    hipLaunchKernelGGL((k_gemm_skinny<FA, FB, MT, false, PACKED>), grid, dim3(kSkThreads), 0, st, g.a, g.lda, g.b,
                       g.ldb, g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, vec);
}

template <int FA, int FB>
void launch_fmt(const GemmArgs& g, hipStream_t st, int vec) {
  if (g.b_packed) launch_mt<FA, FB, 1, true>(g, st, vec);
  else launch_mt<FA, FB, 1, false>(g, st, vec);
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
  // per-tensor or per-row scales (selected, not divided); whole 128-deep K steps
  const bool rows_ok = (g.era == 1 || g.era >= g.M) && (g.erb == 1 || g.erb >= g.N);
  return rows_ok && !g.pow2_mx && g.eca >= g.K && g.ecb >= g.K && g.M <= kSkMaxM && g.K % 128 == 0;
}

hipError_t launch_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp,
                                 hipStream_t st) {
  const int64_t nchunks = (N + 15) / 16 * (K / 128) * 128;  // 16-byte pieces
  const int64_t nb = std::min<int64_t>((nchunks + 255) / 256, int64_t(1) << 20);
  hipLaunchKernelGGL(k_pack_weights16, dim3(static_cast<unsigned>(nb)), dim3(256), 0, st, q, N, K, ldq, qp, nchunks);
  return hipGetLastError();
}

hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t st) {
  const int esz = g.yt == FP8RT_BF16 ? 2 : 4;
  const int vec = ((g.ldy * esz) % (4 * esz) == 0) && ((reinterpret_cast<uintptr_t>(g.y) & (4 * esz - 1)) == 0);
  if (g.fa == FP8RT_E4M3) launch_fmt<0, 0>(g, st, vec);
  else launch_fmt<1, 0>(g, st, vec);
  return hipGetLastError();
}

}  // namespace fp8rt
