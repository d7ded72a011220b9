// gemm_wonly.hip -- weight-only FP8 GEMM: FP8 weights with their scales
// times BF16 activations, for decode-shaped layers (a few activation rows).
//
// Method: "FP8 formats and scaling for LLM inference", section "Weight-only
// FP8 and W8A8 FP8" (weights stored as FP8, activations kept in BF16, the
// kernel converts the weight after reading it; the gain is weight bytes) and
// section "Per-channel and block scaling" (per-channel and K-group scales):
//   Y[m,n] = sum_k x[m,k] s_w(n,k) dec(W[n,k]) + bias[n].
//
// Design for MI355X:
//  - Every E4M3 and E5M2 value is exactly a bf16 value, so the codes are
//    widened to bf16 in registers (v_cvt_scalef32_pk_bf16_fp8 / _bf8 with
//    scale 1, two codes per instruction) and multiplied on
//    v_mfma_f32_16x16x32_bf16, whose bf16 x bf16 products are exact in FP32.
//    The weight scale is applied in FP32: once in the epilogue for tensor /
//    channel scales, or to each 128-deep step's partial sum for K-group
//    scales (group widths are multiples of 128).
//  - With M <= 16 per workgroup row the work is streaming W once from HBM.
//    A workgroup of 16 waves owns 32 output columns (two 16-row tiles of W);
//    wave w takes the w-th sixteenth of the 128-deep K steps.  Per step a
//    lane loads 32 contiguous bytes of one W row (the four lane quarters
//    cover the row's whole 128-byte line, nontemporally: W is read once) and
//    the matching 32 bf16 activations (from L2: every workgroup reads all of
//    X), and each activation load serves both column tiles.
//  - MFMA operand order: W as the first operand, so each lane ends with 4
//    consecutive output columns of one activation row.  Within one MFMA,
//    lane quarter q and sub-step j cover K [32 q + 8 j, +8) of the step on
//    both operands.
//  - The 16 partial sums meet in LDS; wave 0 adds them in wave order,
//    scales, adds the bias, rounds and stores.
//  - Fragment-ordered W (fp8_pack_weights16): the lane's two 16-byte pieces
//    of a step sit at the same place of its tile's two KB halves, so each
//    weight load instruction reads 1 KB contiguous; the MFMA gets the same
//    bytes as from row-major W and the results are identical.  A packed W has
//    K a multiple of 128 (no tail step).
//  - A K tail (K a multiple of 16) is handled in the last step by loading
//    whole 16-byte pieces from the row start and zeroing them (both operands,
//    so no code beyond K can contribute a NaN).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWoWaves = 16;
constexpr int kWoThreads = kWoWaves * 64;
constexpr int kWoTiles = 2;            // 16-column tiles per workgroup
constexpr int kWoCols = 16 * kWoTiles;

// Two FP8 codes of a dword half -> two bf16 in one dword (element order
// kept), by one conversion whose scale operand is 1.0: exact.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
template <int F, bool HI>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
  bf16x2 h;
  if constexpr (F == kE4M3) {
    h = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<int>(w), 1.0f, HI);
  } else {
    h = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(static_cast<int>(w), 1.0f, HI);
  }
  return __builtin_bit_cast(uint32_t, h);
}

// 8 codes (2 dwords, K order) -> 8 bf16 in K order.
template <int F>
__device__ __forceinline__ bf16x8 widen8(uint32_t w0, uint32_t w1) {
  const u32x4 o = u32x4{widen2<F, false>(w0), widen2<F, true>(w0), widen2<F, false>(w1), widen2<F, true>(w1)};
  return __builtin_bit_cast(bf16x8, o);
}

struct Step {
  u32x4 w[kWoTiles][2];  // K [32 q, +32) of the lane's W row in each tile
  u32x4 x[4];            // K [32 q + 8 j, +8) of the lane's activation row
};

// Row-major W: wrow[t] is the lane's row, the piece at K offset off.  Packed
// W: wrow[t] is the lane's slot of its group's first tile; step ko / 128 is
// 2048 bytes further, half h 1024 (GUARD is never taken: K % 128 == 0).
template <bool GUARD, bool PACKED>
__device__ __forceinline__ void load_step(Step& s, const uint8_t* const (&wrow)[kWoTiles], const uint16_t* xrow,
                                          int64_t ko, int q, int64_t K) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t off = ko + 32 * q + 16 * h;
    const bool ok = !GUARD || off < K;
    const int64_t woff = PACKED ? (ko >> 7) * 2048 + 1024 * h : off;
#pragma unroll
    for (int t = 0; t < kWoTiles; ++t) {
      const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(wrow[t] + (ok ? woff : 0)));
      s.w[t][h] = ok ? v : u32x4{0u, 0u, 0u, 0u};
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t off = ko + 32 * q + 8 * j;
    const bool ok = !GUARD || off < K;
    const u32x4 v = *reinterpret_cast<const u32x4*>(xrow + (ok ? off : 0));
    s.x[j] = ok ? v : u32x4{0u, 0u, 0u, 0u};
  }
}

// One step's products into p[t] (p[t] is added to; GROUPED callers pass zeros).
template <int F>
__device__ __forceinline__ void mma_step(const Step& s, f32x4 (&p)[kWoTiles]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const bf16x8 xf = __builtin_bit_cast(bf16x8, s.x[j]);
#pragma unroll
    for (int t = 0; t < kWoTiles; ++t) {
      const u32x4& w = s.w[t][j >> 1];
      const bf16x8 wf = widen8<F>(w[2 * (j & 1)], w[2 * (j & 1) + 1]);
      p[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf, p[t], 0, 0, 0);
    }
  }
}

template <int F, bool GROUPED, bool BF16OUT, bool PACKED>
__global__ __launch_bounds__(kWoThreads, 1) void k_gemm_wonly(
    const uint16_t* __restrict__ X, int64_t ldx, const uint8_t* __restrict__ W, int64_t ldw, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sw, int64_t erw, int64_t ecw, int64_t ncw,
    const void* __restrict__ bias, int bias_bf16, void* __restrict__ Y, int64_t ldy, int vec_store) {
  __shared__ f32x4 red[kWoWaves - 1][kWoTiles][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, q = lane >> 4;
  const int64_t n0 = static_cast<int64_t>(blockIdx.x) * kWoCols;
  const int64_t m = static_cast<int64_t>(blockIdx.y) * 16 + r;
  const uint16_t* xrow = X + min(m, M - 1) * ldx;
  const uint8_t* wrow[kWoTiles];
#pragma unroll
  for (int t = 0; t < kWoTiles; ++t) {
    if constexpr (PACKED) {
      // 16-row group 2 blockIdx.x + t, clamped to the last one (a tile past N
      // loads valid bytes whose outputs are never stored)
      const int64_t grp = min(static_cast<int64_t>(blockIdx.x) * kWoTiles + t, (N + 15) / 16 - 1);
      wrow[t] = W + grp * (K / 128) * 2048 + lane * 16;
    } else {
      wrow[t] = W + min(n0 + 16 * t + r, N - 1) * ldw;
    }
  }

  // K-group scales: element offsets of the scale rows of the lane's output
  // columns n0 + 16 t + 4 q + v (the table has fewer than 2^31 entries)
  int soff[kWoTiles][4];
  if constexpr (GROUPED) {
#pragma unroll
    for (int t = 0; t < kWoTiles; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        soff[t][v] = static_cast<int>((min(n0 + 16 * t + 4 * q + v, N - 1) / erw) * ncw);
  }

  const int nk = static_cast<int>((K + 127) / 128);
  const int s0 = (nk * wave) / kWoWaves, s1 = (nk * (wave + 1)) / kWoWaves;
  f32x4 acc[kWoTiles];
#pragma unroll
  for (int t = 0; t < kWoTiles; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto run = [&](const Step& s, int st) {
    if constexpr (GROUPED) {
      f32x4 p[kWoTiles];
#pragma unroll
      for (int t = 0; t < kWoTiles; ++t) p[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      mma_step<F>(s, p);
      const int grp = static_cast<int>((static_cast<int64_t>(st) * 128) / ecw);
#pragma unroll
      for (int t = 0; t < kWoTiles; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] += sw[soff[t][v] + grp] * p[t][v];
    } else {
      mma_step<F>(s, acc);
    }
  };

  // Two steps per iteration: the loads of both are issued before either
  // step's MFMAs.  An odd last step is run alone.  K-group scales take one
  // step per iteration (the scales and partial sums of a second step in
  // flight do not fit the 128 VGPRs of a 16-wave workgroup).
  int st = s0;
  for (; !GROUPED && st + 1 < s1; st += 2) {
    const int64_t ko = static_cast<int64_t>(st) * 128;
    Step a, b;
    if (ko + 256 <= K) {
      load_step<false, PACKED>(a, wrow, xrow, ko, q, K);
      load_step<false, PACKED>(b, wrow, xrow, ko + 128, q, K);
    } else {
      load_step<true, PACKED>(a, wrow, xrow, ko, q, K);
      load_step<true, PACKED>(b, wrow, xrow, ko + 128, q, K);
    }
    run(a, st);
    run(b, st + 1);
  }
  for (; st < s1; ++st) {
    const int64_t ko = static_cast<int64_t>(st) * 128;
    Step a;
    if (ko + 128 <= K) load_step<false, PACKED>(a, wrow, xrow, ko, q, K);
    else load_step<true, PACKED>(a, wrow, xrow, ko, q, K);
    run(a, st);
  }

  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < kWoTiles; ++t) red[wave - 1][t][lane] = acc[t];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int t = 0; t < kWoTiles; ++t)
#pragma unroll 5  // 15 partials: three batches of 5 reads in flight
    for (int w = 0; w < kWoWaves - 1; ++w) acc[t] += red[w][t][lane];
  if (m >= M) return;

#pragma unroll
  for (int t = 0; t < kWoTiles; ++t) {
    const int64_t nb = n0 + 16 * t + 4 * q;  // this lane's 4 output columns
    if (nb >= N) continue;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t n = min(nb + e, N - 1);
      float bv = 0.0f;
      if (bias)
        bv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[n]) << 16)
                       : static_cast<const float*>(bias)[n];
      if constexpr (GROUPED) {
        v[e] = acc[t][e] + bv;
      } else {
        v[e] = acc[t][e] * sw[n / erw] + bv;
      }
    }
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

template <int F, bool GROUPED, bool PACKED>
void launch_fp(const WonlyArgs& g, hipStream_t st, int vec) {
  const dim3 grid(static_cast<unsigned>((g.N + kWoCols - 1) / kWoCols), static_cast<unsigned>((g.M + 15) / 16));
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
  const int64_t ncw = (g.K + g.ecw - 1) / g.ecw;
  if (g.yt == FP8RT_BF16)
    hipLaunchKernelGGL((k_gemm_wonly<F, GROUPED, true, PACKED>), grid, dim3(kWoThreads), 0, st, g.x, g.ldx, g.w,
                       g.ldw, g.M, g.N, g.K, g.sw, g.erw, g.ecw, ncw, g.bias, bb, g.y, g.ldy, vec);
  else
    hipLaunchKernelGGL((k_gemm_wonly<F, GROUPED, false, PACKED>), grid, dim3(kWoThreads), 0, st, g.x, g.ldx, g.w,
                       g.ldw, g.M, g.N, g.K, g.sw, g.erw, g.ecw, ncw, g.bias, bb, g.y, g.ldy, vec);
}

template <int F, bool GROUPED>
void launch_f(const WonlyArgs& g, hipStream_t st, int vec) {
  if (g.w_packed) launch_fp<F, GROUPED, true>(g, st, vec);
  else launch_fp<F, GROUPED, false>(g, st, vec);
}

}  // namespace

hipError_t launch_gemm_wonly(const WonlyArgs& g, hipStream_t st) {
  const int esz = g.yt == FP8RT_BF16 ? 2 : 4;
  const int vec = ((g.ldy * esz) % (4 * esz) == 0) && ((reinterpret_cast<uintptr_t>(g.y) & (4 * esz - 1)) == 0);
  const bool grouped = g.ecw < g.K;
  if (g.fw == FP8RT_E4M3) {
    if (grouped) launch_f<kE4M3, true>(g, st, vec);
    else launch_f<kE4M3, false>(g, st, vec);
  } else {
    if (grouped) launch_f<kE5M2, true>(g, st, vec);
    else launch_f<kE5M2, false>(g, st, vec);
  }
  return hipGetLastError();
}

}  // namespace fp8rt
