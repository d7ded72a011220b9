// ledger.hip -- the FP8 granularity ledger: the reconstruction error of a
// quantized weight (k_quant_error + k_ledger_finish) and the host routine
// that quantizes one weight at each requested granularity and reports scale
// metadata against error.
//
// Method: "Quantization W8A16" (datawhalechina llm-algo-leetcode), its
// granularity comparison: for a fixed weight and fixed inputs, each
// granularity's scale count and bytes, the total state bytes, the restored
// weight's mean squared error, and the layer output's mean squared error and
// cosine similarity against the unquantized layer.  Here the weight is
// quantized to FP8 ("FP8 formats and scaling for LLM inference", sections
// "How a scale fits a tensor into E4M3" and "Per-channel and block scaling":
// finer groups trade scale metadata for precision).
//
// Readings: the restored weight is the dequantization fl32(s dec(q)); the
// output error is the quantization's, not a GEMM's rounding: y_ref = x W^T
// and d = y_q - y_ref = x (W_hat - W)^T with FP32 products summed over
// 8-element runs and combined in binary64; cosine = <y_ref, y_q> /
// max(|y_ref| |y_q|, 1e-8).
//
// Design for MI355X: a wave takes 4 weight rows (grid-stride), lane l taking
// 8 consecutive elements of every 512-wide K chunk, so W, its codes and each
// activation row are read with 16-, 8- and 16-byte loads, and one activation
// load serves the 4 rows (the activations are re-read from L2 once per 4
// weight rows).  The weight sums are binary64 (e is exact there); each output
// dot product keeps one FP32 partial per lane (8 activation rows per pass),
// reduced across the wave in a fixed butterfly.  Per-block partials go to a
// finisher that adds them in a fixed order: the result does not depend on
// scheduling.
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <vector>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

constexpr int kLgWaves = 4;
constexpr int kLgThreads = kLgWaves * 64;
constexpr int kLgM = 8;        // activation rows per pass
constexpr int kLgR = 4;        // weight rows per wave
constexpr int kLgMaxBlocks = 4096;

// {sum e^2, sum w^2, max |e|, sum d^2, sum y_ref^2, sum y_q^2, sum y_ref y_q, any NaN e}
struct LedgerPartial {
  double v[8];
};

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}

template <typename WT, int F>
__global__ __launch_bounds__(kLgThreads) void k_quant_error(const WT* __restrict__ W, int64_t ldw,
                                                            const uint8_t* __restrict__ Q, int64_t ldq, int64_t N,
                                                            int64_t K, const float* __restrict__ S, int64_t er,
                                                            int64_t ec, int64_t nc, const uint16_t* __restrict__ X,
                                                            int64_t M, int64_t ldx,
                                                            LedgerPartial* __restrict__ part) {
  __shared__ double red[kLgWaves][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nwaves = static_cast<int64_t>(gridDim.x) * kLgWaves;
  double se = 0.0, sw = 0.0, emax = 0.0, sd = 0.0, syr = 0.0, syq = 0.0, syrq = 0.0;
  uint32_t nan = 0;
  const int64_t nchunks = (K + 511) / 512;
  const int npass = X ? static_cast<int>((M + kLgM - 1) / kLgM) : 1;
  // kLgR weight rows per wave: each activation octet loaded serves all of them
  for (int64_t n0 = (static_cast<int64_t>(blockIdx.x) * kLgWaves + wave) * kLgR; n0 < N; n0 += nwaves * kLgR) {
    const WT* wrow[kLgR];
    const uint8_t* qrow[kLgR];
    const float* srow[kLgR];
    bool live[kLgR];
#pragma unroll
    for (int i = 0; i < kLgR; ++i) {
      live[i] = n0 + i < N;
      const int64_t n = live[i] ? n0 + i : N - 1;  // clamped: loads stay in bounds, results unused
      wrow[i] = W + n * ldw;
      qrow[i] = Q + n * ldq;
      srow[i] = S + (n / er) * nc;
    }
    for (int p = 0; p < npass; ++p) {
      float ad[kLgR][kLgM], ay[kLgR][kLgM];
#pragma unroll
      for (int i = 0; i < kLgR; ++i)
#pragma unroll
        for (int mm = 0; mm < kLgM; ++mm) ad[i][mm] = ay[i][mm] = 0.0f;
      for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t k0 = c * 512 + 8 * lane;
        if (k0 >= K) continue;  // K is a multiple of 8: a started octet is whole
        float e[kLgR][8], wv[kLgR][8];
#pragma unroll
        for (int i = 0; i < kLgR; ++i) {
          Octet<WT> wo;
          wo.load(wrow[i] + k0);
          const u32x2 qv = *reinterpret_cast<const u32x2*>(qrow[i] + k0);
          const float sv = srow[i][k0 / ec];
          float dq[8];
          decode4<F>(qv[0], dq);
          decode4<F>(qv[1], dq + 4);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float wh = sv * dq[j];  // the dequantization fl32(s dec(q))
            wv[i][j] = wo.get(j);
            e[i][j] = wh - wv[i][j];
            if (p == 0 && live[i]) {
              const double ed = static_cast<double>(wh) - static_cast<double>(wv[i][j]);  // exact
              se += ed * ed;
              sw += static_cast<double>(wv[i][j]) * static_cast<double>(wv[i][j]);
              nan |= (ed != ed) ? 1u : 0u;
              emax = fmax(emax, fabs(ed));
            }
          }
        }
        if (X) {
#pragma unroll
          for (int mm = 0; mm < kLgM; ++mm) {
            const int64_t m = static_cast<int64_t>(p) * kLgM + mm;
            if (m >= M) break;
            Octet<uint16_t> xo;
            xo.load(X + m * ldx + k0);
#pragma unroll
            for (int i = 0; i < kLgR; ++i) {
              float pd = 0.0f, py = 0.0f;
#pragma unroll
              for (int j = 0; j < 8; ++j) {
                pd += xo.get(j) * e[i][j];
                py += xo.get(j) * wv[i][j];
              }
              ad[i][mm] += pd;
              ay[i][mm] += py;
            }
          }
        }
      }
      if (X) {
#pragma unroll
        for (int i = 0; i < kLgR; ++i)
#pragma unroll
          for (int mm = 0; mm < kLgM; ++mm) {
            const int64_t m = static_cast<int64_t>(p) * kLgM + mm;
            if (m >= M) break;
            const double dd = static_cast<double>(wave_sum_f32(ad[i][mm]));
            const double yr = static_cast<double>(wave_sum_f32(ay[i][mm]));
            if (lane == 0 && live[i]) {
              const double yq = yr + dd;
              sd += dd * dd;
              syr += yr * yr;
              syq += yq * yq;
              syrq += yr * yq;
            }
          }
      }
    }
  }
  // lane partials -> wave -> block (fixed orders)
  se = wave_sum_f64(se);
  sw = wave_sum_f64(sw);
  emax = wave_max_f64(emax);
  nan = wave_max_u32(nan);
  if (lane == 0) {
    red[wave][0] = se;
    red[wave][1] = sw;
    red[wave][2] = emax;
    red[wave][3] = sd;
    red[wave][4] = syr;
    red[wave][5] = syq;
    red[wave][6] = syrq;
    red[wave][7] = nan ? 1.0 : 0.0;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int j = threadIdx.x;
    double a = red[0][j];
    for (int w = 1; w < kLgWaves; ++w) a = (j == 2 || j == 7) ? fmax(a, red[w][j]) : a + red[w][j];
    part[blockIdx.x].v[j] = a;
  }
}

// Adds the block partials in a fixed order: thread t takes partials t,
// t + 256, ..., then a tree in LDS.  stats[7] = the seven sums (max |e| is
// NaN when any e was).
__global__ __launch_bounds__(256) void k_ledger_finish(const LedgerPartial* __restrict__ part, int nb,
                                                       double* __restrict__ stats) {
  __shared__ double red[256][8];
  const int t = threadIdx.x;
  double a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int b = t; b < nb; b += 256)
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = (j == 2 || j == 7) ? fmax(a[j], part[b].v[j]) : a[j] + part[b].v[j];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[t][j] = a[j];
  __syncthreads();
  for (int s = 128; s >= 1; s >>= 1) {
    if (t < s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        red[t][j] = (j == 2 || j == 7) ? fmax(red[t][j], red[t + s][j]) : red[t][j] + red[t + s][j];
    __syncthreads();
  }
  if (t < 7) stats[t] = (t == 2 && red[0][7] != 0.0) ? __longlong_as_double(0x7FF8000000000000LL) : red[0][t];
}

}  // namespace

size_t quant_error_partials_bytes(int64_t N) {
  const int64_t nb = std::min<int64_t>((N + kLgWaves * kLgR - 1) / (kLgWaves * kLgR), kLgMaxBlocks);
  return static_cast<size_t>(nb) * sizeof(LedgerPartial);
}

hipError_t launch_quant_error(const QuantErrorArgs& g, void* partials, hipStream_t st) {
  const int nb = static_cast<int>(
      std::min<int64_t>((g.N + kLgWaves * kLgR - 1) / (kLgWaves * kLgR), kLgMaxBlocks));
  LedgerPartial* part = static_cast<LedgerPartial*>(partials);
  const int64_t nc = (g.K + g.ec - 1) / g.ec;
#define FP8RT_QE(WT, F)                                                                                      \
  hipLaunchKernelGGL((k_quant_error<WT, F>), dim3(nb), dim3(kLgThreads), 0, st, static_cast<const WT*>(g.w), \
                     g.ldw, g.q, g.ldq, g.N, g.K, g.scale, g.er, g.ec, nc, g.x, g.M, g.ldx, part)
  if (g.wt == FP8RT_BF16) {
    if (g.f == FP8RT_E4M3) FP8RT_QE(uint16_t, kE4M3);
    else FP8RT_QE(uint16_t, kE5M2);
  } else {
    if (g.f == FP8RT_E4M3) FP8RT_QE(float, kE4M3);
    else FP8RT_QE(float, kE5M2);
  }
#undef FP8RT_QE
  hipLaunchKernelGGL(k_ledger_finish, dim3(1), dim3(256), 0, st, part, nb, g.stats);
  return hipGetLastError();
}

}  // namespace fp8rt
