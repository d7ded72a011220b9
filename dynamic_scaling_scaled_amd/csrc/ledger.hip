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
// and d = y_q - y_ref = x (W_hat - W)^T, with FP32 accumulation of exact
// products; cosine = <y_ref, y_q> / max(|y_ref| |y_q|, 1e-8).
//
// Design for MI355X: the weight and its codes are streamed once, with
// nontemporal loads, and the 2 M N K products run on the matrix cores, not
// the vector ALU.
//  - One workgroup of 4 waves owns 16 weight rows (grid-stride over such
//    tiles) and walks K in 512-deep super-steps.  In a super-step wave w
//    reads rows 4 w .. 4 w + 3 row-contiguously: lane l takes 8 elements at K
//    offset 8 l, so each load instruction covers 1 KB of one row (bf16 W) or
//    512 code bytes (whole DRAM bursts of one row; reading 256 bytes from
//    each of 4 rows per instruction left the L1 stalled on its outstanding
//    misses at 2.2 TB/s).  In that layout it forms e = fl32(s dec(q)) - w and
//    the binary64 weight sums (e exact there).
//  - For the products, e (binary32) and W's bits are staged in LDS for the
//    block; after a barrier wave w takes the super-step's w-th 128-deep step
//    in the matrix-core layout: lane (r, q) = (lane % 16, lane / 16) takes
//    row r's K [32 j + 8 q, +8) in run j, the same K positions as its
//    activation row r (read from L2 in that layout).  e is split exactly into
//    three bf16 parts (truncate to the top 8 significant bits, subtract,
//    again): e = e_hi + e_mid + e_lo, so every bf16 x bf16 product on
//    v_mfma_f32_16x16x32_bf16 is exact and only the FP32 accumulation
//    rounds.  x W^T uses W's bf16 bits directly (an fp32 W is split the same
//    way).
//  - The 4 waves' 16 x 16 partial dot products meet in LDS, summed in wave
//    order; wave 0 squares and accumulates them in binary64.  Per-block
//    partials go to a finisher that adds them in a fixed order: the result
//    does not depend on scheduling.
#include <hip/hip_runtime.h>

#include <math.h>

#include <algorithm>
#include <vector>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

constexpr int kLgWaves = 4;  // waves per 16-row tile
constexpr int kLgThreads = kLgWaves * 64;
constexpr int kLgMaxBlocks = 4096;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// {sum e^2, sum w^2, max |e|, sum d^2, sum y_ref^2, sum y_q^2, sum y_ref y_q, any NaN e}
struct LedgerPartial {
  double v[8];
};

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

// Exact split of a binary32 value into three bf16 bit patterns whose sum is
// the value: each part keeps the top 8 significant bits of what is left.  A
// non-finite value goes whole into the first part (NaN stays NaN, +-Inf stays
// +-Inf).
__device__ __forceinline__ void split3(float v, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t hb = __float_as_uint(v) & 0xFFFF0000u;
  float r = v - __uint_as_float(hb);
  r = (__uint_as_float(hb) == v) ? 0.0f : r;  // exact already, or +-Inf
  const uint32_t mb = __float_as_uint(r) & 0xFFFF0000u;
  const float lo = r - __uint_as_float(mb);
  h = hb >> 16;
  m = mb >> 16;
  l = __float_as_uint(lo) >> 16;
}

__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) { return lo16 | (hi16 << 16); }

// 8 weights of one run as floats: bf16 from one 16-byte vector, fp32 from two.
template <typename WT>
struct WRun;
template <>
struct WRun<uint16_t> {
  u32x4 v;
  __device__ __forceinline__ void load(const uint16_t* p) {
    v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  __device__ __forceinline__ void zero() { v = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = v[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
};
template <>
struct WRun<float> {
  u32x4 v[2];
  __device__ __forceinline__ void load(const float* p) {
    v[0] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    v[1] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + 4));
  }
  __device__ __forceinline__ void zero() { v[0] = v[1] = u32x4{0u, 0u, 0u, 0u}; }
  __device__ __forceinline__ float get(int i) const { return __uint_as_float(v[i >> 2][i & 3]); }
};

// The loads of one 512-deep super-step of a lane: 8 weights, 8 codes and a
// scale of each of its wave's 4 rows; lane l takes K offset 8 l, so one load
// instruction reads 1 KB (bf16 W) or 512 bytes (codes) of one row.
template <typename WT>
struct LgStep {
  WRun<WT> wr[4];
  u32x2 qv[4];
  float sv[4];
};

template <typename WT, int F, bool HAS_X>
__global__ __launch_bounds__(kLgThreads) void k_quant_error(const WT* __restrict__ W, int64_t ldw,
                                                            const uint8_t* __restrict__ Q, int64_t ldq, int64_t N,
                                                            int64_t K, const float* __restrict__ S, int64_t er,
                                                            int64_t ec, int64_t nc, const uint16_t* __restrict__ X,
                                                            int64_t M, int64_t ldx,
                                                            LedgerPartial* __restrict__ part) {
  constexpr int kSs = 512;  // K per super-step
  // staged e (binary32) and W bits of a super-step, shared by the block; rows
  // padded so that the 16 rows of a matrix-core read start 4 banks apart
  constexpr int kEd = kSs + 4;                                // floats per row of e
  constexpr int kWd = sizeof(WT) == 2 ? kSs / 2 + 4 : kSs + 4;  // dwords per row of W
  constexpr int kRows = HAS_X ? 16 : 1;
  __shared__ __attribute__((aligned(16))) float lde[kRows][kEd];
  __shared__ __attribute__((aligned(16))) uint32_t ldw_[kRows][kWd];
  __shared__ f32x4 red[kLgWaves][2][64];
  __shared__ double wred[kLgWaves][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r = lane & 15, lq = lane >> 4;
  const int kl = 8 * lane;  // load layout: K offset of this lane's 8 elements in a super-step
  const int64_t tiles = (N + 15) / 16;
  const int nss = static_cast<int>((K + kSs - 1) / kSs);
  const int64_t mtiles = HAS_X ? (M + 15) / 16 : 1;
  double se2[2] = {0.0, 0.0}, sw2[2] = {0.0, 0.0}, emax2[2] = {0.0, 0.0};
  double sd = 0.0, syr = 0.0, syq = 0.0, syrq = 0.0;

  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    // the 4 rows this wave loads: 4 wave + i
    const WT* wrow[4];
    const uint8_t* qrow[4];
    const float* srow[4];
    bool live[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = tile * 16 + 4 * wave + i;
      live[i] = n < N;
      const int64_t nr = live[i] ? n : N - 1;  // clamped: loads stay in bounds, values zeroed
      wrow[i] = W + nr * ldw;
      qrow[i] = Q + nr * ldq;
      srow[i] = S + (nr / er) * nc;
    }
    for (int64_t mt = 0; mt < mtiles; ++mt) {
      const bool first = mt == 0;
      const int64_t m = mt * 16 + r;
      const bool mlive = HAS_X && m < M;
      const uint16_t* xrow = HAS_X ? X + (mlive ? m : M - 1) * ldx : nullptr;
      f32x4 ae = f32x4{0.f, 0.f, 0.f, 0.f}, aw = f32x4{0.f, 0.f, 0.f, 0.f};
      // K % 16 == 0, so 8 elements are wholly inside or wholly past K (then
      // they read offset 0 and are zeroed)
      auto load_step = [&](LgStep<WT>& L, int ss) {
        const int64_t kb = static_cast<int64_t>(ss) * kSs;
        const int64_t kk = kb + kl < K ? kb + kl : 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          L.wr[i].load(wrow[i] + kk);
          L.qv[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(qrow[i] + kk));
        }
        // kk < K and ec = K for whole-row scales: the group index is 0 there
        // (computed without a branch, which would split the loads' block)
        const int sg = static_cast<int>(static_cast<uint32_t>(kk) / static_cast<uint32_t>(ec));
#pragma unroll
        for (int i = 0; i < 4; ++i) L.sv[i] = srow[i][sg];
      };
      // this wave's matrix-core step of a super-step: K [128 wave, +128),
      // run j at 32 j + 8 lq
      auto load_x = [&](u32x4 (&xv)[4], int ss) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t k = static_cast<int64_t>(ss) * kSs + 128 * wave + 32 * j + 8 * lq;
          xv[j] = *reinterpret_cast<const u32x4*>(xrow + (k < K ? k : 0));
        }
      };
      // weights and codes kDepth super-steps ahead (2 for the weight sums
      // alone; 1 with inputs, whose registers allow no more), activations
      // (from L2) one (past the last super-step the last one is reloaded,
      // unused)
      constexpr int kDepth = HAS_X ? 1 : 2;
      LgStep<WT> buf[kDepth + 1];
      u32x4 xcur[4], xnxt[4];
#pragma unroll
      for (int d = 0; d < kDepth; ++d) load_step(buf[d], min(d, nss - 1));
      if constexpr (HAS_X) load_x(xcur, 0);
      for (int ss = 0; ss < nss; ++ss) {
        load_step(buf[kDepth], min(ss + kDepth, nss - 1));
        if constexpr (HAS_X) load_x(xnxt, min(ss + 1, nss - 1));
        const LgStep<WT>& cur = buf[0];
        const int64_t kb = static_cast<int64_t>(ss) * kSs;
        const bool kok = kb + kl < K;
        // e and the weight sums in the load layout; stage e and W for the products
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool use = kok && live[i];
          float dq[8], ev[8];
          decode4<F>(cur.qv[i][0], dq);
          decode4<F>(cur.qv[i][1], dq + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float wv = cur.wr[i].get(e);
            const float wh = cur.sv[i] * dq[e];  // the dequantization fl32(s dec(q))
            if (first && use) {  // two independent chains per sum (even / odd e)
              const double ed = static_cast<double>(wh) - static_cast<double>(wv);  // exact
              se2[e & 1] += ed * ed;
              sw2[e & 1] += static_cast<double>(wv) * static_cast<double>(wv);
              emax2[e & 1] = fmax(emax2[e & 1], fabs(ed));
            }
            ev[e] = use ? wh - wv : 0.0f;
          }
          if constexpr (HAS_X) {
            const int row = 4 * wave + i;
            *reinterpret_cast<f32x4*>(&lde[row][kl]) = f32x4{ev[0], ev[1], ev[2], ev[3]};
            *reinterpret_cast<f32x4*>(&lde[row][kl + 4]) = f32x4{ev[4], ev[5], ev[6], ev[7]};
            if constexpr (sizeof(WT) == 2) {
              *reinterpret_cast<u32x4*>(&ldw_[row][kl / 2]) = use ? cur.wr[i].v : u32x4{0u, 0u, 0u, 0u};
            } else {
              *reinterpret_cast<u32x4*>(&ldw_[row][kl]) = use ? cur.wr[i].v[0] : u32x4{0u, 0u, 0u, 0u};
              *reinterpret_cast<u32x4*>(&ldw_[row][kl + 4]) = use ? cur.wr[i].v[1] : u32x4{0u, 0u, 0u, 0u};
            }
          }
        }
        if constexpr (HAS_X) {
          __syncthreads();  // the block's 16 rows of the super-step are staged
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kc = 128 * wave + 32 * j + 8 * lq;
            const bool xok = mlive && kb + kc < K;
            const f32x4 e0 = *reinterpret_cast<const f32x4*>(&lde[r][kc]);
            const f32x4 e1 = *reinterpret_cast<const f32x4*>(&lde[r][kc + 4]);
            uint32_t eh[8], em[8], el[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              split3(e0[e], eh[e], em[e], el[e]);
              split3(e1[e], eh[e + 4], em[e + 4], el[e + 4]);
            }
            const bf16x8 xb = __builtin_bit_cast(bf16x8, xok ? xcur[j] : u32x4{0u, 0u, 0u, 0u});
            const u32x4 ph = u32x4{pack2(eh[0], eh[1]), pack2(eh[2], eh[3]), pack2(eh[4], eh[5]), pack2(eh[6], eh[7])};
            const u32x4 pm = u32x4{pack2(em[0], em[1]), pack2(em[2], em[3]), pack2(em[4], em[5]), pack2(em[6], em[7])};
            const u32x4 pl = u32x4{pack2(el[0], el[1]), pack2(el[2], el[3]), pack2(el[4], el[5]), pack2(el[6], el[7])};
            ae = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ph), xb, ae, 0, 0, 0);
            ae = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pm), xb, ae, 0, 0, 0);
            ae = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pl), xb, ae, 0, 0, 0);
            if constexpr (sizeof(WT) == 2) {
              const u32x4 wb = *reinterpret_cast<const u32x4*>(&ldw_[r][kc / 2]);
              aw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wb), xb, aw, 0, 0, 0);
            } else {
              const u32x4 w0 = *reinterpret_cast<const u32x4*>(&ldw_[r][kc]);
              const u32x4 w1 = *reinterpret_cast<const u32x4*>(&ldw_[r][kc + 4]);
              uint32_t wh8[8], wm8[8], wl8[8];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                split3(__uint_as_float(w0[e]), wh8[e], wm8[e], wl8[e]);
                split3(__uint_as_float(w1[e]), wh8[e + 4], wm8[e + 4], wl8[e + 4]);
              }
              const u32x4 qh = u32x4{pack2(wh8[0], wh8[1]), pack2(wh8[2], wh8[3]), pack2(wh8[4], wh8[5]),
                                     pack2(wh8[6], wh8[7])};
              const u32x4 qm = u32x4{pack2(wm8[0], wm8[1]), pack2(wm8[2], wm8[3]), pack2(wm8[4], wm8[5]),
                                     pack2(wm8[6], wm8[7])};
              const u32x4 ql = u32x4{pack2(wl8[0], wl8[1]), pack2(wl8[2], wl8[3]), pack2(wl8[4], wl8[5]),
                                     pack2(wl8[6], wl8[7])};
              aw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qh), xb, aw, 0, 0, 0);
              aw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, qm), xb, aw, 0, 0, 0);
              aw = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ql), xb, aw, 0, 0, 0);
            }
          }
          __syncthreads();  // every read done before the next super-step's stores
        }
#pragma unroll
        for (int d = 0; d < kDepth; ++d) buf[d] = buf[d + 1];
        if constexpr (HAS_X) {
#pragma unroll
          for (int j = 0; j < 4; ++j) xcur[j] = xnxt[j];
        }
      }
      if constexpr (HAS_X) {
        // the 4 waves' partial dot products, added in wave order by wave 0
        red[wave][0][lane] = ae;
        red[wave][1][lane] = aw;
        __syncthreads();
        if (wave == 0) {
          f32x4 de = red[0][0][lane], dy = red[0][1][lane];
#pragma unroll 1
          for (int w = 1; w < kLgWaves; ++w) {
            de += red[w][0][lane];
            dy += red[w][1][lane];
          }
          // this lane holds weight rows 16 tile + 4 lq + v of activation row m;
          // padding entries are left out (0 x Inf would be NaN there)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            if (!(mlive && tile * 16 + 4 * lq + v < N)) continue;
            const double dd = static_cast<double>(de[v]);
            const double yr = static_cast<double>(dy[v]);
            const double yq = yr + dd;
            sd += dd * dd;
            syr += yr * yr;
            syq += yq * yq;
            syrq += yr * yq;
          }
        }
        __syncthreads();
      }
    }
  }
  // lane partials -> wave -> block (fixed orders); a NaN e makes sum e^2 NaN
  const double se = wave_sum_f64(se2[0] + se2[1]);
  const double sw = wave_sum_f64(sw2[0] + sw2[1]);
  const double emax = wave_max_f64(fmax(emax2[0], emax2[1]));
  sd = wave_sum_f64(sd);
  syr = wave_sum_f64(syr);
  syq = wave_sum_f64(syq);
  syrq = wave_sum_f64(syrq);
  if (lane == 0) {
    wred[wave][0] = se;
    wred[wave][1] = sw;
    wred[wave][2] = emax;
    wred[wave][3] = sd;
    wred[wave][4] = syr;
    wred[wave][5] = syq;
    wred[wave][6] = syrq;
    wred[wave][7] = (se != se) ? 1.0 : 0.0;
  }
  __syncthreads();
  if (threadIdx.x < 8) {
    const int j = threadIdx.x;
    double a = wred[0][j];
    for (int w = 1; w < kLgWaves; ++w) a = (j == 2 || j == 7) ? fmax(a, wred[w][j]) : a + wred[w][j];
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
  const int64_t nb = std::min<int64_t>((N + 15) / 16, kLgMaxBlocks);
  return static_cast<size_t>(nb) * sizeof(LedgerPartial);
}

hipError_t launch_quant_error(const QuantErrorArgs& g, void* partials, hipStream_t st) {
  const int nb = static_cast<int>(std::min<int64_t>((g.N + 15) / 16, kLgMaxBlocks));
  LedgerPartial* part = static_cast<LedgerPartial*>(partials);
  const int64_t nc = (g.K + g.ec - 1) / g.ec;
#define FP8RT_QE(WT, F)                                                                                           \
  do {                                                                                                            \
    if (g.x)                                                                                                      \
      hipLaunchKernelGGL((k_quant_error<WT, F, true>), dim3(nb), dim3(kLgThreads), 0, st,                        \
                         static_cast<const WT*>(g.w), g.ldw, g.q, g.ldq, g.N, g.K, g.scale, g.er, g.ec, nc, g.x, \
                         g.M, g.ldx, part);                                                                       \
    else                                                                                                          \
      hipLaunchKernelGGL((k_quant_error<WT, F, false>), dim3(nb), dim3(kLgThreads), 0, st,                       \
                         static_cast<const WT*>(g.w), g.ldw, g.q, g.ldq, g.N, g.K, g.scale, g.er, g.ec, nc, g.x, \
                         g.M, g.ldx, part);                                                                       \
  } while (0)
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
