// gemm_big.hip -- the large-shape scaled FP8 GEMM for gfx950 (per-tensor and
// per-row / per-output-channel scales applied in the epilogue).
//
// Method: "FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM": Y ~ s_x s_w (X8 W8) with FP32
// accumulation, BF16/FP32 output and bias; section "Per-channel and block
// scaling" for per-row scales.  Y[m,n] = s_a(m) s_b(n) sum_k dec(A[m,k]) dec(B[n,k]) + bias[n].
//
// Design for MI355X:
//  - 256 x 256 output tile per workgroup of 8 waves (two per SIMD); each wave
//    owns a 128 x 64 sub-tile: 4 x 2 v_mfma_f32_32x32x64_f8f6f4 per 64-deep K
//    step, 128 FP32 accumulators per lane.  Per K step the workgroup reads
//    96 KB of operand fragments from LDS for 8.4 MFLOP.
//  - Operands move HBM -> LDS with global_load_lds_dwordx4 (no VGPR staging):
//    each wave instruction fills 1 KB of LDS (16 rows of 64 bytes); every
//    lane picks the global 16-byte chunk that belongs at its LDS slot, which
//    implements an XOR swizzle of the 4 chunks of each row (conflict-free
//    ds_read_b128 of the MFMA fragments).
//  - Ping-pong between the two waves of each SIMD: waves 0-3 (rows 0-127)
//    and waves 4-7 (rows 128-255) run the same alternation of a load phase
//    (issue the next global->LDS loads, read the step's fragments from LDS)
//    and a compute phase (8 MFMAs), half a step apart, with one s_barrier
//    between phases.  In every phase one wave per SIMD feeds the MFMA pipe
//    while the other one talks to LDS, and each wave needs a single register
//    set of fragments.
//  - Four LDS stages (8 x 16 KB arrays) in a ring: the loads of step k+3 are
//    issued while step k is read.  Every barrier is preceded by an explicit
//    wait that lets the two younger steps' loads stay outstanding (a fenced
//    __syncthreads would drain them); scheduling barriers keep each phase's
//    instructions on its side.
//  - Tile order: blocks are dealt round-robin to the 8 XCDs; each XCD gets a
//    contiguous range of a grouped (GROUP_M M-tiles x all N-tiles) order, so
//    the 32 CUs of an XCD share A and B slices in their own L2.
//  - Epilogue: scales, bias and the bf16 / fp32 conversion, staged through
//    LDS so global stores are 16-byte row chunks.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int TM = 256, TN = 256, TK = 64;
constexpr int kWaves = 8, WAVES_N = 4;            // 2 x 4 waves
constexpr int kThreads = kWaves * 64;
constexpr int WTM = TM / (kWaves / WAVES_N);      // 128 rows per wave
constexpr int WTN = TN / WAVES_N;                 // 64 columns per wave
constexpr int MI = WTM / 32, NJ = WTN / 32;       // 4 x 2 MFMA tiles of 32 x 32
constexpr int kStageA = TM * TK, kStageB = TN * TK;  // 16 KB + 16 KB per stage
constexpr int kDmaA = kStageA / 1024 / kWaves;    // 2 DMA instructions per wave
constexpr int kDmaB = kStageB / 1024 / kWaves;    // 2
constexpr int GROUP_M = 4;

// Byte offset of 16-byte chunk c (0..3) of tile row r (64-byte rows); rows
// r, r+4, r+8, r+12 use four different chunk positions.
__device__ __forceinline__ int swz(int r, int c) { return r * TK + ((c ^ ((r >> 2) & 3)) << 4); }

template <int NDMA>
__device__ __forceinline__ void dma_tile(const uint8_t* base, const uint32_t (&voff)[NDMA], uint8_t* lds,
                                         int wave) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    __builtin_amdgcn_global_load_lds((gbl_void*)(base + voff[j]), (lds_void*)(lds + (wave * NDMA + j) * 1024),
                                     16, 0, 0);
}

// 32x32x64 operand: lane l holds row (l % 32) and the 32 K bytes
// [32 (l / 32), 32 (l / 32) + 32) of the step.
__device__ __forceinline__ i32x8 frag(const uint8_t* lds, int row, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, 2 * g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, 2 * g + 1));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

struct Frags {
  i32x8 a[MI];
  i32x8 b[NJ];
};

__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* la, const uint8_t* lb, int wm, int wn,
                                           int fr, int fg) {
#pragma unroll
  for (int j = 0; j < NJ; ++j) f.b[j] = frag(lb, wn * WTN + j * 32 + fr, fg);
#pragma unroll
  for (int i = 0; i < MI; ++i) f.a[i] = frag(la, wm * WTM + i * 32 + fr, fg);
}

template <int FA, int FB>
__device__ __forceinline__ void mfma_step(const Frags& f, f32x16 (&acc)[MI][NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.a[i], f.b[j], acc[i][j], FA, FB, 0, 0, 0, 0);
}

// Wait until at most N of this wave's vector-memory operations (the LDS
// loads of younger steps) are outstanding and all its LDS reads are done,
// then join the workgroup barrier.  No memory fence: the younger loads keep
// flying across the barrier.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N < 16, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0070 | N);  // vmcnt(N) expcnt(7) lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ uint32_t bf16_rne(float v) {
  const uint32_t u = __float_as_uint(v);
  if ((u & kAbsMask) > kInfBits) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int FA, int FB, bool BF16OUT>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_big(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ sa, int64_t era,
    const float* __restrict__ sb, int64_t erb, const void* __restrict__ bias, int bias_bf16,
    void* __restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_store) {
  __shared__ __attribute__((aligned(16))) uint8_t sA0[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sA2[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sA3[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sB2[kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sB3[kStageB];

  // ---- tile assignment: XCD-contiguous ranges of a grouped order
  const int T = tiles_m * tiles_n;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, loc = bid >> 3;
  const int q = T >> 3, rem = T & 7;
  const int logical = xcd * q + min(xcd, rem) + loc;
  const int group = GROUP_M * tiles_n;
  const int gidx = logical / group;
  const int first_m = gidx * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int within = logical - gidx * group;
  const int tile_m = first_m + within % gm;
  const int tile_n = within / gm;
  const int64_t m0 = static_cast<int64_t>(tile_m) * TM, n0 = static_cast<int64_t>(tile_n) * TN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int fr = lane & 31, fg = lane >> 5;

  // ---- per-lane DMA source offsets (rows past M / N are clamped: their
  // products land in accumulators that are never stored)
  uint32_t voa[kDmaA], vob[kDmaB];
  {
    const int c = (lane & 3) ^ ((lane >> 4) & 3);  // chunk stored at this lane's LDS slot
#pragma unroll
    for (int j = 0; j < kDmaA; ++j) {
      const int r = (wave * kDmaA + j) * 16 + (lane >> 2);
      voa[j] = static_cast<uint32_t>((min(m0 + r, M - 1) - m0) * lda + c * 16);
    }
#pragma unroll
    for (int j = 0; j < kDmaB; ++j) {
      const int r = (wave * kDmaB + j) * 16 + (lane >> 2);
      vob[j] = static_cast<uint32_t>((min(n0 + r, N - 1) - n0) * ldb + c * 16);
    }
  }
  const uint8_t* a_base = A + m0 * lda;
  const uint8_t* b_base = B + n0 * ldb;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // K is a multiple of 4 * TK, so every iteration below runs four full
  // steps.  Load phase of step k: issue the loads of step k+3 into stage
  // (k+3) % 4 (read by both groups during step k-1, so free; the index is
  // clamped to the last step, extra loads land in a stage nobody reads
  // again), read step k's fragments.  Group 1 starts one phase late; every
  // barrier waits for this wave's loads of step k+1 (two younger steps stay
  // in flight), which both groups need before group 0's next load phase.
  constexpr int kDmaStep = kDmaA + kDmaB;
  const int nk = static_cast<int>(K / TK);
  const int grp = wave >> 2;  // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  dma_tile<kDmaA>(a_base, voa, sA0, wave);
  dma_tile<kDmaB>(b_base, vob, sB0, wave);
  dma_tile<kDmaA>(a_base + TK, voa, sA1, wave);
  dma_tile<kDmaB>(b_base + TK, vob, sB1, wave);
  dma_tile<kDmaA>(a_base + 2 * TK, voa, sA2, wave);
  dma_tile<kDmaB>(b_base + 2 * TK, vob, sB2, wave);
  step_barrier<2 * kDmaStep>();
  if (grp == 1) step_barrier<2 * kDmaStep>();
  Frags f;
#define FP8RT_STEP(RA, RB, DA, DB, K3)                                        \
  {                                                                           \
    const int kn = min(K3, nk - 1);                                           \
    dma_tile<kDmaA>(a_base + kn * TK, voa, DA, wave);                         \
    dma_tile<kDmaB>(b_base + kn * TK, vob, DB, wave);                         \
    read_frags(f, RA, RB, wm, wn, fr, fg);                                    \
    step_barrier<2 * kDmaStep>();                                             \
    mfma_step<FA, FB>(f, acc);                                                \
    step_barrier<2 * kDmaStep>();                                             \
  }
  for (int kt = 0; kt < nk; kt += 4) {
    FP8RT_STEP(sA0, sB0, sA3, sB3, kt + 3)
    FP8RT_STEP(sA1, sB1, sA0, sB0, kt + 4)
    FP8RT_STEP(sA2, sB2, sA1, sB1, kt + 5)
    FP8RT_STEP(sA3, sB3, sA2, sB2, kt + 6)
  }
#undef FP8RT_STEP
  if (grp == 0) step_barrier<2 * kDmaStep>();
  step_barrier<0>();  // the clamped extra loads finish before the arrays are reused

  // ---- epilogue: each wave stages 8 KB row bands of its 128 x 64 result in
  // its own half of one stage array, then stores 16-byte row chunks.
  uint8_t* arr = (wave >> 1) == 0 ? sA0 : (wave >> 1) == 1 ? sA1 : (wave >> 1) == 2 ? sA2 : sA3;
  uint8_t* stage = arr + (wave & 1) * (kStageA / 2);
  const int64_t wrow0 = m0 + wm * WTM, wcol0 = n0 + wn * WTN;
  float sbv[NJ], bv[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int64_t col = min(wcol0 + j * 32 + fr, N - 1);
    sbv[j] = sb[col / erb];
    bv[j] = 0.0f;
    if (bias)
      bv[j] = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col]) << 16)
                        : static_cast<const float*>(bias)[col];
  }
  constexpr int ESZ = BF16OUT ? 2 : 4;
  constexpr int ROWS = (kStageA / 2) / (WTN * ESZ);  // 64 (bf16) or 32 (fp32) rows per pass
  constexpr int CHUNKS_PER_ROW = WTN * ESZ / 16;
  constexpr int ELEMS_PER_CHUNK = 16 / ESZ;
#pragma unroll
  for (int pass = 0; pass < WTM / ROWS; ++pass) {
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      if (i * 32 + 32 <= pass * ROWS || i * 32 >= (pass + 1) * ROWS) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        // 32x32 output layout: lane l holds column l % 32 and rows
        // 8 (e / 4) + 4 (l / 32) + (e % 4) of the sub-tile
        const int lrow = i * 32 + 8 * (e >> 2) + 4 * fg + (e & 3);
        const float sav = sa[min(wrow0 + lrow, M - 1) / era];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const float v = acc[i][j][e] * (sav * sbv[j]) + bv[j];
          const int off = ((lrow - pass * ROWS) * WTN + j * 32 + fr) * ESZ;
          if constexpr (BF16OUT) *reinterpret_cast<uint16_t*>(stage + off) = static_cast<uint16_t>(bf16_rne(v));
          else *reinterpret_cast<float*>(stage + off) = v;
        }
      }
    }
    __syncthreads();
    for (int ch = lane; ch < ROWS * CHUNKS_PER_ROW; ch += 64) {
      const int lrow = ch / CHUNKS_PER_ROW, cc = ch % CHUNKS_PER_ROW;
      const int64_t row = wrow0 + pass * ROWS + lrow;
      const int64_t col = wcol0 + cc * ELEMS_PER_CHUNK;
      if (row >= M || col >= N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * WTN * ESZ + cc * 16);
      char* dst = static_cast<char*>(Y) + (row * ldy + col) * ESZ;
      if (vec_store && col + ELEMS_PER_CHUNK <= N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        const char* src = reinterpret_cast<const char*>(&v);
        for (int e = 0; e < ELEMS_PER_CHUNK && col + e < N; ++e)
          for (int b = 0; b < ESZ; ++b) dst[e * ESZ + b] = src[e * ESZ + b];
      }
    }
    __syncthreads();
  }
}

}  // namespace

bool gemm_big_eligible(const GemmArgs& g) {
  return !g.pow2_mx && g.eca >= g.K && g.ecb >= g.K && g.K % (4 * TK) == 0 && g.M >= 128 &&
         g.N >= 128 && g.lda < (int64_t(1) << 23) && g.ldb < (int64_t(1) << 23);
}

hipError_t launch_gemm_big(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = static_cast<int>((g.M + TM - 1) / TM);
  const int tiles_n = static_cast<int>((g.N + TN - 1) / TN);
  const int esz = g.yt == FP8RT_BF16 ? 2 : 4;
  const int vec = ((g.ldy * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(g.y) & 15u) == 0);
  const dim3 grid(tiles_m * tiles_n);
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
#define FP8RT_BIG(FA, FB, OUT)                                                                         \
  hipLaunchKernelGGL((k_gemm_big<FA, FB, OUT>), grid, dim3(kThreads), 0, st, g.a, g.lda, g.b, g.ldb, \
                     g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, tiles_m, tiles_n, vec)
  if (g.fa == FP8RT_E4M3) {
    if (g.yt == FP8RT_BF16) FP8RT_BIG(0, 0, true);
    else FP8RT_BIG(0, 0, false);
  } else {
    if (g.yt == FP8RT_BF16) FP8RT_BIG(1, 0, true);
    else FP8RT_BIG(1, 0, false);
  }
#undef FP8RT_BIG
  return hipGetLastError();
}

}  // namespace fp8rt
