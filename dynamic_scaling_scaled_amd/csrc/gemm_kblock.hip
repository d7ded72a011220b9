// gemm_kblock.hip -- scaled FP8 GEMM with K-blocked scales for large shapes:
// 1 x 128 token-group scales on A and / or 128 x 128 block scales on B.
//
// Method: "FP8 formats and scaling for LLM inference", section "Per-channel
// and block scaling" (one scale per block of the tensor) together with
// section "The full precision contract of one FP8 GEMM" (FP32 accumulation):
//   Y[m,n] = sum_g s_a(m,g) s_b(n,g) sum_{k in g} dec(A[m,k]) dec(B[n,k]) + bias[n]
// with g running over the 128-deep K blocks.  A scale that does not change
// along K (per tensor, per row) is applied once in the epilogue instead.
//
// Design for MI355X:
//  - 256 x 256 output tile per workgroup of 8 waves (two per SIMD, which
//    hide each other's LDS and promotion latency); each wave owns 128 x 64
//    as 8 x 4 tiles of v_mfma_f32_16x16x128_f8f6f4.  One
//    128-deep LDS stage is exactly one scale block and one MFMA per tile, so
//    each tile's block partial comes out of a single MFMA started from zero
//    and is promoted into the FP32 accumulator right away with one FMA per
//    element by f = s_a(m, g) s_b(n-block, g).  The file is compiled with the
//    MFMA results in VGPRs (-amdgpu-mfma-vgpr-form) so the FMA reads them
//    directly; the result is the transposed tile, so a lane's 4 elements of
//    a tile share one output row and one factor.
//  - Operands move HBM -> LDS with buffer_load_dwordx4 ... lds (a uniform
//    descriptor per operand tile, the stage's K offset in an SGPR) into two
//    64 KB stages with 128-byte rows (full cache lines, XOR-swizzled by row / 2);
//    the loads of stage g+1 fly while stage g multiplies; B's fragments are
//    read at the stage start, A's one row tile ahead.  One s_barrier per stage.
//  - A's group scales are transposed once per call (k_transpose_scales) so a
//    stage's row scales are contiguous; B's block scales (two 128-column
//    blocks per tile) sit in LDS for all stages, one scalar per wave and stage.
//  - Tile order as in the per-tensor kernel (XCD-grouped); the epilogue
//    stages the result through LDS and stores 16-byte row chunks with the
//    hardware bf16 rounding.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int TM = 256, TN = 256;
constexpr int TKS = 128;                          // K bytes per LDS stage = one scale block
constexpr int kWaves = 8, WAVES_N = 4;            // 2 x 4 waves, two per SIMD
constexpr int kThreads = kWaves * 64;
constexpr int WTM = TM / (kWaves / WAVES_N);      // 128 rows per wave
constexpr int WTN = TN / WAVES_N;                 // 64 columns per wave
constexpr int MI = WTM / 16, NJ = WTN / 16;       // 8 x 4 MFMA tiles of 16 x 16
constexpr int kStageA = TM * TKS, kStageB = TN * TKS;  // 32 KB + 32 KB per stage
constexpr int kDmaA = kStageA / 1024 / kWaves;    // 4 DMA instructions per wave
constexpr int kDmaB = kStageB / 1024 / kWaves;    // 4
constexpr int GROUP_M = 4;
constexpr int kMaxStages = 2048;  // K / 128 limit (B block scales of a tile live in LDS)

__device__ __forceinline__ int swz(int r, int c) { return r * TKS + ((c ^ ((r >> 1) & 7)) << 4); }

template <int NDMA>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t rs, int soff, const uint32_t (&voff)[NDMA], uint8_t* lds,
                                        int wave) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + (wave * NDMA + j) * 1024), 16,
                                             static_cast<int>(voff[j]), soff, 0, 0);
}

__device__ __forceinline__ void* uniform_ptr(const void* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo);
}

// 16x16x128 operand: lane l holds row l % 16; the matrix core reads its
// first 16 bytes as K [16 g, +16) and the last 16 as K [64 + 16 g, +16) of the
// stage (g = l / 16): chunks g and g + 4.
__device__ __forceinline__ i32x8 frag(const uint8_t* lds, int row, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, g + 4));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS operations are done, then join the barrier.
template <int N>
__device__ __forceinline__ void step_barrier() {
  static_assert(N < 64, "vmcnt field");
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0070 | (N & 15));
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// Epilogue of one wave: lane l holds output row 16 i + (l % 16) and columns
// 16 j + 4 (l / 16) + (0..3) of its 128 x 64 tile; values are scaled (row
// factor sav, column vectors scol / sbias from LDS), staged in the wave's
// quarter of an LDS stage (16-byte chunks XOR-swizzled by row) and stored
// as 16-byte row chunks of ESZ-byte elements (2: bf16, 4: fp32); rows and
// columns at or past (M, N) are skipped.
template <int ESZ>
__device__ __forceinline__ void kb_store(const f32x4 (&acc)[MI][NJ], uint8_t* stage, const float* scol,
                                         const float* sbias, const float (&sav)[MI], int64_t wrow0, int64_t wcol0,
                                         int64_t M, int64_t N, void* __restrict__ Y, int64_t ldy, int vec_store,
                                         int wn, int fr, int fq, int lane) {
  constexpr int RB = WTN * ESZ;                 // staged row bytes: 128 or 256
  constexpr int CPR = RB / 16;                  // 16-byte chunks per row: 8 or 16
  constexpr int ROWS = (kStageA / 4) / RB;      // rows per pass: 64 or 32
  constexpr int IPP = ROWS / 16;                // MFMA row tiles per pass: 4 or 2
  constexpr int EPC = 16 / ESZ;
#pragma unroll
  for (int pass = 0; pass < MI / IPP; ++pass) {
#pragma unroll
    for (int ii = 0; ii < IPP; ++ii) {
      const int i = pass * IPP + ii;
      const int lrow = ii * 16 + fr;
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = j * 16 + 4 * fq;
        const f32x4 scv = *reinterpret_cast<const f32x4*>(&scol[wn * WTN + c]);
        const f32x4 biv = *reinterpret_cast<const f32x4*>(&sbias[wn * WTN + c]);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * (sav[i] * scv[r]) + biv[r];
        const int byte = c * ESZ;
        const int chunk = (byte >> 4) ^ (lrow & (CPR - 1));
        uint8_t* dst = stage + lrow * RB + (chunk << 4) + (byte & 15);
        if constexpr (ESZ == 2) {
          *reinterpret_cast<bf16x4*>(dst) = __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4);
        } else {
          *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
      }
    }
    __syncthreads();
    for (int ch = lane; ch < ROWS * CPR; ch += 64) {
      const int lrow = ch / CPR, cc = ch % CPR;
      const int64_t row = wrow0 + pass * ROWS + lrow;
      const int64_t col = wcol0 + cc * EPC;
      if (row >= M || col >= N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * RB + ((cc ^ (lrow & (CPR - 1))) << 4));
      char* dst = static_cast<char*>(Y) + (row * ldy + col) * ESZ;
      if (vec_store && col + EPC <= N) {
        *reinterpret_cast<u32x4*>(dst) = v;
      } else {
        const char* src = reinterpret_cast<const char*>(&v);
        for (int e = 0; e < EPC && col + e < N; ++e)
          for (int b = 0; b < ESZ; ++b) dst[e * ESZ + b] = src[e * ESZ + b];
      }
    }
    __syncthreads();
  }
}

// sat: A's group scales transposed to [K / 128][M] (null: A scale constant
// along K, taken from sa in the epilogue).  sbk: B's block scales
// [ceil(N / erb)][K / 128] (null: constant along K, from sb in the epilogue).
template <int FA, int FB, bool BF16OUT, bool AKB, bool BKB>
__global__ __launch_bounds__(kThreads, 2) void k_gemm_kblock(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb, int64_t M,
    int64_t N, int64_t K, const float* __restrict__ sat, const float* __restrict__ sa, int64_t era,
    const float* __restrict__ sbk, const float* __restrict__ sb, int64_t erb, const void* __restrict__ bias,
    int bias_bf16, void* __restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_store, int64_t Mp,
    int t_main, int split, int ns_part, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint8_t sA0[kStageA];
  __shared__ __attribute__((aligned(16))) float sSa0[TM];   // A row scales of the stage in sA0
  __shared__ __attribute__((aligned(16))) float sSa1[TM];
  __shared__ float sSb[2][kMaxStages];                      // B block scales of every stage (2 blocks)
  __shared__ __attribute__((aligned(16))) uint8_t sA1[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[kStageB];

  // Blocks below t_main take whole tiles of the grouped order, dealt to the
  // XCDs in contiguous ranges; the rest are split-K units: unit u runs the
  // stages [(u % split) ns_part, +ns_part) of tile t_main + u / split and
  // writes its promoted FP32 sums to part[u] (launch_split_reduce finishes).
  const int bid = blockIdx.x;
  const bool unit = bid >= t_main;
  int logical, s0 = 0;
  if (!unit) {
    const int xcd = bid & 7, loc = bid >> 3;
    const int q = t_main >> 3, rem = t_main & 7;
    logical = xcd * q + min(xcd, rem) + loc;
  } else {
    const int u = bid - t_main;
    logical = t_main + u / split;
    s0 = (u % split) * ns_part;
  }
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

  uint32_t voa[kDmaA], vob[kDmaB];
#pragma unroll
  for (int j = 0; j < kDmaA; ++j) {
    const int r = (wave * kDmaA + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    voa[j] = static_cast<uint32_t>((min(m0 + r, M - 1) - m0) * lda + c * 16);
  }
#pragma unroll
  for (int j = 0; j < kDmaB; ++j) {
    const int r = (wave * kDmaB + j) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r >> 1) & 7);
    vob[j] = static_cast<uint32_t>((min(n0 + r, N - 1) - n0) * ldb + c * 16);
  }
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(A + m0 * lda), 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(B + n0 * ldb), 0, -1, 0x00020000);

  f32x4 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ns = static_cast<int>(K / TKS);  // even
  const int nsl = unit ? ns_part : ns;        // stages this block runs (even), from s0
  const int64_t wrow0 = m0 + wm * WTM;
  const int fr = lane & 15, fq = lane >> 4;
  // B block scales of this tile's block row for every stage, once, in LDS.
  if constexpr (BKB) {
    for (int hb = 0; hb < 2; ++hb) {
      const float* sbk_row = sbk + (min(n0 + hb * 128, N - 1) / erb) * ns;
      for (int i = t; i < ns; i += kThreads) sSb[hb][i] = sbk_row[i];
    }
  }
  // A row scales of a stage: one DMA of the 256 contiguous row scales of the
  // transposed, row-padded table (every wave issues it; the copies carry the
  // same bytes).
  auto sa_dma = [&](int st, float* dst) {
    if constexpr (AKB) {
      const int stc = min(st, ns - 1);
      __builtin_amdgcn_global_load_lds((gbl_void*)(sat + stc * Mp + m0 + lane * 4), (lds_void*)dst, 16, 0, 0);
    }
  };
  // One stage from LDS: B fragments first, A one row tile ahead; each tile's
  // partial is a single MFMA from zero.  The promotion of row tile i's
  // partials (acc += f p) is issued among the MFMAs of row tile i + 1, so
  // the FMAs never wait on an MFMA that has just started; the last row
  // tile's partials are promoted among the next stage's first MFMAs.
  f32x4 pend[NJ];   // partials of the previous row tile, not yet promoted
  float fpend = 0.0f;
  auto stage_mma = [&](const uint8_t* la, const uint8_t* lb, const float* ssa, int st, bool first) {
    const float fb = BKB ? sSb[(wn * WTN) / 128][st] : 1.0f;
    i32x8 bfr[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) bfr[j] = frag(lb, wn * WTN + j * 16 + fr, fq);
    i32x8 afr = frag(la, wm * WTM + fr, fq);
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const i32x8 cur = afr;
      if (i + 1 < MI) afr = frag(la, wm * WTM + (i + 1) * 16 + fr, fq);
      f32x4 p[NJ];
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        p[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], cur, f32x4{0.f, 0.f, 0.f, 0.f}, FB, FA,
                                                               0, 0, 0, 0);
        // promote the previous row tile (of this stage, or the last of the previous one)
        const int ip = i == 0 ? MI - 1 : i - 1;
        if (i > 0 || !first) {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[ip][j][e] = fmaf(fpend, pend[j][e], acc[ip][j][e]);
        }
      }
#pragma unroll
      for (int j = 0; j < NJ; ++j) pend[j] = p[j];
      fpend = (AKB ? ssa[wm * WTM + i * 16 + fr] : 1.0f) * fb;
      __builtin_amdgcn_sched_barrier(0);  // keep each row tile's MFMAs with the previous tile's FMAs
    }
  };
  auto drain = [&]() {
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[MI - 1][j][e] = fmaf(fpend, pend[j][e], acc[MI - 1][j][e]);
  };

  sa_dma(s0, sSa0);
  dma_buf<kDmaA>(ra, s0 * TKS, voa, sA0, wave);
  dma_buf<kDmaB>(rb, s0 * TKS, vob, sB0, wave);
  step_barrier<0>();  // stage s0, its scales and the B scale table landed
  // Stage st (in arrays X): issue the loads of stage st+1 into the other
  // arrays (free: the previous stage ended with a barrier), multiply and
  // promote stage st, wait for everything issued.
#define FP8RT_KSTAGE(LA, LB, LS, DA, DB, DS, ST, FIRST)                        \
  {                                                                           \
    const int kn = s0 + min(ST + 1, nsl - 1);                                 \
    sa_dma(kn, DS);                                                           \
    dma_buf<kDmaA>(ra, kn * TKS, voa, DA, wave);                              \
    dma_buf<kDmaB>(rb, kn * TKS, vob, DB, wave);                              \
    stage_mma(LA, LB, LS, s0 + ST, FIRST);                                    \
    step_barrier<0>();                                                        \
  }
  FP8RT_KSTAGE(sA0, sB0, sSa0, sA1, sB1, sSa1, 0, true)
  FP8RT_KSTAGE(sA1, sB1, sSa1, sA0, sB0, sSa0, 1, false)
  for (int st = 2; st < nsl; st += 2) {
    FP8RT_KSTAGE(sA0, sB0, sSa0, sA1, sB1, sSa1, st, false)
    FP8RT_KSTAGE(sA1, sB1, sSa1, sA0, sB0, sSa0, st + 1, false)
  }
#undef FP8RT_KSTAGE
  drain();

  // ---- epilogue: lane l holds output row 16 i + (l % 16) and columns
  // 16 j + 4 (l / 16) + (0..3) of the wave tile.
  __shared__ __attribute__((aligned(16))) float sCol[2][TN];
  if (t < TN) {
    const int64_t col = min(n0 + t, N - 1);
    sCol[0][t] = (BKB || unit) ? 1.0f : sb[erb == 1 ? col : 0];
    float bvv = 0.0f;
    if (bias && !unit)
      bvv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col]) << 16)
                      : static_cast<const float*>(bias)[col];
    sCol[1][t] = bvv;
  }
  __syncthreads();
  uint8_t* stage = (wave < 4 ? sA0 : sA1) + (wave & 3) * (kStageA / 4);
  float sav[MI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
    sav[i] = (AKB || unit) ? 1.0f : sa[era == 1 ? min(wrow0 + i * 16 + fr, M - 1) : 0];
  if (unit) {
    // raw sums of the unit's stages, the whole 256 x 256 tile, FP32
    kb_store<4>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wm * WTM, wn * WTN, TM, TN,
                part + static_cast<int64_t>(bid - t_main) * (TM * TN), TN, 1, wn, fr, fq, lane);
  } else {
    kb_store<BF16OUT ? 2 : 4>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wrow0, n0 + wn * WTN, M, N, Y, ldy,
                              vec_store, wn, fr, fq, lane);
  }
}

// out[g * Mp + m] = s[m * ng + g]: the group scales of A with the K-block
// index outermost and rows padded to Mp, so one stage's row scales of a tile
// are 256 contiguous floats (the padding rows are never read for stored
// outputs).
__global__ __launch_bounds__(256) void k_transpose_scales(const float* __restrict__ s, int64_t M, int64_t ng,
                                                          int64_t Mp, float* __restrict__ out) {
  __shared__ float tile[32][33];
  const int64_t m_base = static_cast<int64_t>(blockIdx.x) * 32, g_base = static_cast<int64_t>(blockIdx.y) * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int64_t m = m_base + r, g = g_base + tx;
    if (m < M && g < ng) tile[r][tx] = s[m * ng + g];
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int64_t g = g_base + r, m = m_base + tx;
    if (m < M && g < ng) out[g * Mp + m] = tile[tx][r];
  }
}

}  // namespace

bool gemm_kblock_eligible(const GemmArgs& g) {
  if (g.pow2_mx || g.K % (2 * TKS) != 0 || g.K / TKS > kMaxStages || g.M < 65 || g.N < 128) return false;
  if (g.lda >= (int64_t(1) << 23) || g.ldb >= (int64_t(1) << 23)) return false;
  const bool a_kb = g.eca < g.K, b_kb = g.ecb < g.K;
  if (!a_kb && !b_kb) return false;
  if (a_kb && !(g.era == 1 && g.eca == TKS)) return false;
  if (b_kb && !(g.erb % 128 == 0 && g.ecb == TKS)) return false;
  if (!a_kb && !(g.era == 1 || g.era >= g.M)) return false;
  if (!b_kb && !(g.erb == 1 || g.erb >= g.N)) return false;
  return true;
}

size_t gemm_kblock_required_scratch(const GemmArgs& g) {
  if (!(g.eca < g.K)) return 0;
  const int64_t Mp = (g.M + TM - 1) / TM * static_cast<int64_t>(TM);
  return (static_cast<size_t>(Mp * (g.K / TKS)) * sizeof(float) + 255) & ~size_t(255);  // A's scales, transposed
}

hipError_t launch_gemm_kblock(const GemmArgs& g, hipStream_t st) {
  const int tiles_m = static_cast<int>((g.M + TM - 1) / TM);
  const int tiles_n = static_cast<int>((g.N + TN - 1) / TN);
  const int esz = g.yt == FP8RT_BF16 ? 2 : 4;
  const int vec = ((g.ldy * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(g.y) & 15u) == 0);
  const bool a_kb = g.eca < g.K, b_kb = g.ecb < g.K;
  const int64_t ns = g.K / TKS;
  const int64_t Mp = tiles_m * static_cast<int64_t>(TM);  // rows padded to whole tiles
  const int T = tiles_m * tiles_n;
  // Split along K, as in the per-tensor kernel: a grid filling at most half
  // the CUs splits every tile (up to 8 parts), a ragged last wave at most
  // half full its tiles (up to 4); each part an even number of stages.  The
  // scratch holds A's transposed scales, then the parts (256 KB per part
  // and tile).
  const size_t sat_bytes = gemm_kblock_required_scratch(g);
  int t_main = T, split = 1, ns_part = 0;
  size_t part_total = 0;
  {
    const int cus = device_cus();
    const bool small = 2 * T <= cus;
    const int rem = small ? T : T % cus;
    if (small || (T > cus && rem > 0 && 2 * rem <= cus)) {
      const size_t part_bytes = static_cast<size_t>(rem) * TM * TN * sizeof(float);
      int sp = std::min(cus / rem, small ? 8 : 4);
      if (g.fixed_scratch)
        sp = static_cast<int>(std::min<size_t>(
            sp, g.fixed_scratch_bytes > sat_bytes ? (g.fixed_scratch_bytes - sat_bytes) / part_bytes : 0));
      while (sp > 1 && ns % (2 * sp) != 0) --sp;
      if (sp > 1) {
        split = sp;
        t_main = T - rem;
        ns_part = static_cast<int>(ns / sp);
        part_total = part_bytes * sp;
      }
    }
  }
  uint8_t* scratch = nullptr;
  if (sat_bytes + part_total > 0) {
    void* p = nullptr;
    hipError_t e = gemm_scratch(g, st, sat_bytes + part_total, &p);
    if (e != hipSuccess) return e;
    scratch = static_cast<uint8_t*>(p);
  }
  float* sat = a_kb ? reinterpret_cast<float*>(scratch) : nullptr;
  float* part = split > 1 ? reinterpret_cast<float*>(scratch + sat_bytes) : nullptr;
  if (a_kb)
    hipLaunchKernelGGL(k_transpose_scales,
                       dim3(static_cast<unsigned>((g.M + 31) / 32), static_cast<unsigned>((ns + 31) / 32)),
                       dim3(256), 0, st, g.sa, g.M, ns, Mp, sat);
  const float* sbk = b_kb ? g.sb : nullptr;
  const dim3 grid(static_cast<unsigned>(t_main + (T - t_main) * split));
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
#define FP8RT_KB(FA, FB, OUT, AK, BK)                                                                         \
  hipLaunchKernelGGL((k_gemm_kblock<FA, FB, OUT, AK, BK>), grid, dim3(kThreads), 0, st, g.a, g.lda, g.b, g.ldb, \
                     g.M, g.N, g.K, sat, g.sa, g.era, sbk, g.sb, g.erb, g.bias, bb, g.y, g.ldy, tiles_m, tiles_n,  \
                     vec, Mp, t_main, split, ns_part, part)
#define FP8RT_KB_OUT(FA, FB, AK, BK)                    \
  if (g.yt == FP8RT_BF16) FP8RT_KB(FA, FB, true, AK, BK); \
  else FP8RT_KB(FA, FB, false, AK, BK);
#define FP8RT_KB_KIND(FA, FB)                                            \
  if (a_kb && b_kb) { FP8RT_KB_OUT(FA, FB, true, true) }                \
  else if (a_kb) { FP8RT_KB_OUT(FA, FB, true, false) }                  \
  else { FP8RT_KB_OUT(FA, FB, false, true) }
  if (g.fa == FP8RT_E4M3) {
    FP8RT_KB_KIND(0, 0)
  } else {
    FP8RT_KB_KIND(1, 0)
  }
#undef FP8RT_KB_KIND
#undef FP8RT_KB_OUT
#undef FP8RT_KB
  if (split > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // scales constant along K were left to the epilogue: the reduction applies them
    return launch_split_reduce(g, st, part, t_main, split, tiles_m, tiles_n, a_kb ? nullptr : g.sa,
                               b_kb ? nullptr : g.sb, vec);
  }
  return hipGetLastError();
}

}  // namespace fp8rt
