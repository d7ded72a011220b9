// gemm_big.hip -- the large-shape scaled FP8 GEMM for gfx950 (per-tensor and
// per-row / per-output-channel scales applied in the epilogue).
//
// Method: "FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM": Y ~ s_x s_w (X8 W8) with FP32
// accumulation, BF16/FP32 output and bias; section "Per-channel and block
// scaling" for per-row scales.  Y[m,n] = s_a(m) s_b(n) sum_k dec(A[m,k]) dec(B[n,k]) + bias[n].
//
// Design for MI355X:
//  - 256 x 256 output tile per workgroup of 4 waves (one per SIMD); each wave
//    owns a 128 x 128 sub-tile: 4 x 4 v_mfma_f32_32x32x64_f8f6f4 per 64-deep
//    K sub-step, 256 FP32 accumulators per lane held in AGPRs.
//  - Two LDS stages of 128 K bytes (64 KB each).  A stage row is 128 bytes,
//    a whole cache line, so every vector-memory request moves a full line
//    (64-byte half rows doubled the L1->L2 request count and stalled the
//    address path).  Operands move HBM -> LDS with global_load_lds_dwordx4
//    (no VGPR staging): one instruction fills 8 rows; each lane picks the
//    global chunk that belongs at its LDS slot, an XOR swizzle of the 8
//    chunks of a row by (row / 2) that makes the ds_read_b128 fragment reads
//    conflict-free on the 64-bank LDS.
//  - Software pipeline over sub-steps, with two fragment register sets P/Q:
//    even sub-step 2j multiplies P (stage j, K bytes 0-63) while it reads
//    stage j, K bytes 64-127 into Q, then waits for stage j+1 and joins one
//    s_barrier (stage j is then free); odd sub-step 2j+1 multiplies Q while
//    it refills stage j's arrays with stage j+2 and reads stage j+1 into P.
//    One barrier per 128-deep stage; scheduling groups interleave the LDS
//    reads and the loads between the MFMAs.
//  - Tile order: blocks are dealt round-robin to the 8 XCDs; each XCD gets a
//    contiguous range of a grouped (GROUP_M M-tiles x all N-tiles) order, so
//    the 32 CUs of an XCD share A and B slices in their own L2.
//  - The MFMA computes the transposed tile (B as the first operand), so a
//    lane ends with 4 consecutive output columns of one row: the epilogue
//    applies the scales and bias with 4-wide LDS reads of the block's column
//    vectors, converts with the hardware bf16 conversion (round to nearest
//    even), stages 8- or 16-byte pieces in LDS and stores 16-byte row chunks.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

constexpr int TM = 256, TN = 256;
constexpr int TKS = 128;                          // K bytes per LDS stage (full 128-byte rows)
constexpr int TK = 64;                            // K per MFMA sub-step
constexpr int kWaves = 4, WAVES_N = 2;            // 2 x 2 waves
constexpr int kThreads = kWaves * 64;
constexpr int WTM = TM / (kWaves / WAVES_N);      // 128 rows per wave
constexpr int WTN = TN / WAVES_N;                 // 128 columns per wave
constexpr int MI = WTM / 32, NJ = WTN / 32;       // 4 x 4 MFMA tiles of 32 x 32
constexpr int kStageA = TM * TKS, kStageB = TN * TKS;  // 32 KB + 32 KB per stage
constexpr int kDmaA = kStageA / 1024 / kWaves;    // 8 DMA instructions per wave
constexpr int kDmaB = kStageB / 1024 / kWaves;    // 8
constexpr int GROUP_M = 4;

// Byte offset of 16-byte chunk c (0..7) of stage row r (128-byte rows).
__device__ __forceinline__ int swz(int r, int c) { return r * TKS + ((c ^ ((r >> 1) & 7)) << 4); }

template <int NDMA>
__device__ __forceinline__ void dma_tile(const uint8_t* base, const uint32_t (&voff)[NDMA], uint8_t* lds,
                                         int wave) {
#pragma unroll
  for (int j = 0; j < NDMA; ++j)
    __builtin_amdgcn_global_load_lds((gbl_void*)(base + voff[j]), (lds_void*)(lds + (wave * NDMA + j) * 1024),
                                     16, 0, 0);
}

// 32x32x64 operand of sub-step h: lane l holds row (l % 32); the matrix
// core reads the lane's first 16 bytes as K [16 g, 16 g + 16) and the last 16
// as K [32 + 16 g, 48 + 16 g) of the sub-step, g = l / 32, so the lane loads
// chunks 4 h + g and 4 h + g + 2 and K order in LDS equals the hardware's
// (which the 32-element scale blocks of the MX path rely on).
__device__ __forceinline__ i32x8 frag(const uint8_t* lds, int row, int c0) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, c0));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, c0 + 2));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

struct Frags {
  i32x8 a[MI];
  i32x8 b[NJ];
};

__device__ __forceinline__ void read_frags(Frags& f, const uint8_t* la, const uint8_t* lb, int wm, int wn,
                                           int fr, int c0) {
#pragma unroll
  for (int i = 0; i < MI; ++i) f.a[i] = frag(la, wm * WTM + i * 32 + fr, c0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) f.b[j] = frag(lb, wn * WTN + j * 32 + fr, c0);
}

// One 64-deep sub-step of MFMAs.  The first operand is B, so the result is
// the transposed tile.  With MX, each lane passes the E8M0 scales of its own
// row and 32-element K block; OPSEL picks the byte of the sub-step.
template <int FA, int FB, bool MX, int OPSEL>
__device__ __forceinline__ void mfma_step(const Frags& f, f32x16 (&acc)[MI][NJ], const uint32_t (&xa)[MI],
                                          const uint32_t (&xb)[NJ]) {
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      if constexpr (MX)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], FB, FA, OPSEL,
                                                                    xb[j], OPSEL, xa[i]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f.b[j], f.a[i], acc[i][j], FB, FA, 0, 0, 0, 0);
    }
}

// Wait until at most N of this wave's vector-memory operations (the loads of
// the younger stage) are outstanding and all its LDS operations are done,
// then join the workgroup barrier.  No memory fence: younger loads keep
// flying across the barrier.
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

// Tile (tile_m, tile_n) of position `logical` in the grouped order: groups of
// GROUP_M M-tiles by all N-tiles, M-tile fastest inside a group.
__device__ __forceinline__ void tile_of(int logical, int tiles_m, int tiles_n, int& tile_m, int& tile_n) {
  const int group = GROUP_M * tiles_n;
  const int gidx = logical / group;
  const int first_m = gidx * GROUP_M;
  const int gm = min(GROUP_M, tiles_m - first_m);
  const int within = logical - gidx * group;
  tile_m = first_m + within % gm;
  tile_n = within / gm;
}

// Epilogue of one block: lane l holds output row 32 i + (l % 32) and, per
// group g = e / 4, the 4 consecutive columns 32 j + 8 g + 4 (l / 32) + (e % 4)
// of its wave tile (the MFMA computed the transposed tile).  Values are
// scaled (row factor sav, column vectors scol / bias from LDS), converted,
// staged in the wave's 32 KB of LDS (16-byte chunks XOR-swizzled by row) and
// stored as 16-byte row chunks; rows / columns at or past (M, N) are skipped.
// FP8 output (OUT kOutE4M3 / kOutE5M2): codes of v * rq with the quantize
// kernels' saturating RNE cast; the lane's max |v| and counters accumulate
// into mb / sat_l / under_l.  Saturation, underflow and NaN are rare, so a
// group of 4 is screened first (its max and min |v| against conservative
// thresholds, one unordered compare per pair) and the exact per-element work
// runs only for a group that may need it.  EDGE: the wave tile may reach past
// (M, N), so elements are tested before they count.
template <int OUT, bool EDGE = true>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[MI][NJ], uint8_t* stage, const float* scol,
                                           const float* sbias, const float (&sav)[MI], int64_t wrow0, int64_t wcol0,
                                           int64_t M, int64_t N, void* __restrict__ Y, int64_t ldy, int vec_store,
                                           int wn, int fr, int fg, int lane, float rq, uint32_t& mb, uint32_t& sat_l,
                                           uint32_t& under_l) {
  // Screen thresholds on |v| bit patterns.  |f| = fl(|v| |rq|) is monotonic
  // in |v|: no element with |v| <= kMax / |rq| (two ulps below, absorbing the
  // quotient's rounding) saturates, and none with |v| > kZeroEdge / |rq| (two
  // ulps above) underflows.  NaN patterns exceed every finite threshold; a
  // zero, infinite or NaN rq screens nothing.
  uint32_t thr_sat = 0u, thr_und = ~0u;
  if constexpr (OUT >= kOutE4M3) {
    constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
    const float arq = fabsf(rq);
    if (arq > 0.0f && arq <= FLT_MAX) {
      const uint32_t ts = __float_as_uint(Fmt<F>::kMax / arq), tu = __float_as_uint(Fmt<F>::kZeroEdge / arq);
      thr_sat = ts > 2u ? ts - 2u : 0u;
      thr_und = tu + 2u;
    }
  }
  constexpr int ESZ = OUT == kOutF32 ? 4 : OUT == kOutBF16 ? 2 : 1;
  constexpr int RB = WTN * ESZ;                 // staged row bytes: 128, 256 or 512
  constexpr int CPR = RB / 16;                  // 16-byte chunks per row: 8, 16 or 32
  constexpr int SWM = (CPR < 16 ? CPR : 16) - 1;  // chunk swizzle mask
  constexpr int ROWS = kStageA / RB < WTM ? kStageA / RB : WTM;  // rows per pass: 128 or 64
  constexpr int IPP = ROWS / 32;                // MFMA row tiles per pass: 4 or 2
  constexpr int EPC = 16 / ESZ;                 // elements per chunk
#pragma unroll
  for (int pass = 0; pass < MI / IPP; ++pass) {
#pragma unroll
    for (int ii = 0; ii < IPP; ++ii) {
      const int i = pass * IPP + ii;
      const int lrow = ii * 32 + fr;            // row within the pass
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = j * 32 + g * 8 + 4 * fg;  // first of 4 columns within the wave tile
          const f32x4 scv = *reinterpret_cast<const f32x4*>(&scol[wn * WTN + c]);
          const f32x4 biv = *reinterpret_cast<const f32x4*>(&sbias[wn * WTN + c]);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * g + r] * (sav[i] * scv[r]) + biv[r];
          const int byte = c * ESZ;               // byte offset of the 4 values in the row
          const int chunk = (byte >> 4) ^ (lrow & SWM);
          uint8_t* dst = stage + lrow * RB + (chunk << 4) + (byte & 15);
          if constexpr (OUT == kOutBF16) {
            const bf16x4 h = __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4);
            *reinterpret_cast<bf16x4*>(dst) = h;
          } else if constexpr (OUT == kOutF32) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
          } else {
            constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
            // statistics of stored outputs only: the tile's rows / columns
            // past (M, N) hold clamped or unscaled padding
            const bool row_in = !EDGE || wrow0 + pass * ROWS + lrow < M;
            float f[4];
            uint32_t ab[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              f[r] = v[r] * rq;
              const bool in = !EDGE || (row_in && wcol0 + c + r < N);
              ab[r] = in ? (__float_as_uint(v[r]) & kAbsMask) : 0u;  // 0: not counted
            }
            const uint32_t gmax = max(max(ab[0], ab[1]), max(ab[2], ab[3]));
            const uint32_t gmin = min(min(ab[0], ab[1]), min(ab[2], ab[3]));
            mb = max(mb, gmax);
            if (gmax > thr_sat || gmin <= thr_und) {
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                sat_l += (ab[r] != 0u && fabsf(f[r]) > Fmt<F>::kMax) ? 1u : 0u;
                under_l += (ab[r] != 0u && fabsf(f[r]) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
              }
            }
            uint32_t w = cvt4<F>(f[0], f[1], f[2], f[3]);
            if (__builtin_isunordered(f[0], f[1]) || __builtin_isunordered(f[2], f[3]))
              w = cvt4_nan<F>(f[0], f[1], f[2], f[3]);
            *reinterpret_cast<uint32_t*>(dst) = w;
            // opaque per group: otherwise the tile's updates are
            // reassociated into trees that keep every accumulator live
            asm volatile("" : "+v"(mb), "+v"(sat_l), "+v"(under_l));
          }
        }
    }
    __syncthreads();
    for (int ch = lane; ch < ROWS * CPR; ch += 64) {
      const int lrow = ch / CPR, cc = ch % CPR;
      const int64_t row = wrow0 + pass * ROWS + lrow;
      const int64_t col = wcol0 + cc * EPC;
      if (row >= M || col >= N) continue;
      const u32x4 v = *reinterpret_cast<const u32x4*>(stage + lrow * RB + ((cc ^ (lrow & SWM)) << 4));
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

// MX: power-of-two 1x32 scales applied inside the MFMA.  xpa / xpb hold the
// E8M0 exponents repacked by k_pack_e8m0 as [row / 32][stage][row % 32] dwords
// (byte b = K block 4 stage + b).
template <int FA, int FB, int OUT, bool MX>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_big(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ sa, int64_t era,
    const float* __restrict__ sb, int64_t erb, const void* __restrict__ bias, int bias_bf16,
    void* __restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_store,
    const uint32_t* __restrict__ xpa, const uint32_t* __restrict__ xpb, int t_main, int split, int ns_part,
    float* __restrict__ part, const float* __restrict__ sy, const float* __restrict__ ry,
    BlockPartial* __restrict__ ypart) {
  __shared__ __attribute__((aligned(16))) uint8_t sA0[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sA1[kStageA];
  __shared__ __attribute__((aligned(16))) uint8_t sB0[kStageB];
  __shared__ __attribute__((aligned(16))) uint8_t sB1[kStageB];

  // Blocks below t_main take whole tiles [0, t_main) of the grouped order;
  // the rest are split-K units: unit u computes K stages
  // [(u % split) ns_part, +ns_part) of tile t_main + u / split and writes its
  // raw FP32 sums to part[u] (k_split_reduce finishes those tiles).
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
  int tile_m, tile_n;
  tile_of(logical, tiles_m, tiles_n, tile_m, tile_n);
  const int64_t m0 = static_cast<int64_t>(tile_m) * TM, n0 = static_cast<int64_t>(tile_n) * TN;

  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int fr = lane & 31, fg = lane >> 5;

  // DMA j of a wave fills stage rows (wave * NDMA + j) * 8 + (lane / 8); the
  // lane's LDS slot is chunk lane % 8 of that row, which holds global chunk
  // slot ^ ((row >> 1) & 7).
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
  const uint8_t* a_base = A + m0 * lda + static_cast<int64_t>(s0) * TKS;
  const uint8_t* b_base = B + n0 * ldb + static_cast<int64_t>(s0) * TKS;

  f32x16 acc[MI][NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  constexpr int kDmaStage = kDmaA + kDmaB;  // 16
  const int ns_all = static_cast<int>(K / TKS);  // even
  const int ns = unit ? ns_part : ns_all;         // stages this block runs (even)
  const int c_lo = fg, c_hi = 4 + fg;  // first chunk of sub-step 0 / 1
  // MX: per stage the workgroup needs the E8M0 dwords of 8 A and 8 B row
  // groups (256 bytes each, 4 KB): each wave copies 1 KB of them into LDS
  // with one DMA (waves 0/1: A groups 0-3 / 4-7, waves 2/3: B).  Lane l of
  // an MFMA reads the dword of its row and K-half l / 32, whose bytes 0 and 2
  // are the blocks of sub-steps 0 and 1.
  __shared__ __attribute__((aligned(16))) uint32_t sX0[2][8 * 64];
  __shared__ __attribute__((aligned(16))) uint32_t sX1[2][8 * 64];
  uint32_t xa0[MI] = {}, xb0[NJ] = {}, xa1[MI] = {}, xb1[NJ] = {};  // even / odd stages
  const uint32_t* xsrc = nullptr;
  uint32_t xoff = 0;
  if constexpr (MX) {
    // lane l copies 16 bytes of row group 4 (wave & 1) + l / 16
    const bool opb = wave >= 2;
    const int64_t gmax = (opb ? (N - 1) : (M - 1)) / 32;
    const int64_t g = min((opb ? n0 : m0) / 32 + 4 * (wave & 1) + (lane >> 4), gmax);
    xsrc = opb ? xpb : xpa;
    xoff = static_cast<uint32_t>((g * ns_all + s0) * 64 + (lane & 15) * 4);
  }
  auto sc_dma = [&](int st, uint32_t (&dst)[2][8 * 64]) {
    if constexpr (MX) {
      const int64_t stc = min(st, ns - 1);
      __builtin_amdgcn_global_load_lds((gbl_void*)(xsrc + xoff + stc * 64),
                                       (lds_void*)(&dst[wave >> 1][(wave & 1) * 256]), 16, 0, 0);
    }
  };
  auto sc_read = [&](const uint32_t (&src)[2][8 * 64], uint32_t (&xa)[MI], uint32_t (&xb)[NJ]) {
    if constexpr (MX) {
#pragma unroll
      for (int i = 0; i < MI; ++i) xa[i] = src[0][(wm * MI + i) * 64 + fg * 32 + fr];
#pragma unroll
      for (int j = 0; j < NJ; ++j) xb[j] = src[1][(wn * NJ + j) * 64 + fg * 32 + fr];
    }
  };
  sc_dma(0, sX0);
  sc_dma(1, sX1);
  dma_tile<kDmaA>(a_base, voa, sA0, wave);
  dma_tile<kDmaB>(b_base, vob, sB0, wave);
  dma_tile<kDmaA>(a_base + TKS, voa, sA1, wave);
  dma_tile<kDmaB>(b_base + TKS, vob, sB1, wave);
  step_barrier<kDmaStage>();  // stage 0 (and the scales, issued first) landed
  Frags fp, fq;
  read_frags(fp, sA0, sB0, wm, wn, fr, c_lo);
  sc_read(sX0, xa0, xb0);
  // Sub-step 2j: MFMAs on P (stage j, first half), read stage j second half
  // into Q; then wait for stage j+1 and join the barrier (stage j is free).
  // Sub-step 2j+1: MFMAs on Q, refill stage j's arrays with stage j+2, read
  // stage j+1 first half into P.
#define FP8RT_EVEN(LA, LB, XA, XB)                                            \
  {                                                                           \
    read_frags(fq, LA, LB, wm, wn, fr, c_hi);                                 \
    mfma_step<FA, FB, MX, 0>(fp, acc, XA, XB);                                \
    for (int s = 0; s < 4; ++s) {                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      \
    }                                                                         \
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                        \
    step_barrier<0>();                                                        \
  }
#define FP8RT_ODD(DA, DB, DX, KS, LA, LB, LX, XA, XB, NXA, NXB)              \
  {                                                                           \
    sc_read(LX, NXA, NXB);                                                    \
    const int kn = min(KS, ns - 1);                                           \
    dma_tile<kDmaA>(a_base + kn * TKS, voa, DA, wave);                        \
    dma_tile<kDmaB>(b_base + kn * TKS, vob, DB, wave);                        \
    sc_dma(KS, DX);                                                           \
    read_frags(fp, LA, LB, wm, wn, fr, c_lo);                                 \
    mfma_step<FA, FB, MX, 2>(fq, acc, XA, XB);                                \
    for (int s = 0; s < 4; ++s) {                                             \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                      \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                      \
    }                                                                         \
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);                        \
    __builtin_amdgcn_sched_barrier(0);                                        \
  }
  for (int j = 0; j < ns; j += 2) {
    FP8RT_EVEN(sA0, sB0, xa0, xb0)
    FP8RT_ODD(sA0, sB0, sX0, j + 2, sA1, sB1, sX1, xa0, xb0, xa1, xb1)
    FP8RT_EVEN(sA1, sB1, xa1, xb1)
    FP8RT_ODD(sA1, sB1, sX1, j + 3, sA0, sB0, sX0, xa1, xb1, xa0, xb0)
  }
#undef FP8RT_EVEN
#undef FP8RT_ODD
  step_barrier<0>();  // the clamped extra loads finish before the arrays are reused

  // ---- epilogue.  The MFMA computed the transposed tile, so lane l holds
  // output row 32 i + (l % 32) and, per group g = e / 4, the 4 consecutive
  // columns 32 j + 8 g + 4 (l / 32) + (e % 4).  Column scales and bias go
  // through LDS once per block; each wave converts its 128 x 128 result,
  // stages it in its own 32 KB of LDS (16-byte chunks XOR-swizzled by row)
  // and stores 16-byte row chunks.
  __shared__ __attribute__((aligned(16))) float sCol[2][TN];
  if (unit) {
    sCol[0][t] = 1.0f;
    sCol[1][t] = 0.0f;
  } else {
    const int64_t col = min(n0 + t, N - 1);
    sCol[0][t] = MX ? 1.0f : sb[erb == 1 ? col : 0];  // MX scales were applied by the MFMA
    float bvv = 0.0f;
    if (bias)
      bvv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col]) << 16)
                      : static_cast<const float*>(bias)[col];
    sCol[1][t] = bvv;
  }
  __syncthreads();
  uint8_t* stage = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
  float sav[MI];
  uint32_t mb = 0, sat_l = 0, under_l = 0;
  if (unit) {
#pragma unroll
    for (int i = 0; i < MI; ++i) sav[i] = 1.0f;
    float* dst = part + static_cast<int64_t>(bid - t_main) * (TM * TN);
    store_tile<kOutF32>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wm * WTM, wn * WTN, TM, TN, dst, TN, 1, wn, fr,
                        fg, lane, 1.0f, mb, sat_l, under_l);
  } else {
    const int64_t wrow0 = m0 + wm * WTM, wcol0 = n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < MI; ++i) sav[i] = MX ? 1.0f : sa[era == 1 ? min(wrow0 + i * 32 + fr, M - 1) : 0];
    float rq = 1.0f;
    if constexpr (OUT >= kOutE4M3) rq = ry ? ry[0] : 1.0f / sy[0];
    // the whole block tile inside (M, N): every wave takes the same branch
    // (store_tile holds barriers)
    if (OUT >= kOutE4M3 && m0 + TM <= M && n0 + TN <= N)
      store_tile<OUT, false>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wrow0, wcol0, M, N, Y, ldy, vec_store, wn,
                             fr, fg, lane, rq, mb, sat_l, under_l);
    else
      store_tile<OUT, true>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wrow0, wcol0, M, N, Y, ldy, vec_store, wn,
                            fr, fg, lane, rq, mb, sat_l, under_l);
  }
  // FP8 output: a whole tile's max |y| and counters (split-K units hold raw
  // partial sums; k_split_reduce takes the statistics of their tiles)
  if constexpr (OUT >= kOutE4M3)
    if (!unit) block_stats_store<kWaves>(reinterpret_cast<u32x4*>(&ypart[bid]), mb, sat_l, under_l);
}

// Finishes the split-K tiles: tile t_main + k sums its `split` FP32 partials
// part[k split + p] in the order p = 0, 1, ..., applies s_a(row) s_b(col) and
// the bias, rounds and stores.  A block covers kRedQ x 256 quads (4
// consecutive columns each) of one tile, thread t the quads t, t + 256, ...
// FP8 output: codes of y * rq, and the block's max |y| and counters go to
// ypart[t_main + k kRedBlocks + blockIdx.x].
constexpr int kRedQ = 4;
constexpr int kRedBlocks = TM * TN / 4 / 256 / kRedQ;  // blocks per split tile
template <int OUT>
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, int t_main, int split,
                                                      int tiles_m, int tiles_n, int64_t M, int64_t N,
                                                      const float* __restrict__ sa, int64_t era,
                                                      const float* __restrict__ sb, int64_t erb,
                                                      const void* __restrict__ bias, int bias_bf16,
                                                      void* __restrict__ Y, int64_t ldy, int vec_store,
                                                      const float* __restrict__ sy, const float* __restrict__ ry,
                                                      BlockPartial* __restrict__ ypart) {
  const int k = blockIdx.y;
  int tile_m, tile_n;
  tile_of(t_main + k, tiles_m, tiles_n, tile_m, tile_n);
  float rq = 1.0f;
  if constexpr (OUT >= kOutE4M3) rq = ry ? ry[0] : 1.0f / sy[0];
  uint32_t mb = 0, sat_l = 0, under_l = 0;
#pragma unroll
  for (int qi = 0; qi < kRedQ; ++qi) {
    const int idx = (blockIdx.x * kRedQ + qi) * 256 + threadIdx.x;  // quad index in the tile
    const int r = idx / (TN / 4), c = (idx % (TN / 4)) * 4;
    const int64_t row = static_cast<int64_t>(tile_m) * TM + r, col = static_cast<int64_t>(tile_n) * TN + c;
    if (row >= M || col >= N) continue;
    const float* p = part + static_cast<int64_t>(k) * split * (TM * TN) + r * TN + c;
    f32x4 acc = *reinterpret_cast<const f32x4*>(p);
    for (int q = 1; q < split; ++q) acc += *reinterpret_cast<const f32x4*>(p + static_cast<int64_t>(q) * (TM * TN));
    const float sav = sa[era == 1 ? row : 0];
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t cc = min(col + e, N - 1);
      float bv = 0.0f;
      if (bias)
        bv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[cc]) << 16)
                       : static_cast<const float*>(bias)[cc];
      v[e] = acc[e] * (sav * sb[erb == 1 ? cc : 0]) + bv;
    }
    if constexpr (OUT == kOutBF16) {
      const bf16x4 h = __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4);
      uint16_t* dst = static_cast<uint16_t*>(Y) + row * ldy + col;
      if (vec_store && col + 4 <= N) {
        *reinterpret_cast<bf16x4*>(dst) = h;
      } else {
        const u32x2 hb = __builtin_bit_cast(u32x2, h);  // 4 bf16 as 2 words
        for (int e = 0; e < 4 && col + e < N; ++e) dst[e] = static_cast<uint16_t>(hb[e >> 1] >> (16 * (e & 1)));
      }
    } else if constexpr (OUT == kOutF32) {
      float* dst = static_cast<float*>(Y) + row * ldy + col;
      if (vec_store && col + 4 <= N) {
        *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
      } else {
        for (int e = 0; e < 4 && col + e < N; ++e) dst[e] = v[e];
      }
    } else {
      constexpr int F = OUT == kOutE4M3 ? kE4M3 : kE5M2;
      float f[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[e] = v[e] * rq;
        const bool in = col + e < N;
        mb = max(mb, in ? (__float_as_uint(v[e]) & kAbsMask) : 0u);
        sat_l += (in && fabsf(f[e]) > Fmt<F>::kMax) ? 1u : 0u;
        under_l += (in && v[e] != 0.0f && fabsf(f[e]) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
      }
      const uint32_t w = cvt4_nan<F>(f[0], f[1], f[2], f[3]);
      uint8_t* dst = static_cast<uint8_t*>(Y) + row * ldy + col;
      if (vec_store && col + 4 <= N) {
        *reinterpret_cast<uint32_t*>(dst) = w;
      } else {
        for (int e = 0; e < 4 && col + e < N; ++e) dst[e] = static_cast<uint8_t>(w >> (8 * e));
      }
    }
  }
  if constexpr (OUT >= kOutE4M3)
    block_stats_store<4>(reinterpret_cast<u32x4*>(&ypart[t_main + k * kRedBlocks + blockIdx.x]), mb, sat_l,
                         under_l);
}

// Repack power-of-two 1x32 scales (fp32, [rows][K / 32]) as E8M0 exponent
// bytes for the MFMA: dword [row / 32][stage][half][row % 32] holds in bytes 0
// and 2 the exponents of K blocks 4 stage + half and 4 stage + half + 2 (the
// blocks that lane half `half` of an MFMA covers in the stage's two
// sub-steps).  Rows past the end get exponent 127 (scale 1); their products
// are never stored.
__global__ __launch_bounds__(256) void k_pack_e8m0(const float* __restrict__ s, int64_t rows, int64_t nblk,
                                                   int64_t ngroups, int64_t nstage, uint32_t* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= ngroups * nstage * 64) return;
  const int64_t rr = idx & 31, half = (idx >> 5) & 1, gs = idx >> 6;
  const int64_t st = gs % nstage, g = gs / nstage;
  const int64_t row = g * 32 + rr;
  uint32_t w = 0x007F007Fu;
  if (row < rows) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(s + row * nblk + st * 4 + half);
    w = ((src[0] >> 23) & 0xFFu) | (((src[2] >> 23) & 0xFFu) << 16);
  }
  out[idx] = w;
}

}  // namespace

bool gemm_big_eligible(const GemmArgs& g) {
  // per-tensor or per-row scales only (the epilogue selects, it does not divide)
  const bool rows_ok = (g.era == 1 || g.era >= g.M) && (g.erb == 1 || g.erb >= g.N);
  const bool scales_ok = g.pow2_mx ? (g.era == 1 && g.erb == 1 && g.eca == 32 && g.ecb == 32)
                                   : (g.eca >= g.K && g.ecb >= g.K);
  return rows_ok && scales_ok && g.K % (2 * TKS) == 0 && g.M >= 128 &&
         g.N >= 128 && g.lda < (int64_t(1) << 23) && g.ldb < (int64_t(1) << 23);
}

hipError_t launch_gemm_big(const GemmArgs& g, hipStream_t st, int* nparts) {
  const int tiles_m = static_cast<int>((g.M + TM - 1) / TM);
  const int tiles_n = static_cast<int>((g.N + TN - 1) / TN);
  const int okind = gemm_out_kind(g);
  const int esz = okind == kOutF32 ? 4 : okind == kOutBF16 ? 2 : 1;
  const int vec = ((g.ldy * esz) % 16 == 0) && ((reinterpret_cast<uintptr_t>(g.y) & 15u) == 0);
  const int T = tiles_m * tiles_n;
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
  // Ragged last wave: when the tiles fill the CUs a whole number of times
  // plus a last wave at most half full (the 4096 x 29568 up-projection: 7
  // waves + 64 tiles), each last-wave tile is split along K into up to 4
  // units so the last wave fills the CUs; k_split_reduce adds the parts.
  int t_main = T, split = 1, ns_part = 0;
  float* part = nullptr;
  {
    const int cus = device_cus();
    const int rem = T % cus;
    const int64_t ns = g.K / TKS;
    // FP8 output: one statistics slot per whole tile and per reduce block
    const bool slots_ok = okind < kOutE4M3 || (T - rem) + rem * kRedBlocks <= kMaxBlocks;
    if (!g.pow2_mx && slots_ok && T > cus && rem > 0 && 2 * rem <= cus) {
      int sp = std::min(cus / rem, 4);
      while (sp > 1 && ns % (2 * sp) != 0) --sp;  // every part an even number of stages
      if (sp > 1) {
        void* p = nullptr;
        hipError_t e = get_scratch(st, static_cast<size_t>(rem) * sp * TM * TN * sizeof(float), &p);
        if (e != hipSuccess) return e;
        part = static_cast<float*>(p);
        split = sp;
        t_main = T - rem;
        ns_part = static_cast<int>(ns / sp);
      }
    }
  }
  const dim3 grid(static_cast<unsigned>(t_main + (T - t_main) * split));
  uint32_t* xpa = nullptr;
  uint32_t* xpb = nullptr;
  if (g.pow2_mx) {
    const int64_t ns = g.K / TKS, ga = (g.M + 31) / 32, gb = (g.N + 31) / 32;
    void* p = nullptr;
    hipError_t e = get_scratch(st, static_cast<size_t>((ga + gb) * ns * 64) * 4, &p);
    if (e != hipSuccess) return e;
    xpa = static_cast<uint32_t*>(p);
    xpb = xpa + ga * ns * 64;
    hipLaunchKernelGGL(k_pack_e8m0, dim3(static_cast<unsigned>((ga * ns * 64 + 255) / 256)), dim3(256), 0, st,
                       g.sa, g.M, g.K / 32, ga, ns, xpa);
    hipLaunchKernelGGL(k_pack_e8m0, dim3(static_cast<unsigned>((gb * ns * 64 + 255) / 256)), dim3(256), 0, st,
                       g.sb, g.N, g.K / 32, gb, ns, xpb);
  }
#define FP8RT_BIG(FA, FB, OUT, MXV)                                                                         \
  hipLaunchKernelGGL((k_gemm_big<FA, FB, OUT, MXV>), grid, dim3(kThreads), 0, st, g.a, g.lda, g.b, g.ldb, \
                     g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, tiles_m, tiles_n, vec, \
                     xpa, xpb, t_main, split, ns_part, part, g.sy, g.ry, g.part)
#define FP8RT_BIG_OUT(FA, FB, MXV)                                  \
  switch (okind) {                                                  \
    case kOutBF16: FP8RT_BIG(FA, FB, kOutBF16, MXV); break;         \
    case kOutE4M3: FP8RT_BIG(FA, FB, kOutE4M3, MXV); break;         \
    case kOutE5M2: FP8RT_BIG(FA, FB, kOutE5M2, MXV); break;         \
    default: FP8RT_BIG(FA, FB, kOutF32, MXV); break;                \
  }
  if (g.fa == FP8RT_E4M3) {
    if (g.pow2_mx) { FP8RT_BIG_OUT(0, 0, true) } else { FP8RT_BIG_OUT(0, 0, false) }
  } else {
    if (g.pow2_mx) { FP8RT_BIG_OUT(1, 0, true) } else { FP8RT_BIG_OUT(1, 0, false) }
  }
#undef FP8RT_BIG_OUT
#undef FP8RT_BIG
  if (split > 1) {
    const dim3 rgrid(kRedBlocks, static_cast<unsigned>(T - t_main));
#define FP8RT_RED(OUT)                                                                                          \
  hipLaunchKernelGGL(k_split_reduce<OUT>, rgrid, dim3(256), 0, st, part, t_main, split, tiles_m, tiles_n, g.M, \
                     g.N, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, vec, g.sy, g.ry, g.part)
    switch (okind) {
      case kOutBF16: FP8RT_RED(kOutBF16); break;
      case kOutE4M3: FP8RT_RED(kOutE4M3); break;
      case kOutE5M2: FP8RT_RED(kOutE5M2); break;
      default: FP8RT_RED(kOutF32); break;
    }
#undef FP8RT_RED
  }
  if (nparts) *nparts = split > 1 ? t_main + (T - t_main) * kRedBlocks : T;
  return hipGetLastError();
}

}  // namespace fp8rt
