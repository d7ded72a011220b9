// gemm_big.hip -- the large-shape scaled FP8 GEMM for gfx950 (per-tensor and
// per-row / per-output-channel scales applied in the epilogue, 1x32
// power-of-two scales inside the MFMA).
//
// Method: "FP8 formats and scaling for LLM inference", section "The full
// precision contract of one FP8 GEMM": Y ~ s_x s_w (X8 W8) with FP32
// accumulation, BF16/FP32 output and bias; section "Per-channel and block
// scaling" for per-row scales.  Y[m,n] = s_a(m) s_b(n) sum_k dec(A[m,k]) dec(B[n,k]) + bias[n].
//
// Design for MI355X:
//  - 256 x 256 output tile per workgroup of 4 waves (one per SIMD); each wave
//    owns a 128 x 128 sub-tile: 8 x 8 v_mfma_f32_16x16x128_f8f6f4 per 128-deep
//    K stage (one instruction consumes a whole stage), 64 four-wide FP32
//    accumulators per lane held in AGPRs.
//  - Two LDS stages of 128 K bytes (64 KB each).  A stage row is 128 bytes,
//    a whole cache line, so every vector-memory request moves a full line
//    (64-byte half rows doubled the L1->L2 request count and stalled the
//    address path).  Operands move HBM -> LDS with buffer_load_dwordx4 ...
//    lds (no VGPR staging; a uniform buffer descriptor per operand tile, the
//    lane's row / chunk offset in a VGPR and the stage's K offset in an SGPR,
//    so no per-load address arithmetic): one instruction fills 8 rows; each
//    lane picks the global chunk that belongs at its LDS slot, an XOR swizzle
//    of the 8 chunks of a row by (row / 2) that makes the ds_read_b128
//    fragment reads conflict-free on the 64-bank LDS.
//  - The schedule inside a stage and its two barriers are described with the
//    kernel (k_gemm_big16).
//  - 1x32 power-of-two scales: the scaled form of the same MFMA applies one
//    E8M0 exponent per row and 32-element K block of each operand, repacked
//    once per call (k_pack_e8m0_16).
//  - Tile order: blocks are dealt round-robin to the 8 XCDs; each XCD gets a
//    contiguous range of a grouped (GROUP_M M-tiles x all N-tiles) order, so
//    the 32 CUs of an XCD share A and B slices in their own L2.
//  - The MFMA computes the transposed tile (B as the first operand), so a
//    lane ends with 4 consecutive output columns of one row: the epilogue
//    applies the scales and bias with 4-wide LDS reads of the block's column
//    vectors, converts with the hardware bf16 conversion (round to nearest
//    even) or the FP8 cast, stages pieces in LDS and stores 16-byte row chunks.
//  - A ragged last wave, or a grid of at most half the CUs, is split along K
//    (k_split_reduce adds the parts).
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
constexpr int TKS = 128;                          // K bytes per LDS stage (full 128-byte rows)
constexpr int kWaves = 4, WAVES_N = 2;            // 2 x 2 waves
constexpr int kThreads = kWaves * 64;
constexpr int WTM = TM / (kWaves / WAVES_N);      // 128 rows per wave
constexpr int WTN = TN / WAVES_N;                 // 128 columns per wave
constexpr int MI16 = WTM / 16, NJ16 = WTN / 16;   // 8 x 8 MFMA tiles of 16 x 16 per wave
constexpr int kStageA = TM * TKS, kStageB = TN * TKS;  // 32 KB + 32 KB per stage
constexpr int kDmaA = kStageA / 1024 / kWaves;    // 8 DMA instructions per wave
constexpr int kDmaB = kStageB / 1024 / kWaves;    // 8
constexpr int GROUP_M = 4;

// Byte offset of 16-byte chunk c (0..7) of stage row r (128-byte rows).
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

// Epilogue of one block: lane l holds output row 16 i + (l % 16) and
// columns 16 j + 4 (l / 16) + e of its wave tile (the MFMA computed the
// transposed tile, accumulator acc[i][j][e]).  Values are
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
__device__ __forceinline__ void store_tile(const f32x4 (&acc)[MI16][NJ16], uint8_t* stage, const float* scol,
                                           const float* sbias, const float (&sav)[MI16], int64_t wrow0, int64_t wcol0,
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
  constexpr int IPP = ROWS / 16;                // MFMA row tiles per pass
  constexpr int EPC = 16 / ESZ;                 // elements per chunk
#pragma unroll
  for (int pass = 0; pass < MI16 / IPP; ++pass) {
#pragma unroll
    for (int ii = 0; ii < IPP; ++ii) {
      const int i = pass * IPP + ii;
      const int lrow = ii * 16 + fr;            // row within the pass
#pragma unroll
      for (int j = 0; j < NJ16; ++j) {
          const int c = j * 16 + 4 * fg;          // first of 4 columns within the wave tile
          const f32x4 scv = *reinterpret_cast<const f32x4*>(&scol[wn * WTN + c]);
          const f32x4 biv = *reinterpret_cast<const f32x4*>(&sbias[wn * WTN + c]);
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][r] * (sav[i] * scv[r]) + biv[r];
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

// ---- 16x16x128 kernel (per-tensor / per-row scales; BF16, FP32 or FP8 output).
// The same 256 x 256 tile, 4 waves of 128 x 128, LDS stages, DMA and tile
// order as described at the top; each wave issues 8 x 8 v_mfma_f32_16x16x128_f8f6f4
// per 128-deep stage (one instruction consumes the whole stage).  On random
// operands this instruction sustains a higher rate than 32x32x64 (the chip
// holds a higher clock for it).  Registers: 64 four-wide accumulators (256
// AGPRs, updated in place by inline MFMAs), B's 8 fragments of the current
// and of the next stage (2 x 64 VGPRs) and A's 8 fragments (64 VGPRs).  Two
// barriers per stage: one after the stage's last LDS read (row tile 1), after
// which the stage after next is loaded into its arrays, and one at row tile 5
// for the next stage's loads, so each stage's loads fly for 1.4 stages (with
// a single barrier per stage, 1 stage, the kernel ran 5-10% slower).

// 16x16x128 operand: lane l holds row l % 16; the matrix core reads its first
// 16 bytes as K [16 g, +16) and its last 16 as K [64 + 16 g, +16) of the
// stage, g = l / 16 (A and B use the same map, so each product pairs equal K).
__device__ __forceinline__ i32x8 frag16(const uint8_t* lds, int row, int g) {
  const u32x4 lo = *reinterpret_cast<const u32x4*>(lds + swz(row, g));
  const u32x4 hi = *reinterpret_cast<const u32x4*>(lds + swz(row, g + 4));
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// One 16x16x128 MFMA, acc += B-fragment x A-fragment (the transposed tile),
// written inline with the accumulator as one tied operand, so it stays in
// the same AGPRs from stage to stage (the builtin's untied form made the
// register allocator rotate the 64 accumulators between the two unrolled
// stages and copy them back, about 100 moves per stage).  A E5M2 (FA = 1) is
// the instruction's second source: blgp:1.
template <int FA>
__device__ __forceinline__ void mfma16(f32x4& acc, const i32x8& b, const i32x8& a) {
  if constexpr (FA == 0)
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(b), "v"(a));
  else
    asm volatile("v_mfma_f32_16x16x128_f8f6f4 %0, %1, %2, %0 blgp:1" : "+a"(acc) : "v"(b), "v"(a));
}

// The same with 1x32 power-of-two scales: E8M0 exponent bytes, byte OB of
// sb for the B operand (the instruction's first source) and byte OA of sa
// for A; each lane supplies the exponent of its row and of K block
// (lane / 16) of the stage, the block its lane group's bytes belong to.
#define FP8RT_MFMA16X(ALO, AHI, BLO, BHI, FMT)                                                                \
  asm volatile("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #BLO "," #ALO              \
               ",0] op_sel_hi:[" #BHI "," #AHI ",0]" FMT                                                      \
               : "+a"(acc)                                                                                     \
               : "v"(b), "v"(a), "v"(sb), "v"(sa))
template <int FA, int OA, int OB>
__device__ __forceinline__ void mfma16x(f32x4& acc, const i32x8& b, const i32x8& a, uint32_t sb, uint32_t sa) {
  if constexpr (FA == 0 && OA == 0 && OB == 0) FP8RT_MFMA16X(0, 0, 0, 0, "");
  else if constexpr (FA == 0 && OA == 0 && OB == 1) FP8RT_MFMA16X(0, 0, 1, 0, "");
  else if constexpr (FA == 0 && OA == 0 && OB == 2) FP8RT_MFMA16X(0, 0, 0, 1, "");
  else if constexpr (FA == 0 && OA == 0 && OB == 3) FP8RT_MFMA16X(0, 0, 1, 1, "");
  else if constexpr (FA == 0 && OA == 1 && OB == 0) FP8RT_MFMA16X(1, 0, 0, 0, "");
  else if constexpr (FA == 0 && OA == 1 && OB == 1) FP8RT_MFMA16X(1, 0, 1, 0, "");
  else if constexpr (FA == 0 && OA == 1 && OB == 2) FP8RT_MFMA16X(1, 0, 0, 1, "");
  else if constexpr (FA == 0 && OA == 1 && OB == 3) FP8RT_MFMA16X(1, 0, 1, 1, "");
  else if constexpr (FA == 0 && OA == 2 && OB == 0) FP8RT_MFMA16X(0, 1, 0, 0, "");
  else if constexpr (FA == 0 && OA == 2 && OB == 1) FP8RT_MFMA16X(0, 1, 1, 0, "");
  else if constexpr (FA == 0 && OA == 2 && OB == 2) FP8RT_MFMA16X(0, 1, 0, 1, "");
  else if constexpr (FA == 0 && OA == 2 && OB == 3) FP8RT_MFMA16X(0, 1, 1, 1, "");
  else if constexpr (FA == 0 && OA == 3 && OB == 0) FP8RT_MFMA16X(1, 1, 0, 0, "");
  else if constexpr (FA == 0 && OA == 3 && OB == 1) FP8RT_MFMA16X(1, 1, 1, 0, "");
  else if constexpr (FA == 0 && OA == 3 && OB == 2) FP8RT_MFMA16X(1, 1, 0, 1, "");
  else if constexpr (FA == 0 && OA == 3 && OB == 3) FP8RT_MFMA16X(1, 1, 1, 1, "");
  else if constexpr (FA == 1 && OA == 0 && OB == 0) FP8RT_MFMA16X(0, 0, 0, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 0 && OB == 1) FP8RT_MFMA16X(0, 0, 1, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 0 && OB == 2) FP8RT_MFMA16X(0, 0, 0, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 0 && OB == 3) FP8RT_MFMA16X(0, 0, 1, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 1 && OB == 0) FP8RT_MFMA16X(1, 0, 0, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 1 && OB == 1) FP8RT_MFMA16X(1, 0, 1, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 1 && OB == 2) FP8RT_MFMA16X(1, 0, 0, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 1 && OB == 3) FP8RT_MFMA16X(1, 0, 1, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 2 && OB == 0) FP8RT_MFMA16X(0, 1, 0, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 2 && OB == 1) FP8RT_MFMA16X(0, 1, 1, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 2 && OB == 2) FP8RT_MFMA16X(0, 1, 0, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 2 && OB == 3) FP8RT_MFMA16X(0, 1, 1, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 3 && OB == 0) FP8RT_MFMA16X(1, 1, 0, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 3 && OB == 1) FP8RT_MFMA16X(1, 1, 1, 0, " blgp:1");
  else if constexpr (FA == 1 && OA == 3 && OB == 2) FP8RT_MFMA16X(1, 1, 0, 1, " blgp:1");
  else if constexpr (FA == 1 && OA == 3 && OB == 3) FP8RT_MFMA16X(1, 1, 1, 1, " blgp:1");
}
#undef FP8RT_MFMA16X

// Wait states between VALU accesses of the accumulators and the inline MFMAs
// (which the compiler's hazard recognizer does not see): 24, more than the
// 8-pass MFMA's write-to-VALU-read distance and the VALU-write-to-MFMA one.
__device__ __forceinline__ void acc_fence(f32x4 (&acc)[MI16][NJ16]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[0][4]),
                 "+a"(acc[0][5]), "+a"(acc[0][6]), "+a"(acc[0][7]), "+a"(acc[1][0]), "+a"(acc[1][1]),
                 "+a"(acc[1][2]), "+a"(acc[1][3]), "+a"(acc[1][4]), "+a"(acc[1][5]), "+a"(acc[1][6]),
                 "+a"(acc[1][7]), "+a"(acc[2][0]), "+a"(acc[2][1]), "+a"(acc[2][2]), "+a"(acc[2][3]),
                 "+a"(acc[2][4]), "+a"(acc[2][5]), "+a"(acc[2][6]), "+a"(acc[2][7]), "+a"(acc[3][0]),
                 "+a"(acc[3][1]), "+a"(acc[3][2]), "+a"(acc[3][3]), "+a"(acc[3][4]), "+a"(acc[3][5]),
                 "+a"(acc[3][6]), "+a"(acc[3][7]), "+a"(acc[4][0]), "+a"(acc[4][1]), "+a"(acc[4][2]),
                 "+a"(acc[4][3]), "+a"(acc[4][4]), "+a"(acc[4][5]), "+a"(acc[4][6]), "+a"(acc[4][7]),
                 "+a"(acc[5][0]), "+a"(acc[5][1]), "+a"(acc[5][2]), "+a"(acc[5][3]), "+a"(acc[5][4]),
                 "+a"(acc[5][5]), "+a"(acc[5][6]), "+a"(acc[5][7]), "+a"(acc[6][0]), "+a"(acc[6][1]),
                 "+a"(acc[6][2]), "+a"(acc[6][3]), "+a"(acc[6][4]), "+a"(acc[6][5]), "+a"(acc[6][6]),
                 "+a"(acc[6][7]), "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
                 "+a"(acc[7][4]), "+a"(acc[7][5]), "+a"(acc[7][6]), "+a"(acc[7][7]));
}

// Wait for this wave's LDS reads (its vector-memory loads keep flying) and
// join the workgroup barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt at their maximum
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_sched_barrier(0);
}

// One DMA instruction of a stage: 1 KB (8 rows of 128 bytes) into slot k.
__device__ __forceinline__ void dma1(__amdgpu_buffer_rsrc_t rs, int soff, uint32_t voff, uint8_t* lds, int k) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(lds + k * 1024), 16, static_cast<int>(voff), soff, 0, 0);
}

// One MFMA of row tile I, column tile J: plain, or with the exponent bytes
// I % 4 of xa and J % 4 of xb (1x32 scales).
template <int FA, bool MX>
__device__ __forceinline__ void mf16(f32x4& acc, const i32x8& b, const i32x8& a, uint32_t xb, uint32_t xa, int i,
                                     int j) {
  if constexpr (!MX) {
    mfma16<FA>(acc, b, a);
  } else {
    // i and j are constants after unrolling: one asm form each
    switch (((i & 3) << 2) | (j & 3)) {
      case 0: mfma16x<FA, 0, 0>(acc, b, a, xb, xa); break;
      case 1: mfma16x<FA, 0, 1>(acc, b, a, xb, xa); break;
      case 2: mfma16x<FA, 0, 2>(acc, b, a, xb, xa); break;
      case 3: mfma16x<FA, 0, 3>(acc, b, a, xb, xa); break;
      case 4: mfma16x<FA, 1, 0>(acc, b, a, xb, xa); break;
      case 5: mfma16x<FA, 1, 1>(acc, b, a, xb, xa); break;
      case 6: mfma16x<FA, 1, 2>(acc, b, a, xb, xa); break;
      case 7: mfma16x<FA, 1, 3>(acc, b, a, xb, xa); break;
      case 8: mfma16x<FA, 2, 0>(acc, b, a, xb, xa); break;
      case 9: mfma16x<FA, 2, 1>(acc, b, a, xb, xa); break;
      case 10: mfma16x<FA, 2, 2>(acc, b, a, xb, xa); break;
      case 11: mfma16x<FA, 2, 3>(acc, b, a, xb, xa); break;
      case 12: mfma16x<FA, 3, 0>(acc, b, a, xb, xa); break;
      case 13: mfma16x<FA, 3, 1>(acc, b, a, xb, xa); break;
      case 14: mfma16x<FA, 3, 2>(acc, b, a, xb, xa); break;
      default: mfma16x<FA, 3, 3>(acc, b, a, xb, xa); break;
    }
  }
}

// Row tile at which the 16x16x128 kernel's second barrier sits (the next
// stage's fragments are read from there to row 7): rows 4, 5 and 6 measured
// within 1-3% of each other at the large shapes, 5 the best or equal.
constexpr int kRowB16 = 5;

template <int FA, int FB, int OUT, bool MX, int RB>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_big16(
    const uint8_t* __restrict__ A, int64_t lda, const uint8_t* __restrict__ B, int64_t ldb,
    int64_t M, int64_t N, int64_t K, const float* __restrict__ sa, int64_t era,
    const float* __restrict__ sb, int64_t erb, const void* __restrict__ bias, int bias_bf16,
    void* __restrict__ Y, int64_t ldy, int tiles_m, int tiles_n, int vec_store, int t_main, int split,
    int ns_part, float* __restrict__ part, const float* __restrict__ sy, const float* __restrict__ ry,
    BlockPartial* __restrict__ ypart, const u32x2* __restrict__ xpa, const u32x2* __restrict__ xpb) {
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
  const int fr = lane & 15, fg = lane >> 4;

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
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(A + m0 * lda + static_cast<int64_t>(s0) * TKS), 0, -1, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(B + n0 * ldb + static_cast<int64_t>(s0) * TKS), 0, -1, 0x00020000);

  f32x4 acc[MI16][NJ16];
#pragma unroll
  for (int i = 0; i < MI16; ++i)
#pragma unroll
    for (int j = 0; j < NJ16; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  // the zeros are written to the accumulators by VALU moves, which the first
  // (inline) MFMAs read: wait states between them
  acc_fence(acc);

  constexpr int kDmaStage = kDmaA + kDmaB;
  const int ns = unit ? ns_part : static_cast<int>(K / TKS);  // even
  const int ra0 = wm * WTM + fr, rb0 = wn * WTN + fr;         // the lane's first A / B fragment row

  // 1x32 scales: the lane's 8 exponent bytes of A (one per row tile) and of
  // B for a stage, repacked by k_pack_e8m0_16 as [128-row block][stage]
  // [lane]; x0 / x1 hold the even / odd stage's, loaded one stage ahead
  // (issued before the DMA of the stage after next, so the second barrier's
  // wait covers them).
  const int ns_all = static_cast<int>(K / TKS);
  const u32x2* xra = nullptr;
  const u32x2* xrb = nullptr;
  u32x2 xa0 = {}, xb0 = {}, xa1 = {}, xb1 = {};
  if constexpr (MX) {
    xra = xpa + ((m0 / WTM + wm) * ns_all + s0) * 64 + lane;
    xrb = xpb + ((n0 / WTN + wn) * ns_all + s0) * 64 + lane;
    xa0 = xra[0];
    xb0 = xrb[0];
  }
  dma_buf<kDmaA>(ra, 0, voa, sA0, wave);
  dma_buf<kDmaB>(rb, 0, vob, sB0, wave);
  dma_buf<kDmaA>(ra, TKS, voa, sA1, wave);
  dma_buf<kDmaB>(rb, TKS, vob, sB1, wave);
  step_barrier<kDmaStage>();  // stage 0 landed (and stage 0's exponents, loaded before it)
  if constexpr (MX) asm volatile("" : "+v"(xa0), "+v"(xb0));
  i32x8 bx[NJ16], by[NJ16], af[MI16];
#pragma unroll
  for (int j = 0; j < NJ16; ++j) bx[j] = frag16(sB0, rb0 + j * 16, fg);
  af[0] = frag16(sA0, ra0, fg);

  // One stage s (arrays LA / LB), row tiles 0-7 with A fragment i in af[i]:
  //  - rows 0-1 read A row tiles 1-7 of stage s, the last reads of this
  //    stage's arrays;
  //  - a barrier (every wave has read stage s), then rows 2-3 issue the DMA
  //    of stage s + 2 into stage s's arrays (one load after each MFMA; two
  //    after each MFMA of row 2 alone ran 10% slower);
  //  - a second barrier at row RB (every wave's loads of stage s + 1 have
  //    landed; stage s + 2's stay in flight), then rows RB-7 read stage
  //    s + 1's B fragments 0-7 and A row tile 0 (9 fragments, evenly).
  // A stage's loads are in flight from row 2 of one stage to row RB of the
  // next.  The MFMAs are inline and volatile, so every memory operation
  // keeps its place between them as written here.
  constexpr int kNR = MI16 - RB;                     // rows that read the next stage
  constexpr int kPer = (NJ16 + 1 + kNR - 1) / kNR;   // fragments per such row
#define FP8RT_STAGE16(LA, LB, NA, NB, BC, BN, XA, XB, NXA, NXB, KS)                                                              \
  {                                                                                                            \
    _Pragma("unroll") for (int i = 0; i < 2; ++i) {                                                             \
      _Pragma("unroll") for (int j = 0; j < NJ16; ++j) {                                                        \
        mf16<FA, MX>(acc[i][j], BC[j], af[i], XB[j >> 2], XA[i >> 2], i, j);                                                                   \
        const int t2 = 4 * i + j + 1;  /* A row tile read after this MFMA */                                   \
        if (j < 4 && t2 < MI16) af[t2] = frag16(LA, ra0 + t2 * 16, fg);                                        \
      }                                                                                                        \
    }                                                                                                          \
    lds_barrier();                                                                                             \
    const int kn = min(KS, ns - 1);                                                                            \
    if constexpr (MX) {                                                                                        \
      const int kx = min(KS - 1, ns - 1);  /* the next stage's exponents */                                    \
      NXA = xra[kx * 64];                                                                                      \
      NXB = xrb[kx * 64];                                                                                      \
    }                                                                                                          \
    _Pragma("unroll") for (int i = 2; i < RB; ++i) {                                                            \
      _Pragma("unroll") for (int j = 0; j < NJ16; ++j) {                                                        \
        mf16<FA, MX>(acc[i][j], BC[j], af[i], XB[j >> 2], XA[i >> 2], i, j);                                                                   \
        if (i < 4) {   /* 16 DMA instructions, one after each MFMA of rows 2-3: A's 8, then B's 8 */        \
          const int d = (i - 2) * NJ16 + j;                                                                    \
          if (d < kDmaA) dma1(ra, kn * TKS, voa[d], LA, wave * kDmaA + d);                                      \
          else dma1(rb, kn * TKS, vob[d - kDmaA], LB, wave * kDmaB + d - kDmaA);                                \
        }                                                                                                      \
      }                                                                                                        \
    }                                                                                                          \
    step_barrier<kDmaStage>();                                                                                 \
    /* the next stage's exponents have landed (the wait above covers them): an \
       opaque use here keeps the compiler from waiting for every load at the \
       loop head, where it would otherwise meet them still marked in flight */ \
    if constexpr (MX) asm volatile("" : "+v"(NXA), "+v"(NXB));                                                  \
    _Pragma("unroll") for (int i = RB; i < MI16; ++i) {                                                         \
      _Pragma("unroll") for (int j = 0; j < NJ16; ++j) {                                                        \
        mf16<FA, MX>(acc[i][j], BC[j], af[i], XB[j >> 2], XA[i >> 2], i, j);                                                                   \
        const int k = (i - RB) * kPer + j;  /* item k: B 0, A 0, B 1 .. B 7 */                                 \
        if (j < kPer && k <= NJ16) {                                                                           \
          if (k == 1) af[0] = frag16(NA, ra0, fg);                                                             \
          else { const int jb = k == 0 ? 0 : k - 1; BN[jb] = frag16(NB, rb0 + jb * 16, fg); }                  \
        }                                                                                                      \
      }                                                                                                        \
    }                                                                                                          \
  }
  for (int s = 0; s < ns; s += 2) {
    FP8RT_STAGE16(sA0, sB0, sA1, sB1, bx, by, xa0, xb0, xa1, xb1, s + 2)
    FP8RT_STAGE16(sA1, sB1, sA0, sB0, by, bx, xa1, xb1, xa0, xb0, s + 3)
  }
#undef FP8RT_STAGE16
  // the last MFMAs' results are read by VALU instructions below: wait states
  acc_fence(acc);
  step_barrier<0>();  // the clamped extra loads finish before the arrays are reused

  __shared__ __attribute__((aligned(16))) float sCol[2][TN];
  if (unit) {
    sCol[0][t] = 1.0f;
    sCol[1][t] = 0.0f;
  } else {
    const int64_t col = min(n0 + t, N - 1);
    sCol[0][t] = MX ? 1.0f : sb[erb == 1 ? col : 0];  // 1x32 scales were applied by the MFMA
    float bvv = 0.0f;
    if (bias)
      bvv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[col]) << 16)
                      : static_cast<const float*>(bias)[col];
    sCol[1][t] = bvv;
  }
  __syncthreads();
  uint8_t* stage = wave == 0 ? sA0 : wave == 1 ? sA1 : wave == 2 ? sB0 : sB1;
  float sav[MI16];
  uint32_t mb = 0, sat_l = 0, under_l = 0;
  if (unit) {
#pragma unroll
    for (int i = 0; i < MI16; ++i) sav[i] = 1.0f;
    float* dst = part + static_cast<int64_t>(bid - t_main) * (TM * TN);
    store_tile<kOutF32, true>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wm * WTM, wn * WTN, TM, TN, dst, TN, 1,
                                  wn, fr, fg, lane, 1.0f, mb, sat_l, under_l);
  } else {
    const int64_t wrow0 = m0 + wm * WTM, wcol0 = n0 + wn * WTN;
#pragma unroll
    for (int i = 0; i < MI16; ++i) sav[i] = MX ? 1.0f : sa[era == 1 ? min(wrow0 + i * 16 + fr, M - 1) : 0];
    float rq = 1.0f;
    if constexpr (OUT >= kOutE4M3) rq = ry ? ry[0] : 1.0f / sy[0];
    // the whole block tile inside (M, N): every wave takes the same branch
    // (store_tile holds barriers)
    if (OUT >= kOutE4M3 && m0 + TM <= M && n0 + TN <= N)
      store_tile<OUT, false>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wrow0, wcol0, M, N, Y, ldy, vec_store,
                                 wn, fr, fg, lane, rq, mb, sat_l, under_l);
    else
      store_tile<OUT, true>(acc, stage, &sCol[0][0], &sCol[1][0], sav, wrow0, wcol0, M, N, Y, ldy, vec_store,
                                wn, fr, fg, lane, rq, mb, sat_l, under_l);
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
    const float sav = sa ? sa[era == 1 ? row : 0] : 1.0f;  // null: applied inside the MFMA (1x32 scales)
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t cc = min(col + e, N - 1);
      float bv = 0.0f;
      if (bias)
        bv = bias_bf16 ? __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(bias)[cc]) << 16)
                       : static_cast<const float*>(bias)[cc];
      v[e] = acc[e] * (sav * (sb ? sb[erb == 1 ? cc : 0] : 1.0f)) + bv;
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

// 1x32 power-of-two scales (fp32, [rows][K / 32]) as the exponent bytes that
// k_gemm_big16 reads: u32x2 [row / 128][stage][lane], byte i (0-7) the
// exponent of row 128 (row / 128) + 16 i + lane % 16 and K block
// 4 stage + lane / 16.  Rows past the end get exponent 127 (scale 1); their
// products are never stored.
__global__ __launch_bounds__(256) void k_pack_e8m0_16(const float* __restrict__ s, int64_t rows, int64_t nblk,
                                                      int64_t nrb, int64_t nstage, u32x2* __restrict__ out) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= nrb * nstage * 64) return;
  const int64_t lane = idx & 63, rs = idx >> 6;
  const int64_t st = rs % nstage, rb = rs / nstage;
  const int64_t kb = st * 4 + (lane >> 4);
  uint32_t w0 = 0, w1 = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t row = rb * WTM + 16 * i + (lane & 15);
    const uint32_t e = row < rows ? (reinterpret_cast<const uint32_t*>(s)[row * nblk + kb] >> 23) & 0xFFu : 127u;
    if (i < 4) w0 |= e << (8 * i);
    else w1 |= e << (8 * (i - 4));
  }
  out[idx] = u32x2{w0, w1};
}

}  // namespace

bool gemm_big_eligible(const GemmArgs& g) {
  // per-tensor or per-row scales only (the epilogue selects, it does not divide)
  const bool rows_ok = (g.era == 1 || g.era >= g.M) && (g.erb == 1 || g.erb >= g.N);
  const bool scales_ok = g.pow2_mx ? (g.era == 1 && g.erb == 1 && g.eca == 32 && g.ecb == 32)
                                   : (g.eca >= g.K && g.ecb >= g.K);
  // M from 65 (below, the decode kernel): a few hundred rows make a grid of
  // fewer tiles than CUs, which the launch splits along K
  return rows_ok && scales_ok && g.K % (2 * TKS) == 0 && g.M >= 65 &&
         g.N >= 128 && g.lda < (int64_t(1) << 23) && g.ldb < (int64_t(1) << 23);
}

size_t gemm_big_required_scratch(const GemmArgs& g) {
  if (!g.pow2_mx) return 0;
  // whole 256-row tiles: a last tile's second wave reads its own (padding) block
  const int64_t ns = g.K / TKS, ra = (g.M + TM - 1) / TM * (TM / WTM), rb = (g.N + TN - 1) / TN * (TN / WTN);
  return (static_cast<size_t>((ra + rb) * ns * 64) * 8 + 255) & ~size_t(255);  // E8M0 exponent bytes
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
  // A grid of at most half the CUs in all (a few hundred rows of A) is one
  // such wave: every tile is split, into up to 8 parts.
  // One scratch region holds both: the repacked 1x32 exponents (MX) first,
  // then the FP32 K-parts of split tiles (256-byte aligned).
  const size_t mx_bytes = (gemm_big_required_scratch(g) + 255) & ~size_t(255);
  int t_main = T, split = 1, ns_part = 0;
  size_t part_total = 0;
  {
    const int cus = device_cus();
    const bool small = 2 * T <= cus;
    const int rem = small ? T : T % cus;
    const int64_t ns = g.K / TKS;
    // FP8 output: one statistics slot per whole tile and per reduce block
    const bool slots_ok = okind < kOutE4M3 || (T - rem) + rem * kRedBlocks <= kMaxBlocks;
    if (slots_ok && (small || (T > cus && rem > 0 && 2 * rem <= cus))) {
      const size_t part_bytes = static_cast<size_t>(rem) * TM * TN * sizeof(float);  // per K part
      int sp = std::min(cus / rem, small ? 8 : 4);
      if (g.fixed_scratch)  // a fixed buffer: as many parts as fit beside the exponents
        sp = static_cast<int>(std::min<size_t>(
            sp, g.fixed_scratch_bytes > mx_bytes ? (g.fixed_scratch_bytes - mx_bytes) / part_bytes : 0));
      while (sp > 1 && ns % (2 * sp) != 0) --sp;  // every part an even number of stages
      if (sp > 1) {
        split = sp;
        t_main = T - rem;
        ns_part = static_cast<int>(ns / sp);
        part_total = part_bytes * sp;
      }
    }
  }
  uint8_t* scratch = nullptr;
  if (mx_bytes + part_total > 0) {
    void* p = nullptr;
    hipError_t e = gemm_scratch(g, st, mx_bytes + part_total, &p);
    if (e != hipSuccess) return e;
    scratch = static_cast<uint8_t*>(p);
  }
  float* part = split > 1 ? reinterpret_cast<float*>(scratch + mx_bytes) : nullptr;
  const dim3 grid(static_cast<unsigned>(t_main + (T - t_main) * split));
  u32x2* xpa16 = nullptr;
  u32x2* xpb16 = nullptr;
  if (g.pow2_mx) {
    // whole 256-row tiles: a last tile's second wave reads its own (padding) block
    const int64_t ns = g.K / TKS, ra = (g.M + TM - 1) / TM * (TM / WTM), rb = (g.N + TN - 1) / TN * (TN / WTN);
    xpa16 = reinterpret_cast<u32x2*>(scratch);
    xpb16 = xpa16 + ra * ns * 64;
    hipLaunchKernelGGL(k_pack_e8m0_16, dim3(static_cast<unsigned>((ra * ns * 64 + 255) / 256)), dim3(256), 0, st,
                       g.sa, g.M, g.K / 32, ra, ns, xpa16);
    hipLaunchKernelGGL(k_pack_e8m0_16, dim3(static_cast<unsigned>((rb * ns * 64 + 255) / 256)), dim3(256), 0, st,
                       g.sb, g.N, g.K / 32, rb, ns, xpb16);
  }
#define FP8RT_BIG16(FA, FB, OUT, MXV)                                                                         \
  hipLaunchKernelGGL((k_gemm_big16<FA, FB, OUT, MXV, kRowB16>), grid, dim3(kThreads), 0, st, g.a, g.lda, g.b,  \
                     g.ldb, g.M, g.N, g.K, g.sa, g.era, g.sb, g.erb, g.bias, bb, g.y, g.ldy, tiles_m, tiles_n,  \
                     vec, t_main, split, ns_part, part, g.sy, g.ry, g.part, xpa16, xpb16)
#define FP8RT_BIG16_OUT(FA, FB, MXV)                                \
  switch (okind) {                                                  \
    case kOutBF16: FP8RT_BIG16(FA, FB, kOutBF16, MXV); break;       \
    case kOutE4M3: FP8RT_BIG16(FA, FB, kOutE4M3, MXV); break;       \
    case kOutE5M2: FP8RT_BIG16(FA, FB, kOutE5M2, MXV); break;       \
    default: FP8RT_BIG16(FA, FB, kOutF32, MXV); break;              \
  }
  if (g.fa == FP8RT_E4M3) {
    if (g.pow2_mx) { FP8RT_BIG16_OUT(0, 0, true) } else { FP8RT_BIG16_OUT(0, 0, false) }
  } else {
    if (g.pow2_mx) { FP8RT_BIG16_OUT(1, 0, true) } else { FP8RT_BIG16_OUT(1, 0, false) }
  }
#undef FP8RT_BIG16_OUT
#undef FP8RT_BIG16
  if (split > 1) {
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_split_reduce(g, st, part, t_main, split, tiles_m, tiles_n, g.pow2_mx ? nullptr : g.sa,
                            g.pow2_mx ? nullptr : g.sb, vec);
    if (e != hipSuccess) return e;
  }
  if (nparts) *nparts = split > 1 ? t_main + (T - t_main) * kRedBlocks : T;
  return hipGetLastError();
}

hipError_t launch_split_reduce(const GemmArgs& g, hipStream_t st, const float* part, int t_main, int split,
                               int tiles_m, int tiles_n, const float* sa, const float* sb, int vec) {
  const int T = tiles_m * tiles_n;
  const int bb = g.bias_t == FP8RT_BF16 ? 1 : 0;
  const dim3 rgrid(kRedBlocks, static_cast<unsigned>(T - t_main));
#define FP8RT_RED(OUT)                                                                                          \
  hipLaunchKernelGGL(k_split_reduce<OUT>, rgrid, dim3(256), 0, st, part, t_main, split, tiles_m, tiles_n, g.M, \
                     g.N, sa, g.era, sb, g.erb, g.bias, bb, g.y, g.ldy, vec, g.sy, g.ry, g.part)
  switch (gemm_out_kind(g)) {
    case kOutBF16: FP8RT_RED(kOutBF16); break;
    case kOutE4M3: FP8RT_RED(kOutE4M3); break;
    case kOutE5M2: FP8RT_RED(kOutE5M2); break;
    default: FP8RT_RED(kOutF32); break;
  }
#undef FP8RT_RED
  return hipGetLastError();
}

}  // namespace fp8rt
