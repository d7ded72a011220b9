// quant_kernels.hip -- amax reduction, scale, saturating FP8 cast, dequantize
// and the delayed-scaling history update for gfx950.
//
// Method ("FP8 formats and scaling for LLM inference"):
//   section "How a scale fits a tensor into E4M3": a_max = max|X|,
//     s = a_max / F_max, X_fp8 = cast(clip(X / s)), X_hat = s X_fp8;
//   section "Per-channel and block scaling": one scale per row / block,
//     s_g = a_g / F_max;
//   section "Current scaling": reduce amax -> scale -> cast in the same step;
//   section "Delayed scaling": s_{t+1} = f(a_t .. a_{t-h+1}) / F_max;
//   section "What numerical validation looks at": saturation and underflow
//     rates.
// "FP8 production quantization guide", dynamic quantize listing: eps clamp of
// amax, x * inv_scale, clamp to +-F_max, cast.
//
// Design (HBM-bound work): 16-byte loads of 8-element octets, exact integer
// max on |x| bit patterns, one FP32 multiply, a clamp and the packed
// v_cvt_pk_{fp8,bf8}_f32 convert per element; 8-byte code stores.  Group
// maxima are reduced across lanes with shuffles and across a workgroup in LDS.
// Cross-block results (per-tensor amax, counters) go through per-block
// partials in a per-stream device workspace, written with plain stores and
// combined by the next kernel on the stream.  Device-scope fences and
// same-address atomics are avoided: with one L2 per XCD they cost more than
// a small extra launch.
#include <float.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace fp8rt {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / 64;

template <typename T> constexpr int oct_unroll() { return sizeof(T) == 2 ? 4 : 2; }

// Block-wide max (all threads receive it).  Uses sh[kWaves].
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* sh) {
  v = wave_max_u32(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) sh[w] = v;
  __syncthreads();
  uint32_t m = sh[0];
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = max(m, sh[i]);
  return m;
}

// Writes this block's partial: the block max of the lane amax bits mb and
// the block sums of the per-lane counters sat_l / under_l.
__device__ __forceinline__ void store_block_partial(BlockPartial* bp, uint32_t mb, uint32_t sat_l,
                                                   uint32_t under_l) {
  __shared__ uint32_t sh_m[kWaves];
  __shared__ unsigned long long sh_s[kWaves], sh_u[kWaves];
  mb = wave_max_u32(mb);
  const unsigned long long sat_w = wave_sum_u64(sat_l), under_w = wave_sum_u64(under_l);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh_m[w] = mb;
    sh_s[w] = sat_w;
    sh_u[w] = under_w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = 0;
    unsigned long long s = 0, u = 0;
    for (int i = 0; i < kWaves; ++i) {
      m = max(m, sh_m[i]);
      s += sh_s[i];
      u += sh_u[i];
    }
    *reinterpret_cast<u32x4*>(&bp[blockIdx.x]) =
        u32x4{m, static_cast<uint32_t>(s), static_cast<uint32_t>(u), 0u};
  }
}

// Converts one octet with multiplier r; returns the 8 codes as two words and
// adds this lane's saturation / underflow counts.
template <typename T, int F, bool STATS>
__device__ __forceinline__ u32x2 cast_octet(const Octet<T>& v, float r, bool nan_path, uint32_t& sat_l,
                                            uint32_t& under_l) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v.get(i) * r;
  u32x2 out;
  if (nan_path) {
    out[0] = cvt4_nan<F>(f[0], f[1], f[2], f[3]);
    out[1] = cvt4_nan<F>(f[4], f[5], f[6], f[7]);
  } else {
    out[0] = cvt4<F>(f[0], f[1], f[2], f[3]);
    out[1] = cvt4<F>(f[4], f[5], f[6], f[7]);
  }
  if constexpr (STATS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sat_l += fabsf(f[i]) > Fmt<F>::kMax ? 1u : 0u;
      under_l += (v.get(i) != 0.0f && fabsf(f[i]) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
    }
  }
  return out;
}

// ---------------------------------------------------------------------------
// Per-tensor, pass 1: one amax partial per block.  The work is split in
// segments of kBlock * U octets of one row.

template <typename T>
__global__ __launch_bounds__(kBlock) void k_tensor_amax(const T* __restrict__ x, int64_t rows,
                                                        int64_t opr, int64_t ldx,
                                                        int64_t segs_per_row,
                                                        BlockPartial* __restrict__ part,
                                                        unsigned long long* zero_counts) {
  // the cast pass of a small grid adds its counts straight into these
  if (zero_counts && blockIdx.x == 0 && threadIdx.x < 2) zero_counts[threadIdx.x] = 0ull;
  constexpr int U = oct_unroll<T>();
  __shared__ uint32_t sh[kWaves];
  uint32_t m = 0;
  const int64_t nseg = rows * segs_per_row;
  for (int64_t sg = blockIdx.x; sg < nseg; sg += gridDim.x) {
    const int64_t r = sg / segs_per_row;
    const int64_t s = sg - r * segs_per_row;
    const T* xr = x + r * ldx;
    Octet<T> v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (s * U + u) * kBlock + threadIdx.x;
      v[u].load_nt(xr + min(o, opr - 1) * 8);
      v[u].keep_if(o < opr);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) m = max(m, v[u].absmax_bits());
  }
  m = block_max_u32(m, sh);
  if (threadIdx.x == 0) part[blockIdx.x].amax_bits = m;
}

// Byte offset of the 8 codes that start at (row, col), col a multiple of 8:
// row-major with pitch ldq when img == 0; else in the fragment-ordered
// weight image of a matrix with 128 img columns, whose 16-row group G,
// 128-deep step s, half h, lane l and byte b sit at
// ((G img + s) 2 + h) 1024 + 16 l + b, with l = 16 ((col / 32) % 4) +
// row % 16, h = (col / 16) % 2 and b = col % 16 (8 codes never straddle
// two 16-byte slots).
__device__ __forceinline__ int64_t code_off(int64_t row, int64_t col, int64_t ldq, int64_t img) {
  if (img == 0) return row * ldq + col;
  const int64_t l = (((col >> 5) & 3) << 4) | (row & 15);
  return (((row >> 4) * img + (col >> 7)) * 2 + ((col >> 4) & 1)) * 1024 + (l << 4) + (col & 15);
}

// The 8 codes c at q + off.  Row-major codes stream out (nontemporal); the
// image's 128-byte lines each take 16 bytes from 8 rows, so its stores stay
// in L2 until the other rows' bytes have joined them.
__device__ __forceinline__ void store_codes(uint8_t* q, int64_t off, u32x2 c, int64_t img) {
  if (img == 0) __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(q + off));
  else *reinterpret_cast<u32x2*>(q + off) = c;
}

// First work item of this workgroup in a grid-stride loop.  Image mode, on
// a grid that is a multiple of 8: workgroup b starts at (b % 8) (grid / 8) +
// b / 8, so the workgroups of each XCD (dealt round-robin) take a contiguous
// run of items, and the 16 rows of an image group are cast by one XCD at
// about the same time and meet in its L2.
__device__ __forceinline__ int64_t first_item(int64_t img) {
  if (img == 0 || (gridDim.x & 7u) != 0) return blockIdx.x;
  return static_cast<int64_t>(blockIdx.x & 7u) * (gridDim.x >> 3) + (blockIdx.x >> 3);
}

// Pass 2 of DYNAMIC (every block combines the pass-1 partials and derives
// (s, r) itself; block 0 writes scale / inv_scale / amax_out) or the single
// pass of GIVEN mode.  Counters and the observed amax go to per-block
// partials for the finisher.
template <typename T, int F, bool GIVEN, bool STATS, bool AMAX, bool IMG>
__global__ __launch_bounds__(kBlock) void k_tensor_cast(
    const T* __restrict__ x, int64_t rows, int64_t opr, int64_t ldx, int64_t segs_per_row,
    uint8_t* __restrict__ q, int64_t ldq, int64_t img, const BlockPartial* __restrict__ part1, int nparts,
    float eps, int pow2, const float* __restrict__ s_in, const float* __restrict__ r_in,
    float* s_out, float* r_out, float* amax_out, BlockPartial* __restrict__ part2,
    unsigned long long* acc_counts) {
  constexpr int U = oct_unroll<T>();
  __shared__ uint32_t sh[kWaves];
  const int64_t nseg = rows * segs_per_row;
  Octet<T> v[U];
  auto load_seg = [&](int64_t sg) {
    const int64_t rr = sg / segs_per_row;
    const int64_t sr = sg - rr * segs_per_row;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (sr * U + u) * kBlock + threadIdx.x;
      v[u].load_nt(x + rr * ldx + min(o, opr - 1) * 8);  // clamped: every load stays in flight
    }
  };
  // the first segment's loads fly while the scale is derived from the partials
  const int64_t sg0 = IMG ? first_item(img) : blockIdx.x;
  if (sg0 < nseg) load_seg(sg0);
  float r;
  if constexpr (!GIVEN) {
    uint32_t m = 0;
    for (int i = threadIdx.x; i < nparts; i += 4 * kBlock) {  // four partials in flight per thread
      uint32_t b[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) b[k] = part1[min(i + k * kBlock, nparts - 1)].amax_bits;  // clamped: a repeat
#pragma unroll
      for (int k = 0; k < 4; ++k) m = max(m, b[k]);
    }
    m = block_max_u32(m, sh);
    const float a = __uint_as_float(m);
    float s;
    scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, s, r);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      s_out[0] = s;
      if (r_out) r_out[0] = r;
      if (amax_out) amax_out[0] = a;
    }
  } else {
    const float s = s_in[0];
    r = r_in ? r_in[0] : 1.0f / s;
  }
  const bool r_bad = !(fabsf(r) <= FLT_MAX);
  uint32_t mb = 0;
  uint32_t sat_l = 0, under_l = 0;
  for (int64_t sg = sg0; sg < nseg; sg += gridDim.x) {
    const int64_t rr = sg / segs_per_row;
    const int64_t s = sg - rr * segs_per_row;
    uint8_t* qr = q + rr * ldq;
    if (sg != sg0) load_seg(sg);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t o = (s * U + u) * kBlock + threadIdx.x;
      if (o < opr) {
        bool nan_path = r_bad;
        if constexpr (GIVEN) {
          const uint32_t omb = v[u].absmax_bits();
          if constexpr (AMAX) mb = max(mb, omb);
          nan_path |= omb > kInfBits;
        }
        const u32x2 c = cast_octet<T, F, STATS>(v[u], r, nan_path, sat_l, under_l);
        if constexpr (IMG) store_codes(q, code_off(rr, o * 8, ldq, img), c, img);
        else __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(qr + o * 8));
      }
    }
  }
  if constexpr (STATS && !GIVEN) {
    if (acc_counts) {
      // a small grid: one device-scope add per block and counter instead of
      // a finisher launch (the amax pass zeroed the counters)
      __shared__ unsigned long long sh_s[kWaves], sh_u[kWaves];
      const unsigned long long sw = wave_sum_u64(sat_l), uw = wave_sum_u64(under_l);
      if ((threadIdx.x & 63) == 0) {
        sh_s[threadIdx.x >> 6] = sw;
        sh_u[threadIdx.x >> 6] = uw;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        unsigned long long st = 0, ut = 0;
        for (int i = 0; i < kWaves; ++i) {
          st += sh_s[i];
          ut += sh_u[i];
        }
        atomicAdd(&acc_counts[0], st);
        atomicAdd(&acc_counts[1], ut);
      }
      return;
    }
  }
  if constexpr (STATS || AMAX) store_block_partial(part2, mb, sat_l, under_l);
}

// Combines n block partials into amax_out[0] (as binary32, if non-null) and
// counts[0..1] (if non-null).  One workgroup of 1024 threads, four partials
// (16-byte loads) in flight per thread.
constexpr int kFinThreads = 1024;
__global__ __launch_bounds__(kFinThreads) void k_finish(const BlockPartial* __restrict__ bp, int n,
                                                        float* amax_out, unsigned long long* counts) {
  __shared__ uint32_t sh_m[kFinThreads / 64];
  __shared__ unsigned long long sh_s[kFinThreads / 64], sh_u[kFinThreads / 64];
  uint32_t m = 0;
  unsigned long long s = 0, u = 0;
  for (int i = threadIdx.x; i < n; i += 4 * kFinThreads) {
    u32x4 w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) w[k] = *reinterpret_cast<const u32x4*>(&bp[min(i + k * kFinThreads, n - 1)]);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const bool in = i + k * kFinThreads < n;  // the clamped repeats add no counts
      m = max(m, w[k][0]);
      s += in ? w[k][1] : 0u;
      u += in ? w[k][2] : 0u;
    }
  }
  m = wave_max_u32(m);
  s = wave_sum_u64(s);
  u = wave_sum_u64(u);
  if ((threadIdx.x & 63) == 0) {
    sh_m[threadIdx.x >> 6] = m;
    sh_s[threadIdx.x >> 6] = s;
    sh_u[threadIdx.x >> 6] = u;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tm = 0;
    unsigned long long ts = 0, tu = 0;
    for (int i = 0; i < kFinThreads / 64; ++i) {
      tm = max(tm, sh_m[i]);
      ts += sh_s[i];
      tu += sh_u[i];
    }
    if (amax_out) amax_out[0] = __uint_as_float(tm);
    if (counts) {
      counts[0] = ts;
      counts[1] = tu;
    }
  }
}

// ---------------------------------------------------------------------------
// Row groups: groups of one row and L octets (8L elements, L a power of two,
// 2 <= L <= 64).  Each row is padded to nCg * L octets so every group spans
// exactly L lanes; padding and ragged tail octets load as zero and are not
// stored.  A unit of kBlock * U padded octets holds kBlock * U / L groups:
// lanes reduce their group's maximum with shuffles, one thread per group
// computes (s, r) into LDS, then every lane casts its octets.

template <typename T, int F, int L, bool GIVEN, bool STATS, bool AMAX_ONLY, bool IMG>
__global__ __launch_bounds__(kBlock) void k_rowgroups(
    const T* __restrict__ x, uint32_t rows, uint32_t oct_cols, int64_t ldx, FastDiv div_opr,
    uint32_t nCg, uint32_t units, uint8_t* __restrict__ q, int64_t ldq, int64_t img, float eps, int pow2,
    float* s_io, float* r_io, float* amax_out, DevWorkspace* ws, unsigned long long* counts) {
  constexpr int U = sizeof(T) == 2 ? 8 : 4;
  constexpr int GPU = kBlock * U / L;  // groups per unit
  __shared__ uint32_t sh_amax[GPU];
  __shared__ float sh_r[GPU];
  const uint32_t opr = nCg * L;
  const int t = threadIdx.x;
  uint32_t sat_l = 0, under_l = 0;
  for (uint32_t unit = IMG ? static_cast<uint32_t>(first_item(img)) : blockIdx.x; unit < units; unit += gridDim.x) {
    const uint32_t base = unit * (kBlock * U);
    Octet<T> v[U];
    uint32_t omb[U];
    uint32_t row[U], oc[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t po = base + u * kBlock + t;
      row[u] = div_opr.div(po);
      oc[u] = po - row[u] * opr;
      const bool ok = row[u] < rows && oc[u] < oct_cols;
      v[u].load_nt(x + static_cast<int64_t>(min(row[u], rows - 1)) * ldx + min(oc[u], oct_cols - 1) * 8);
      v[u].keep_if(ok);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      omb[u] = v[u].absmax_bits();
      const uint32_t gm = segment_max_u32<L>(omb[u]);
      if ((t & (L - 1)) == 0) sh_amax[(u * kBlock + t) / L] = gm;
    }
    __syncthreads();
    for (int gi = t; gi < GPU; gi += kBlock) {
      const uint32_t po = base + gi * L;
      const uint32_t gr = div_opr.div(po);
      if (gr < rows) {
        const uint32_t cg = (po - gr * opr) / L;
        const int64_t g = static_cast<int64_t>(gr) * nCg + cg;
        const float a = __uint_as_float(sh_amax[gi]);
        if (amax_out) amax_out[g] = a;
        if constexpr (!AMAX_ONLY) {
          float s, r;
          if constexpr (GIVEN) {
            s = s_io[g];
            r = r_io ? r_io[g] : 1.0f / s;
          } else {
            scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, s, r);
            s_io[g] = s;
            if (r_io) r_io[g] = r;
          }
          sh_r[gi] = r;
        }
      }
    }
    if constexpr (!AMAX_ONLY) {
      __syncthreads();
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (row[u] < rows && oc[u] < oct_cols) {
          const float r = sh_r[(u * kBlock + t) / L];
          const bool nan_path = omb[u] > kInfBits || !(fabsf(r) <= FLT_MAX);
          const u32x2 c = cast_octet<T, F, STATS>(v[u], r, nan_path, sat_l, under_l);
          if constexpr (IMG) store_codes(q, code_off(row[u], oc[u] * 8, ldq, img), c, img);
          else __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(q + static_cast<int64_t>(row[u]) * ldq + oc[u] * 8));
        }
      }
    }
    __syncthreads();
  }
  if constexpr (STATS) store_block_partial(ws->pass2, 0, sat_l, under_l);
}

// ---------------------------------------------------------------------------
// Block tiles: one workgroup per group of er x ec elements (any extents; the
// last group along each dimension may be short).  REG: the group fits in
// registers (<= kBlock * U octets) and is read once; otherwise it is read
// twice (max, then cast; the second read mostly hits L2).

template <typename T, int F, bool GIVEN, bool STATS, bool AMAX_ONLY, bool REG, bool IMG>
__global__ __launch_bounds__(kBlock) void k_blocktile(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, int64_t er, int64_t ec,
    int64_t nCg, int64_t ngroups, FastDiv div_full, FastDiv div_tail, uint8_t* __restrict__ q,
    int64_t ldq, int64_t img, float eps, int pow2, float* s_io, float* r_io, float* amax_out,
    DevWorkspace* ws, unsigned long long* counts) {
  constexpr int U = sizeof(T) == 2 ? 8 : 4;
  __shared__ uint32_t sh[kWaves];
  __shared__ float sh_r;
  const int t = threadIdx.x;
  uint32_t sat_l = 0, under_l = 0;
  for (int64_t g = IMG ? first_item(img) : blockIdx.x; g < ngroups; g += gridDim.x) {
    const int64_t gi = g / nCg, gj = g - gi * nCg;
    const int64_t r0 = gi * er, c0 = gj * ec;
    const int64_t nr = min(er, rows - r0);
    const int64_t ncol = min(ec, cols - c0);
    const uint32_t oct_row = static_cast<uint32_t>(ncol / 8);
    const FastDiv& dv = (ncol == ec) ? div_full : div_tail;
    const uint32_t n_oct = static_cast<uint32_t>(nr) * oct_row;
    const T* xg = x + r0 * ldx + c0;
    uint8_t* qg = q + r0 * ldq + c0;
    uint32_t mb = 0;
    Octet<T> v[REG ? U : 1];
    if constexpr (REG) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const uint32_t o = u * kBlock + t;
        const uint32_t oc = min(o, n_oct - 1);
        const uint32_t rr = dv.div(oc), cc = oc - rr * oct_row;
        v[u].load_nt(xg + static_cast<int64_t>(rr) * ldx + cc * 8);
        v[u].keep_if(o < n_oct);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) mb = max(mb, v[u].absmax_bits());
    } else {
      for (uint32_t o = t; o < n_oct; o += kBlock) {
        const uint32_t rr = dv.div(o), cc = o - rr * oct_row;
        v[0].load(xg + static_cast<int64_t>(rr) * ldx + cc * 8);
        mb = max(mb, v[0].absmax_bits());
      }
    }
    const uint32_t gmb = block_max_u32(mb, sh);
    const float a = __uint_as_float(gmb);
    if (t == 0) {
      if (amax_out) amax_out[g] = a;
      if constexpr (!AMAX_ONLY) {
        float s, r;
        if constexpr (GIVEN) {
          s = s_io[g];
          r = r_io ? r_io[g] : 1.0f / s;
        } else {
          scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, s, r);
          s_io[g] = s;
          if (r_io) r_io[g] = r;
        }
        sh_r = r;
      }
    }
    if constexpr (!AMAX_ONLY) {
      __syncthreads();
      const float r = sh_r;
      const bool r_bad = !(fabsf(r) <= FLT_MAX);
      if constexpr (REG) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const uint32_t o = u * kBlock + t;
          if (o < n_oct) {
            const uint32_t rr = dv.div(o), cc = o - rr * oct_row;
            const bool nan_path = r_bad || v[u].absmax_bits() > kInfBits;
            const u32x2 c = cast_octet<T, F, STATS>(v[u], r, nan_path, sat_l, under_l);
            if constexpr (IMG) store_codes(q, code_off(r0 + rr, c0 + cc * 8, ldq, img), c, img);
            else __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(qg + static_cast<int64_t>(rr) * ldq + cc * 8));
          }
        }
      } else {
        for (uint32_t o = t; o < n_oct; o += kBlock) {
          const uint32_t rr = dv.div(o), cc = o - rr * oct_row;
          v[0].load_nt(xg + static_cast<int64_t>(rr) * ldx + cc * 8);
          const bool nan_path = r_bad || v[0].absmax_bits() > kInfBits;
          const u32x2 c = cast_octet<T, F, STATS>(v[0], r, nan_path, sat_l, under_l);
          if constexpr (IMG) store_codes(q, code_off(r0 + rr, c0 + cc * 8, ldq, img), c, img);
            else __builtin_nontemporal_store(c, reinterpret_cast<u32x2*>(qg + static_cast<int64_t>(rr) * ldq + cc * 8));
        }
      }
    }
    __syncthreads();
  }
  if constexpr (STATS) store_block_partial(ws->pass2, 0, sat_l, under_l);
}


// ---------------------------------------------------------------------------
// Quantize straight into the weight image, with one scale per row or per
// tensor, for K up to 128 x 16 x NS.  One workgroup of 16 waves per 16-row
// group; wave w holds the group's steps w, w + 16, ... (NS at most) in
// registers.  A step (16 rows x 128 values) is read as whole row segments:
// load u of lane l takes row 4 u + l / 16, values 8 (l % 16) .. +8, so each
// load instruction reads 4 contiguous row segments.  Per-row scales: row
// maxima over the 16 lanes of a segment (shuffles) and the 16 waves (LDS),
// then (s, r) of each row; per tensor: r from the given scale or from the
// amax pass's partials.  The codes of a step go through the wave's own
// 16 x 128-byte LDS tile (row pitch 144 bytes, so the 16 rows of a read fall
// in different banks) and come back in the image's lane order -- lane l:
// row l % 16, bytes 32 (l / 16) .. +32 -- so each wave stores two contiguous
// 1 KB runs per step.  Rows past the end load as zeros and leave zero codes,
// uncounted.

constexpr int kImgWaves = 16;
constexpr int kImgPitch = 144;

template <typename T, int F, int NS, bool ROW, bool GIVEN, bool STATS, bool AMAX>
__global__ __launch_bounds__(kImgWaves * 64) void k_image_rows(
    const T* __restrict__ x, int64_t rows, int64_t steps, int64_t ldx, uint8_t* __restrict__ qp,
    const BlockPartial* __restrict__ part1, int nparts, float eps, int pow2, float* s_io, float* r_io,
    float* amax_out, BlockPartial* __restrict__ part2) {
  __shared__ uint32_t sh_m[kImgWaves][16];
  __shared__ float sh_r[16];
  __shared__ unsigned long long sh_s[kImgWaves], sh_u[kImgWaves];
  __shared__ __attribute__((aligned(16))) uint8_t tile[kImgWaves][16 * kImgPitch];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int seg = lane & 15, rq = lane >> 4;  // loads: value octet seg of rows 4 u + rq
  const int64_t G = blockIdx.x;
  Octet<T> v[NS][4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t row = G * 16 + 4 * u + rq;
    const T* xr = x + min(row, rows - 1) * ldx + 8 * seg;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const int64_t st = wave + j * kImgWaves;
      v[j][u].load_nt(xr + min(st, steps - 1) * 128);  // clamped: every load stays in flight
      v[j][u].keep_if(row < rows && st < steps);
    }
  }
  uint32_t mb = 0;  // this lane's max |x| bits
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int u = 0; u < 4; ++u) mb = max(mb, v[j][u].absmax_bits());
  float r[4];  // multiplier of each of the lane's 4 rows
  if constexpr (ROW) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t m = 0;
#pragma unroll
      for (int j = 0; j < NS; ++j) m = max(m, v[j][u].absmax_bits());
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) m = max(m, static_cast<uint32_t>(__shfl_xor(static_cast<int>(m), o)));
      if (seg == 0) sh_m[wave][4 * u + rq] = m;
    }
    __syncthreads();
    if (threadIdx.x < 16) {
      uint32_t am = sh_m[0][threadIdx.x];
#pragma unroll
      for (int i = 1; i < kImgWaves; ++i) am = max(am, sh_m[i][threadIdx.x]);
      const int64_t rr = G * 16 + threadIdx.x;
      float sv = 1.0f, rv = 1.0f;
      if (rr < rows) {
        const float a = __uint_as_float(am);
        if (amax_out) amax_out[rr] = a;
        if constexpr (GIVEN) {
          sv = s_io[rr];
          rv = r_io ? r_io[rr] : 1.0f / sv;
        } else {
          scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, sv, rv);
          s_io[rr] = sv;
          if (r_io) r_io[rr] = rv;
        }
      }
      sh_r[threadIdx.x] = rv;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = sh_r[4 * u + rq];
  } else {
    float rt;
    if constexpr (GIVEN) {
      rt = r_io ? r_io[0] : 1.0f / s_io[0];
    } else {
      // the tensor's amax from the amax pass's partials
      uint32_t m = 0;
      for (int i = threadIdx.x; i < nparts; i += kImgWaves * 64) m = max(m, part1[i].amax_bits);
      m = wave_max_u32(m);
      if (lane == 0) sh_m[wave][0] = m;
      __syncthreads();
      m = sh_m[0][0];
#pragma unroll
      for (int i = 1; i < kImgWaves; ++i) m = max(m, sh_m[i][0]);
      const float a = __uint_as_float(m);
      float sv;
      scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, sv, rt);
      if (blockIdx.x == 0 && threadIdx.x == 0) {
        s_io[0] = sv;
        if (r_io) r_io[0] = rt;
        if (amax_out) amax_out[0] = a;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = rt;
  }
  uint32_t sat_l = 0, under_l = 0;
  uint8_t* wt = tile[wave];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int64_t st = wave + j * kImgWaves;
    if (st < steps) {  // wave-uniform
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const bool nan_path = !(fabsf(r[u]) <= FLT_MAX) || v[j][u].absmax_bits() > kInfBits;
        const u32x2 c = cast_octet<T, F, STATS>(v[j][u], r[u], nan_path, sat_l, under_l);
        // the counters pass through an opaque copy per octet: otherwise the
        // increments of the unrolled octets are reassociated into one tree
        // that keeps every product live (126 instead of 104 VGPRs at three
        // steps per wave; spills at four)
        if constexpr (STATS) asm volatile("" : "+v"(sat_l), "+v"(under_l));
        *reinterpret_cast<u32x2*>(wt + (4 * u + rq) * kImgPitch + 8 * seg) = c;
      }
      // the wave's own tile: its LDS operations complete in order
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const uint8_t* src = wt + (lane & 15) * kImgPitch + 32 * (lane >> 4);
      const u32x4 h0 = *reinterpret_cast<const u32x4*>(src);
      const u32x4 h1 = *reinterpret_cast<const u32x4*>(src + 16);
      uint8_t* dst = qp + (G * steps + st) * 2048 + lane * 16;
      __builtin_nontemporal_store(h0, reinterpret_cast<u32x4*>(dst));
      __builtin_nontemporal_store(h1, reinterpret_cast<u32x4*>(dst + 1024));
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
  if constexpr (STATS || (AMAX && !ROW)) {
    // this workgroup's partial: max |x| bits and the counts
    const uint32_t mw = wave_max_u32(mb);
    const unsigned long long sw = wave_sum_u64(sat_l), uw = wave_sum_u64(under_l);
    __syncthreads();  // sh_m may still be read above
    if (lane == 0) {
      sh_m[wave][0] = mw;
      sh_s[wave] = sw;
      sh_u[wave] = uw;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t m = 0;
      unsigned long long sa = 0, ua = 0;
      for (int i = 0; i < kImgWaves; ++i) {
        m = max(m, sh_m[i][0]);
        sa += sh_s[i];
        ua += sh_u[i];
      }
      *reinterpret_cast<u32x4*>(&part2[blockIdx.x]) =
          u32x4{m, static_cast<uint32_t>(sa), static_cast<uint32_t>(ua), 0u};
    }
  }
}

// ---------------------------------------------------------------------------
// Cast-transpose: the cast of the quantize kernels, with every code written
// twice: row-major to q and transposed (K-major) to qt.  GIVEN scales only
// (the host runs the amax and scale kernels first in DYNAMIC mode).  Groups:
// GK 0 tensor, 1 row, 2 column.  128 x 128 tiles: 16-byte loads of 8
// elements, 8-byte row-major code stores, byte writes into an LDS tile kept
// transposed (132-byte pitch: lanes of one write instruction fall in
// different banks), 16-byte K-major stores of whole 128-byte lines.

constexpr int kCtR = 128, kCtC = 128, kCtW = 132;

template <typename T, int F, bool STATS>
__device__ __forceinline__ u32x2 cast_octet_r8(const Octet<T>& v, const float (&r)[8], bool nan_path,
                                               uint32_t& sat_l, uint32_t& under_l) {
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = v.get(i) * r[i];
  // the NaN fix-up as selects, not a branch (a branch here keeps both paths'
  // values live and halves the occupancy of the cast-transpose kernel)
  (void)nan_path;
  u32x2 out;
  out[0] = cvt4_nan<F>(f[0], f[1], f[2], f[3]);
  out[1] = cvt4_nan<F>(f[4], f[5], f[6], f[7]);
  if constexpr (STATS) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sat_l += fabsf(f[i]) > Fmt<F>::kMax ? 1u : 0u;
      under_l += (v.get(i) != 0.0f && fabsf(f[i]) <= Fmt<F>::kZeroEdge) ? 1u : 0u;
    }
  }
  return out;
}

template <typename T, int F, int GK, bool STATS, bool AMAX>
__global__ __launch_bounds__(kBlock) void k_cast_transpose(
    const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx, const float* __restrict__ s_in,
    const float* __restrict__ r_in, uint8_t* __restrict__ q, int64_t ldq, uint8_t* __restrict__ qt,
    int64_t ldqt, int tiles_c, int ntiles, BlockPartial* __restrict__ part) {
  // [tile column][tile row] codes; a thread owns 4 consecutive tile rows of 8
  // columns per pass, so each column's 4 codes go to LDS as one word
  __shared__ __attribute__((aligned(16))) uint32_t tl[kCtC * kCtW / 4];
  auto rmul = [&](int64_t g) { return r_in ? r_in[g] : 1.0f / s_in[g]; };
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  uint32_t mb = 0, sat_l = 0, under_l = 0;
  for (int tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int tr = tile / tiles_c, tc = tile - tr * tiles_c;
    const int64_t r0 = static_cast<int64_t>(tr) * kCtR, c0 = static_cast<int64_t>(tc) * kCtC;
    const int64_t col = c0 + cg * 8;
    const bool col_ok = col < cols;
    const int64_t colc = min(col, cols - 8);
    float rv[8];
    bool rbad_c = false;
    if constexpr (GK == 0) {
      const float r = rmul(0);
#pragma unroll
      for (int k = 0; k < 8; ++k) rv[k] = r;
    } else if constexpr (GK == 2) {
#pragma unroll
      for (int k = 0; k < 8; ++k) rv[k] = rmul(colc + k);
    }
    if constexpr (GK != 1) {
#pragma unroll
      for (int k = 0; k < 8; ++k) rbad_c |= !(fabsf(rv[k]) <= FLT_MAX);
    }
    if (tile != static_cast<int>(blockIdx.x)) __syncthreads();  // the previous tile's LDS reads are done
    // tile row of pass p, row u of the thread: 64 p + 4 rl + u
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      Octet<T> v[1][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = r0 + 64 * p + 4 * rl + u;
        v[0][u].load_nt(x + min(row, rows - 1) * ldx + colc);  // clamped: every load stays in flight
        v[0][u].keep_if(col_ok && row < rows);
      }
      u32x2 c[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t row = r0 + 64 * p + 4 * rl + u;
        float rr[8];
        bool rbad = rbad_c;
        if constexpr (GK == 1) {
          const float r = rmul(min(row, rows - 1));
#pragma unroll
          for (int k = 0; k < 8; ++k) rr[k] = r;
          rbad = !(fabsf(r) <= FLT_MAX);
        } else {
#pragma unroll
          for (int k = 0; k < 8; ++k) rr[k] = rv[k];
        }
        const uint32_t omb = v[0][u].absmax_bits();
        if constexpr (AMAX) mb = max(mb, omb);
        c[u] = cast_octet_r8<T, F, STATS>(v[0][u], rr, rbad || omb > kInfBits, sat_l, under_l);
        if (col_ok && row < rows) __builtin_nontemporal_store(c[u], reinterpret_cast<u32x2*>(q + row * ldq + col));
        // the counters pass through an opaque copy per octet: otherwise the
        // 64 increments of a tile are reassociated into one tree that keeps
        // every product of the tile live (141 VGPRs, 3 waves per SIMD)
        if constexpr (STATS) asm volatile("" : "+v"(sat_l), "+v"(under_l));
      }
      // column k's codes of the 4 rows, packed row-ascending into one word
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int sh = 8 * (k & 3), wd = k >> 2;
        const uint32_t w = ((c[0][wd] >> sh) & 0xFFu) | (((c[1][wd] >> sh) & 0xFFu) << 8) |
                           (((c[2][wd] >> sh) & 0xFFu) << 16) | (((c[3][wd] >> sh) & 0xFFu) << 24);
        tl[(cg * 8 + k) * (kCtW / 4) + 16 * p + rl] = w;
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the next pass's loads here (registers)
    }
    __syncthreads();
    // qt row c0 + qc holds tile column qc: 8 parts of 16 codes (tile rows)
#pragma unroll
    for (int j = 0; j < kCtR * kCtC / 16 / kBlock; ++j) {
      const int id = j * kBlock + threadIdx.x;
      const int qc = id >> 3, pc = id & 7;
      const int64_t orow = c0 + qc, ocol = r0 + pc * 16;
      if (orow < cols && ocol < rows) {  // rows is a multiple of 16: a part is whole or absent
        const uint32_t* src = tl + qc * (kCtW / 4) + pc * 4;
        __builtin_nontemporal_store(u32x4{src[0], src[1], src[2], src[3]},
                                    reinterpret_cast<u32x4*>(qt + orow * ldqt + ocol));
      }
    }
  }
  if constexpr (STATS || AMAX) store_block_partial(part, mb, sat_l, under_l);
}

// Column maxima, pass 1: block (bx, by) takes columns [128 bx, +128) of rows
// [by rpc, +rpc): 16 x 16 threads (8 columns by every 16th row each, four
// rows in flight), reduced over the row lanes in LDS; one partial per (row
// chunk, column) as binary32 bits of |x| (NaN patterns exceed Inf).
template <typename T>
__global__ __launch_bounds__(kBlock) void k_col_amax(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                     int64_t ldx, int64_t rpc, uint32_t* __restrict__ part) {
  __shared__ uint32_t sh[16][129];
  const int cg = threadIdx.x & 15, rl = threadIdx.x >> 4;
  const int64_t c0 = static_cast<int64_t>(blockIdx.x) * 128;
  const int64_t colc = min(c0 + cg * 8, cols - 8);
  const int64_t rb0 = static_cast<int64_t>(blockIdx.y) * rpc, rb1 = min(rb0 + rpc, rows);
  uint32_t m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = rb0 + rl; r < rb1; r += 64) {
    Octet<T> v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u].load_nt(x + min(r + 16 * u, rb1 - 1) * ldx + colc);  // clamped: a repeat
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int k = 0; k < 8; ++k) m[k] = max(m[k], __float_as_uint(v[u].get(k)) & kAbsMask);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) sh[rl][cg * 8 + k] = m[k];
  __syncthreads();
  if (threadIdx.x < 128 && c0 + threadIdx.x < cols) {
    uint32_t mm = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) mm = max(mm, sh[i][threadIdx.x]);
    part[blockIdx.y * cols + c0 + threadIdx.x] = mm;
  }
}

__global__ __launch_bounds__(kBlock) void k_col_amax_finish(const uint32_t* __restrict__ part, int64_t nchunk,
                                                            int64_t cols, float* __restrict__ amax) {
  const int64_t c = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x;
  if (c >= cols) return;
  uint32_t m = 0;
  for (int64_t k = 0; k < nchunk; ++k) m = max(m, part[k * cols + c]);
  amax[c] = __uint_as_float(m);
}

// The per-column DYNAMIC finish in one launch: each column's amax from the
// nchunk row-chunk partials part[k][c] (wave w of a block reads chunks w,
// w + 4, ... of 64 consecutive columns: coalesced), the waves' maxima
// combined in LDS, then s and r of the column as k_compute_scale derives them;
// amax_out (nullable) receives the amax.
template <int F>
__global__ __launch_bounds__(kBlock) void k_col_amax_scale(const uint32_t* __restrict__ part, int64_t nchunk,
                                                           int64_t cols, float eps, int pow2, float* amax_out,
                                                           float* s_out, float* r_out) {
  __shared__ uint32_t sh[kWaves][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t c = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const int64_t cc = min(c, cols - 1);
  uint32_t m = 0;
  for (int64_t k = w; k < nchunk; k += kWaves) m = max(m, part[k * cols + cc]);
  sh[w][lane] = m;
  __syncthreads();
  if (w != 0 || c >= cols) return;
#pragma unroll
  for (int i = 1; i < kWaves; ++i) m = max(m, sh[i][lane]);
  const float a = __uint_as_float(m);
  float s, r;
  scale_from_amax(a, Fmt<F>::kMax, eps, pow2 != 0, s, r);
  if (amax_out) amax_out[c] = a;
  s_out[c] = s;
  if (r_out) r_out[c] = r;
}

// Zero codes of the weight image for the rows past `rows` in its last
// 16-row group (rows % 16 != 0): one thread per (step, half, lane) slot of
// that group, 16 bytes each.
__global__ __launch_bounds__(256) void k_image_pad_rows(uint8_t* __restrict__ q, int64_t rows, int64_t img) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (s * 2 + h) * 64 + l
  if (i >= img * 128 || (i & 15) < (rows & 15)) return;
  *reinterpret_cast<u32x4*>(q + ((rows >> 4) * img * 2) * 1024 + i * 16) = u32x4{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Host launchers.

namespace {

// Largest cast grid whose counters go straight to the output by atomics:
// 2 x 128 device-scope adds cost less than a finisher launch.
constexpr int kSmallCountGrid = 128;

// Image mode: a grid-stride grid rounded down to a multiple of 8 (the
// kernels' per-XCD order of work items needs it).
int img_grid(const QuantArgs& a, int grid) { return (a.img != 0 && grid >= 8) ? grid & ~7 : grid; }

template <typename T, int F>
hipError_t quant_tensor(const QuantArgs& a, hipStream_t st) {
  // A contiguous tensor is one long row for per-tensor work (not when the
  // codes go to the weight image, whose offsets need the true row).
  int64_t rows = a.rows, cols = a.cols;
  if (a.img == 0 && a.ldx == a.cols && a.ldq == a.cols) {
    cols = a.rows * a.cols;
    rows = 1;
  }
  const int64_t opr = cols / 8;
  constexpr int U = oct_unroll<T>();
  const int64_t seg = static_cast<int64_t>(kBlock) * U;
  const int64_t spr = ceil_div(opr, seg);
  const int64_t nseg = rows * spr;
  const int cus = device_cus();
  const bool given = a.mode == FP8RT_GIVEN;
  const bool stats = a.counts != nullptr;
  const bool am = a.amax_out != nullptr;
  const int grid = img_grid(a, static_cast<int>(std::min<int64_t>({nseg, int64_t(8) * cus, int64_t(kMaxBlocks)})));
  const int grid1 = static_cast<int>(std::min<int64_t>({nseg, int64_t(4) * cus, int64_t(kMaxBlocks)}));
  DevWorkspace* ws = nullptr;
  hipError_t e = get_workspace(st, &ws);
  if (e != hipSuccess) return e;
  const T* x = static_cast<const T*>(a.x);
  // DYNAMIC with counters on a small grid: the cast pass adds its counts
  // into the output (zeroed by the amax pass), no finisher launch
  const bool small_counts = !given && stats && !a.amax_only && grid <= kSmallCountGrid;
  if (a.amax_only) {
    hipLaunchKernelGGL(k_tensor_amax<T>, dim3(grid1), dim3(kBlock), 0, st, x, rows, opr, a.ldx, spr,
                       ws->pass1, nullptr);
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass1, grid1, a.amax_out, nullptr);
    return hipGetLastError();
  }
#define FP8RT_CAST_I(GV, ST, AM, IM)                                                                      \
  hipLaunchKernelGGL((k_tensor_cast<T, F, GV, ST, AM, IM>), dim3(grid), dim3(kBlock), 0, st, x, rows, opr, \
                     a.ldx, spr, a.q, a.ldq, a.img, ws->pass1, grid1, a.eps, a.pow2, a.scale, a.inv_scale,   \
                     a.scale, a.inv_scale, a.amax_out, ws->pass2, small_counts ? a.counts : nullptr)
#define FP8RT_CAST(GV, ST, AM)                     \
  if (a.img != 0) FP8RT_CAST_I(GV, ST, AM, true); \
  else FP8RT_CAST_I(GV, ST, AM, false)
  if (!given) {
    hipLaunchKernelGGL(k_tensor_amax<T>, dim3(grid1), dim3(kBlock), 0, st, x, rows, opr, a.ldx, spr,
                       ws->pass1, small_counts ? a.counts : nullptr);
    if (stats) FP8RT_CAST(false, true, false);
    else FP8RT_CAST(false, false, false);
  } else {
    if (stats && am) FP8RT_CAST(true, true, true);
    else if (stats) FP8RT_CAST(true, true, false);
    else if (am) FP8RT_CAST(true, false, true);
    else FP8RT_CAST(true, false, false);
  }
#undef FP8RT_CAST
#undef FP8RT_CAST_I
  if ((stats && !small_counts) || (given && am))
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass2, grid,
                       given ? a.amax_out : nullptr, a.counts);
  return hipGetLastError();
}

template <typename T, int F, int L, bool GIVEN, bool STATS, bool AO, bool IMG = false>
void launch_rowgroups_t(const QuantArgs& a, hipStream_t st, int grid, uint32_t units, FastDiv dv,
                        uint32_t nCg, DevWorkspace* ws) {
  if constexpr (!IMG && !AO) {
    if (a.img != 0) return launch_rowgroups_t<T, F, L, GIVEN, STATS, AO, true>(a, st, grid, units, dv, nCg, ws);
  }
  hipLaunchKernelGGL((k_rowgroups<T, F, L, GIVEN, STATS, AO, IMG>), dim3(grid), dim3(kBlock), 0, st,
                     static_cast<const T*>(a.x), static_cast<uint32_t>(a.rows),
                     static_cast<uint32_t>(a.cols / 8), a.ldx, dv, nCg, units, a.q, a.ldq, a.img, a.eps,
                     a.pow2, a.scale, a.inv_scale, a.amax_out, ws, a.counts);
}

template <typename T, int F, int L>
void rowgroups_dispatch(const QuantArgs& a, hipStream_t st, int grid, uint32_t units, FastDiv dv,
                        uint32_t nCg, DevWorkspace* ws) {
  const bool given = a.mode == FP8RT_GIVEN, stats = a.counts != nullptr;
  if (a.amax_only) launch_rowgroups_t<T, F, L, false, false, true>(a, st, grid, units, dv, nCg, ws);
  else if (given && stats) launch_rowgroups_t<T, F, L, true, true, false>(a, st, grid, units, dv, nCg, ws);
  else if (given) launch_rowgroups_t<T, F, L, true, false, false>(a, st, grid, units, dv, nCg, ws);
  else if (stats) launch_rowgroups_t<T, F, L, false, true, false>(a, st, grid, units, dv, nCg, ws);
  else launch_rowgroups_t<T, F, L, false, false, false>(a, st, grid, units, dv, nCg, ws);
}

template <typename T, int F>
hipError_t quant_rowgroups(const QuantArgs& a, int L, hipStream_t st) {
  constexpr int U = sizeof(T) == 2 ? 8 : 4;
  const int64_t nCg = ceil_div(a.cols, a.ec);
  const int64_t padded = a.rows * nCg * L;
  const uint32_t units = static_cast<uint32_t>(ceil_div(padded, static_cast<int64_t>(kBlock) * U));
  const int grid = img_grid(a, static_cast<int>(std::min<int64_t>({int64_t(units), int64_t(8) * device_cus(),
                                                                   int64_t(kMaxBlocks)})));
  DevWorkspace* ws = nullptr;
  hipError_t e = get_workspace(st, &ws);
  if (e != hipSuccess) return e;
  const FastDiv dv(static_cast<uint32_t>(nCg * L));
  const uint32_t ncg = static_cast<uint32_t>(nCg);
  switch (L) {
    case 2: rowgroups_dispatch<T, F, 2>(a, st, grid, units, dv, ncg, ws); break;
    case 4: rowgroups_dispatch<T, F, 4>(a, st, grid, units, dv, ncg, ws); break;
    case 8: rowgroups_dispatch<T, F, 8>(a, st, grid, units, dv, ncg, ws); break;
    case 16: rowgroups_dispatch<T, F, 16>(a, st, grid, units, dv, ncg, ws); break;
    case 32: rowgroups_dispatch<T, F, 32>(a, st, grid, units, dv, ncg, ws); break;
    case 64: rowgroups_dispatch<T, F, 64>(a, st, grid, units, dv, ncg, ws); break;
    default: return hipErrorInvalidValue;
  }
  if (a.counts && !a.amax_only)
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass2, grid, nullptr, a.counts);
  return hipGetLastError();
}

template <typename T, int F, bool GIVEN, bool STATS, bool AO, bool REG, bool IMG = false>
void launch_blocktile_t(const QuantArgs& a, hipStream_t st, int grid, int64_t nCg, int64_t ng,
                        FastDiv df, FastDiv dt, DevWorkspace* ws) {
  if constexpr (!IMG && !AO) {
    if (a.img != 0) return launch_blocktile_t<T, F, GIVEN, STATS, AO, REG, true>(a, st, grid, nCg, ng, df, dt, ws);
  }
  hipLaunchKernelGGL((k_blocktile<T, F, GIVEN, STATS, AO, REG, IMG>), dim3(grid), dim3(kBlock), 0, st,
                     static_cast<const T*>(a.x), a.rows, a.cols, a.ldx, a.er, a.ec, nCg, ng, df, dt,
                     a.q, a.ldq, a.img, a.eps, a.pow2, a.scale, a.inv_scale, a.amax_out, ws, a.counts);
}

template <typename T, int F, bool REG>
void blocktile_dispatch(const QuantArgs& a, hipStream_t st, int grid, int64_t nCg, int64_t ng,
                        FastDiv df, FastDiv dt, DevWorkspace* ws) {
  const bool given = a.mode == FP8RT_GIVEN, stats = a.counts != nullptr;
  if (a.amax_only) launch_blocktile_t<T, F, false, false, true, REG>(a, st, grid, nCg, ng, df, dt, ws);
  else if (given && stats) launch_blocktile_t<T, F, true, true, false, REG>(a, st, grid, nCg, ng, df, dt, ws);
  else if (given) launch_blocktile_t<T, F, true, false, false, REG>(a, st, grid, nCg, ng, df, dt, ws);
  else if (stats) launch_blocktile_t<T, F, false, true, false, REG>(a, st, grid, nCg, ng, df, dt, ws);
  else launch_blocktile_t<T, F, false, false, false, REG>(a, st, grid, nCg, ng, df, dt, ws);
}

template <typename T, int F>
hipError_t quant_blocktile(const QuantArgs& a, hipStream_t st) {
  constexpr int U = sizeof(T) == 2 ? 8 : 4;
  const int64_t nCg = ceil_div(a.cols, a.ec);
  const int64_t ng = ceil_div(a.rows, a.er) * nCg;
  // up to 32 workgroups per CU: one group each where possible (8 per CU left
  // each workgroup several groups in sequence: 8192 x 8192 per-row 41.1 us,
  // 37.3 at 32)
  const int grid = img_grid(a, static_cast<int>(std::min<int64_t>({ng, int64_t(32) * device_cus(), int64_t(kMaxBlocks)})));
  DevWorkspace* ws = nullptr;
  hipError_t e = get_workspace(st, &ws);
  if (e != hipSuccess) return e;
  const int64_t tail = a.cols - (nCg - 1) * a.ec;
  const FastDiv df(static_cast<uint32_t>(a.ec / 8)), dt(static_cast<uint32_t>(tail / 8));
  const bool reg = a.er * (a.ec / 8) <= static_cast<int64_t>(kBlock) * U;
  if (reg) blocktile_dispatch<T, F, true>(a, st, grid, nCg, ng, df, dt, ws);
  else blocktile_dispatch<T, F, false>(a, st, grid, nCg, ng, df, dt, ws);
  if (a.counts && !a.amax_only)
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass2, grid, nullptr, a.counts);
  return hipGetLastError();
}

// Into the weight image with per-row or per-tensor scales: k_image_rows,
// when a row's steps fit its registers (NS per wave) and the 16-row groups
// one grid of partials.
// (fp32 with counters one step less: the per-element counting would spill.)
template <typename T> constexpr int img_max_ns(bool stats) {
  return sizeof(T) == 2 ? 4 : (stats ? 1 : 2);
}

template <typename T>
bool image_rows_eligible(const QuantArgs& a) {
  if (a.img == 0 || a.amax_only || a.ec != a.cols) return false;
  return (a.er == 1 || a.er == a.rows) && a.img <= kImgWaves * img_max_ns<T>(a.counts != nullptr) &&
         ceil_div(a.rows, 16) <= kMaxBlocks;
}

template <typename T, int F, int NS, bool ROW, bool GV, bool ST, bool AM>
void launch_image_t(const QuantArgs& a, hipStream_t st, int grid, int nparts, DevWorkspace* ws) {
  hipLaunchKernelGGL((k_image_rows<T, F, NS, ROW, GV, ST, AM>), dim3(grid), dim3(kImgWaves * 64), 0, st,
                     static_cast<const T*>(a.x), a.rows, a.img, a.ldx, a.q, ws->pass1, nparts, a.eps, a.pow2,
                     a.scale, a.inv_scale, a.amax_out, ws->pass2);
}

template <typename T, int F, int NS, bool ST>
void image_dispatch_st(const QuantArgs& a, hipStream_t st, int grid, int nparts, DevWorkspace* ws, bool row) {
  const bool given = a.mode == FP8RT_GIVEN, am = a.amax_out != nullptr;
  if (row) {  // a row's observed amax is written directly
    if (given) launch_image_t<T, F, NS, true, true, ST, false>(a, st, grid, nparts, ws);
    else launch_image_t<T, F, NS, true, false, ST, false>(a, st, grid, nparts, ws);
  } else if (!given) {
    launch_image_t<T, F, NS, false, false, ST, false>(a, st, grid, nparts, ws);
  } else {
    if (am) launch_image_t<T, F, NS, false, true, ST, true>(a, st, grid, nparts, ws);
    else launch_image_t<T, F, NS, false, true, ST, false>(a, st, grid, nparts, ws);
  }
}

// false: no variant for these steps (image_rows_eligible rules it out)
template <typename T, int F, int NS>
bool image_dispatch(const QuantArgs& a, hipStream_t st, int grid, int nparts, DevWorkspace* ws, bool row) {
  if constexpr (NS > img_max_ns<T>(false)) {
    return false;
  } else {
    if (a.counts == nullptr) {
      image_dispatch_st<T, F, NS, false>(a, st, grid, nparts, ws, row);
      return true;
    }
    if constexpr (NS <= img_max_ns<T>(true)) {
      image_dispatch_st<T, F, NS, true>(a, st, grid, nparts, ws, row);
      return true;
    }
    return false;
  }
}

template <typename T, int F>
hipError_t quant_image_rows(const QuantArgs& a, hipStream_t st) {
  DevWorkspace* ws = nullptr;
  hipError_t e = get_workspace(st, &ws);
  if (e != hipSuccess) return e;
  const bool row = a.er != a.rows, given = a.mode == FP8RT_GIVEN;
  const int grid = static_cast<int>(ceil_div(a.rows, 16));
  int nparts = 0;
  if (!row && !given) {
    // the tensor's amax pass (as the row-major per-tensor path runs it)
    int64_t rows = a.rows, cols = a.cols;
    if (a.ldx == a.cols) {
      cols = a.rows * a.cols;
      rows = 1;
    }
    const int64_t opr = cols / 8;
    const int64_t spr = ceil_div(opr, static_cast<int64_t>(kBlock) * oct_unroll<T>());
    nparts = static_cast<int>(std::min<int64_t>({rows * spr, int64_t(4) * device_cus(), int64_t(kMaxBlocks)}));
    hipLaunchKernelGGL(k_tensor_amax<T>, dim3(nparts), dim3(kBlock), 0, st, static_cast<const T*>(a.x), rows, opr,
                       a.ldx, spr, ws->pass1, nullptr);
  }
  bool ok = false;
  switch (ceil_div(a.img, int64_t(kImgWaves))) {
    case 1: ok = image_dispatch<T, F, 1>(a, st, grid, nparts, ws, row); break;
    case 2: ok = image_dispatch<T, F, 2>(a, st, grid, nparts, ws, row); break;
    case 3: ok = image_dispatch<T, F, 3>(a, st, grid, nparts, ws, row); break;
    case 4: ok = image_dispatch<T, F, 4>(a, st, grid, nparts, ws, row); break;
    default: break;
  }
  if (!ok) return hipErrorInvalidValue;
  if (a.counts || (given && !row && a.amax_out))
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass2, grid,
                       (given && !row) ? a.amax_out : nullptr, a.counts);
  return hipGetLastError();
}

template <typename T, int F>
hipError_t quant_typed(const QuantArgs& a, hipStream_t st) {
  if (image_rows_eligible<T>(a)) return quant_image_rows<T, F>(a, st);
  if (a.img != 0 && a.rows % 16 != 0) {
    // the image's rows past the last one of a short last 16-row group
    const int64_t n = a.img * 128;
    hipLaunchKernelGGL(k_image_pad_rows, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, st, a.q,
                       a.rows, a.img);
  }
  if (a.er == a.rows && a.ec == a.cols) return quant_tensor<T, F>(a, st);
  if (a.er == 1) {
    const int64_t L = a.ec / 8;
    // L is a power of two in [2, 64] and the padded octet space fits 31 bits
    const bool pow2L = L >= 2 && L <= 64 && (L & (L - 1)) == 0;
    if (pow2L && a.rows * ceil_div(a.cols, a.ec) * L < (int64_t(1) << 31) - 4096)
      return quant_rowgroups<T, F>(a, static_cast<int>(L), st);
  }
  return quant_blocktile<T, F>(a, st);
}


// ---------------------------------------------------------------------------
// Cast-transpose launcher.

template <typename T, int F, int GK, bool STATS, bool AM>
void launch_ct_t(const QuantArgs& a, const float* r, uint8_t* qt, int64_t ldqt, int grid, int tiles_c,
                 int ntiles, DevWorkspace* ws, hipStream_t st) {
  hipLaunchKernelGGL((k_cast_transpose<T, F, GK, STATS, AM>), dim3(grid), dim3(kBlock), 0, st,
                     static_cast<const T*>(a.x), a.rows, a.cols, a.ldx, a.scale, r, a.q, a.ldq, qt, ldqt,
                     tiles_c, ntiles, ws->pass2);
}

template <typename T, int F>
hipError_t quant_transpose_typed(const QuantArgs& a, uint8_t* qt, int64_t ldqt, hipStream_t st) {
  const int gk = (a.er == a.rows && a.ec == a.cols) ? 0 : (a.er == 1 && a.ec == a.cols) ? 1 : 2;
  const int64_t G = gk == 0 ? 1 : gk == 1 ? a.rows : a.cols;
  const bool dynamic = a.mode == FP8RT_DYNAMIC;
  const bool need_amax = dynamic || (a.amax_out && gk != 0);
  DevWorkspace* ws = nullptr;
  hipError_t e = get_workspace(st, &ws);
  if (e != hipSuccess) return e;
  // scratch: amax [G] (when amax_out is null), r [G] (when inv_scale is null),
  // column partials [nchunk][cols]
  const int64_t colblocks = ceil_div(a.cols, 128);
  const int64_t nchunk =
      gk == 2 ? std::max<int64_t>(1, std::min<int64_t>(ceil_div(a.rows, 64), ceil_div(8 * device_cus(), colblocks)))
              : 0;
  const int64_t rpc = gk == 2 ? ceil_div(a.rows, nchunk) : 0;
  void* scr = nullptr;
  e = get_scratch(st, static_cast<size_t>(2 * G + nchunk * a.cols) * 4 + 256, &scr);
  if (e != hipSuccess) return e;
  float* amax = a.amax_out ? a.amax_out : static_cast<float*>(scr);
  float* rbuf = static_cast<float*>(scr) + G;
  uint32_t* cpart = reinterpret_cast<uint32_t*>(static_cast<float*>(scr) + 2 * G);
  const float* r = a.inv_scale;
  bool scaled = false;  // s and r already derived (per-column DYNAMIC)
  if (need_amax) {
    if (gk == 2) {
      hipLaunchKernelGGL(k_col_amax<T>, dim3(static_cast<unsigned>(colblocks), static_cast<unsigned>(nchunk)),
                         dim3(kBlock), 0, st, static_cast<const T*>(a.x), a.rows, a.cols, a.ldx, rpc, cpart);
      if (dynamic) {  // the column amax, s and r in one launch
        float* rw = a.inv_scale ? a.inv_scale : rbuf;
        hipLaunchKernelGGL(k_col_amax_scale<F>, dim3(static_cast<unsigned>(ceil_div(a.cols, 64))), dim3(kBlock),
                           0, st, cpart, nchunk, a.cols, a.eps, a.pow2, a.amax_out, a.scale, rw);
        r = rw;
        scaled = true;
      } else {
        hipLaunchKernelGGL(k_col_amax_finish, dim3(static_cast<unsigned>(ceil_div(a.cols, kBlock))),
                           dim3(kBlock), 0, st, cpart, nchunk, a.cols, amax);
      }
    } else {
      QuantArgs b = a;
      b.amax_only = true;
      b.amax_out = amax;
      b.counts = nullptr;
      e = launch_quantize(b, st);
      if (e != hipSuccess) return e;
    }
  }
  if (dynamic && !scaled) {
    float* rw = a.inv_scale ? a.inv_scale : rbuf;
    e = launch_compute_scale(amax, G, a.fmt, a.eps, a.pow2 != 0, a.scale, rw, st);
    if (e != hipSuccess) return e;
    r = rw;
  }
  const bool stats = a.counts != nullptr;
  const bool am = gk == 0 && !dynamic && a.amax_out != nullptr;  // observed per-tensor amax
  const int tiles_c = static_cast<int>(ceil_div(a.cols, kCtC));
  const int64_t nt = ceil_div(a.rows, kCtR) * tiles_c;
  if (nt > (int64_t(1) << 30)) return hipErrorInvalidValue;
  const int ntiles = static_cast<int>(nt);
  const int grid = static_cast<int>(std::min<int64_t>(nt, int64_t(kMaxBlocks)));
#define FP8RT_CT(GK)                                                                                         \
  if (stats && am) launch_ct_t<T, F, GK, true, true>(a, r, qt, ldqt, grid, tiles_c, ntiles, ws, st);       \
  else if (stats) launch_ct_t<T, F, GK, true, false>(a, r, qt, ldqt, grid, tiles_c, ntiles, ws, st);       \
  else if (am) launch_ct_t<T, F, GK, false, true>(a, r, qt, ldqt, grid, tiles_c, ntiles, ws, st);          \
  else launch_ct_t<T, F, GK, false, false>(a, r, qt, ldqt, grid, tiles_c, ntiles, ws, st);
  if (gk == 0) { FP8RT_CT(0) }
  else if (gk == 1) { FP8RT_CT(1) }
  else { FP8RT_CT(2) }
#undef FP8RT_CT
  if (stats || am)
    hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, ws->pass2, grid, am ? a.amax_out : nullptr,
                       a.counts);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_quantize(const QuantArgs& a, hipStream_t st) {
  if (a.xt == FP8RT_BF16) {
    return a.fmt == FP8RT_E4M3 ? quant_typed<uint16_t, kE4M3>(a, st)
                               : quant_typed<uint16_t, kE5M2>(a, st);
  }
  return a.fmt == FP8RT_E4M3 ? quant_typed<float, kE4M3>(a, st) : quant_typed<float, kE5M2>(a, st);
}

hipError_t launch_finish(const BlockPartial* part, int n, float* amax_out, unsigned long long* counts,
                         hipStream_t st) {
  hipLaunchKernelGGL(k_finish, dim3(1), dim3(kFinThreads), 0, st, part, n, amax_out, counts);
  return hipGetLastError();
}

hipError_t launch_quantize_transpose(const QuantArgs& a, uint8_t* qt, int64_t ldqt, hipStream_t st) {
  if (a.xt == FP8RT_BF16) {
    return a.fmt == FP8RT_E4M3 ? quant_transpose_typed<uint16_t, kE4M3>(a, qt, ldqt, st)
                               : quant_transpose_typed<uint16_t, kE5M2>(a, qt, ldqt, st);
  }
  return a.fmt == FP8RT_E4M3 ? quant_transpose_typed<float, kE4M3>(a, qt, ldqt, st)
                             : quant_transpose_typed<float, kE5M2>(a, qt, ldqt, st);
}

// ---------------------------------------------------------------------------
// Scale from amax, elementwise.

template <int F>
__global__ __launch_bounds__(kBlock) void k_compute_scale(const float* __restrict__ amax, int64_t n,
                                                          float eps, int pow2, float* s_out,
                                                          float* r_out) {
  for (int64_t i = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kBlock) {
    float s, r;
    scale_from_amax(amax[i], Fmt<F>::kMax, eps, pow2 != 0, s, r);
    s_out[i] = s;
    if (r_out) r_out[i] = r;
  }
}

hipError_t launch_compute_scale(const float* amax, int64_t n, int fmt, float eps, int pow2,
                                float* scale, float* inv_scale, hipStream_t st) {
  const int grid = static_cast<int>(std::min<int64_t>(ceil_div(n, kBlock), 4 * device_cus()));
  if (fmt == FP8RT_E4M3)
    hipLaunchKernelGGL(k_compute_scale<kE4M3>, dim3(grid), dim3(kBlock), 0, st, amax, n, eps, pow2,
                       scale, inv_scale);
  else
    hipLaunchKernelGGL(k_compute_scale<kE5M2>, dim3(grid), dim3(kBlock), 0, st, amax, n, eps, pow2,
                       scale, inv_scale);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Dequantize: y = fl32(s_g * dec(code)); bf16 output rounds that binary32 to
// nearest even (NaN -> 0x7FC0).  The hardware decode of one code is exact.

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & kAbsMask) > kInfBits) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int F, bool BF16OUT>
__global__ __launch_bounds__(kBlock) void k_dequantize(const uint8_t* __restrict__ q, int64_t rows,
                                                       int64_t cols, int64_t ldq, int64_t er,
                                                       FastDiv div_ec, int64_t nCg,
                                                       const float* __restrict__ scale, void* y,
                                                       int64_t ldy) {
  const int64_t opr = cols / 8;
  const int64_t total = rows * opr;
  for (int64_t o = blockIdx.x * static_cast<int64_t>(kBlock) + threadIdx.x; o < total;
       o += static_cast<int64_t>(gridDim.x) * kBlock) {
    const int64_t r = o / opr;
    const int64_t c = (o - r * opr) * 8;
    const u32x2 w = *reinterpret_cast<const u32x2*>(q + r * ldq + c);
    const float s = scale[(r / er) * nCg + div_ec.div(static_cast<uint32_t>(c))];
    float d[8];
    decode4<F>(w[0], d);
    decode4<F>(w[1], d + 4);
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = s * d[i];
    if constexpr (BF16OUT) {
      u32x4 o4;
      o4[0] = f32_to_bf16_bits(d[0]) | (f32_to_bf16_bits(d[1]) << 16);
      o4[1] = f32_to_bf16_bits(d[2]) | (f32_to_bf16_bits(d[3]) << 16);
      o4[2] = f32_to_bf16_bits(d[4]) | (f32_to_bf16_bits(d[5]) << 16);
      o4[3] = f32_to_bf16_bits(d[6]) | (f32_to_bf16_bits(d[7]) << 16);
      *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + r * ldy + c) = o4;
    } else {
      u32x4* yp = reinterpret_cast<u32x4*>(static_cast<float*>(y) + r * ldy + c);
      yp[0] = u32x4{__float_as_uint(d[0]), __float_as_uint(d[1]), __float_as_uint(d[2]), __float_as_uint(d[3])};
      yp[1] = u32x4{__float_as_uint(d[4]), __float_as_uint(d[5]), __float_as_uint(d[6]), __float_as_uint(d[7])};
    }
  }
}

hipError_t launch_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                             int64_t er, int64_t ec, const float* scale, void* y, int yt,
                             int64_t ldy, hipStream_t st) {
  const int64_t total = rows * (cols / 8);
  const int grid = static_cast<int>(std::min<int64_t>(ceil_div(total, kBlock), 8 * device_cus()));
  const FastDiv dv(static_cast<uint32_t>(ec));
  const int64_t nCg = ceil_div(cols, ec);
  if (fmt == FP8RT_E4M3) {
    if (yt == FP8RT_BF16)
      hipLaunchKernelGGL((k_dequantize<kE4M3, true>), dim3(grid), dim3(kBlock), 0, st, q, rows, cols,
                         ldq, er, dv, nCg, scale, y, ldy);
    else
      hipLaunchKernelGGL((k_dequantize<kE4M3, false>), dim3(grid), dim3(kBlock), 0, st, q, rows,
                         cols, ldq, er, dv, nCg, scale, y, ldy);
  } else {
    if (yt == FP8RT_BF16)
      hipLaunchKernelGGL((k_dequantize<kE5M2, true>), dim3(grid), dim3(kBlock), 0, st, q, rows, cols,
                         ldq, er, dv, nCg, scale, y, ldy);
    else
      hipLaunchKernelGGL((k_dequantize<kE5M2, false>), dim3(grid), dim3(kBlock), 0, st, q, rows,
                         cols, ldq, er, dv, nCg, scale, y, ldy);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Delayed scaling: one wave pushes a_t into the ring, takes the window
// maximum (integer max of the binary32 patterns of non-negative entries, NaN
// kept), and derives the next step's (s, r) on the device.

// Recipe variants (same section: the history function may be the latest
// value or the window maximum; recipes add a margin): fn 1 takes a_t alone
// (the ring still advances), and the scale is derived from f * 2^margin
// (v_ldexp_f32: exact, or Inf -> NaN scale on overflow).
template <int F>
__global__ __launch_bounds__(64) void k_history_update(float* history, int32_t len, int32_t* head,
                                                       const float* amax_new, float eps, int pow2, int fn,
                                                       int margin, float* s_next, float* r_next) {
  const int lane = threadIdx.x;
  int32_t h = head[0];
  h = ((h % len) + len) % len;
  const float an = amax_new[0];
  // ordering key: NaN above everything, non-positive values as zero
  auto key_of = [](float v) {
    const uint32_t b = __float_as_uint(v);
    return ((b & kAbsMask) > kInfBits) ? kQNaN : (v > 0.0f ? b : 0u);
  };
  uint32_t m = 0;
  if (fn == 0) {
    for (int i = lane; i < len; i += 64) m = max(m, key_of((i == h) ? an : history[i]));
    m = wave_max_u32(m);
  } else {
    m = key_of(an);
  }
  if (lane == 0) {
    history[h] = an;
    head[0] = (h + 1) % len;
    float s, r;
    scale_from_amax(ldexpf(__uint_as_float(m), margin), Fmt<F>::kMax, eps, pow2 != 0, s, r);
    s_next[0] = s;
    if (r_next) r_next[0] = r;
  }
}

hipError_t launch_history_update(float* history, int32_t len, int32_t* head, const float* amax_new,
                                 int fmt, float eps, int pow2, int fn, int margin, float* scale_next,
                                 float* inv_scale_next, hipStream_t st) {
  if (fmt == FP8RT_E4M3)
    hipLaunchKernelGGL(k_history_update<kE4M3>, dim3(1), dim3(64), 0, st, history, len, head,
                       amax_new, eps, pow2, fn, margin, scale_next, inv_scale_next);
  else
    hipLaunchKernelGGL(k_history_update<kE5M2>, dim3(1), dim3(64), 0, st, history, len, head,
                       amax_new, eps, pow2, fn, margin, scale_next, inv_scale_next);
  return hipGetLastError();
}

}  // namespace fp8rt
