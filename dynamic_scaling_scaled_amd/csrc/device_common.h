// device_common.h -- gfx950 device helpers shared by the library's kernels:
// format constants, 16-byte loads of bf16 / fp32 octets, the packed
// FP32 -> FP8 convert, the scale rule and small reductions.
//
// Scale rule ("FP8 formats and scaling for LLM inference", section "How a
// scale fits a tensor into E4M3"; "FP8 production quantization guide",
// dynamic quantize listing): a_c = max(amax, eps), s = a_c / F_max (the
// dequantization scale), r = F_max / a_c (the quantization multiplier), each a
// correctly rounded binary32 quotient; optional power-of-two rounding of s
// (same section's list of recipe options).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8rt {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

constexpr int kE4M3 = 0;
constexpr int kE5M2 = 1;

// Largest finite magnitude ("How the 8 bits are allocated": 448 and 57344).
template <int F> struct Fmt;
template <> struct Fmt<kE4M3> {
  static constexpr float kMax = 448.0f;
  // |v| <= kZeroEdge rounds to a zero code (half the smallest subnormal 2^-9,
  // ties to even go to zero).
  static constexpr float kZeroEdge = 0x1p-10f;
};
template <> struct Fmt<kE5M2> {
  static constexpr float kMax = 57344.0f;
  static constexpr float kZeroEdge = 0x1p-17f;  // half of 2^-16
};

__host__ __device__ inline float fmax_of(int f) { return f == kE4M3 ? 448.0f : 57344.0f; }

constexpr uint32_t kQNaN = 0x7FC00000u;
constexpr uint32_t kAbsMask = 0x7FFFFFFFu;
constexpr uint32_t kInfBits = 0x7F800000u;

// Scale and inverse scale from one amax.  A non-finite amax (NaN or Inf)
// gives NaN s and r.  eps is validated on the host (finite, >= 2^-96), so
// every quotient below is a normal binary32 and '/' is correctly rounded
// (hipcc's default fp32 division).
__device__ __forceinline__ void scale_from_amax(float a, float F, float eps, bool pow2, float& s,
                                                float& r) {
  const uint32_t ab = __float_as_uint(a) & kAbsMask;
  if (ab >= kInfBits) {
    s = __uint_as_float(kQNaN);
    r = __uint_as_float(kQNaN);
    return;
  }
  const float ac = a < eps ? eps : a;
  s = ac / F;
  r = F / ac;
  if (pow2) {
    uint32_t b = __float_as_uint(s);
    if (b & 0x007FFFFFu) b = (b & 0x7F800000u) + 0x00800000u;  // round up to 2^ceil(log2 s)
    s = __uint_as_float(b);
    r = 1.0f / s;  // exact for a power of two
  }
}

// ---------------------------------------------------------------------------
// Octets: 8 consecutive elements of a row (16 bytes of bf16, 32 of fp32).

template <typename T> struct Octet;

template <> struct Octet<uint16_t> {  // bf16 carried as raw bits
  u32x4 raw;
  // Streaming load (last use of the data).
  __device__ __forceinline__ void load_nt(const uint16_t* p) {
    raw = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  }
  // Cached load (the data is read again soon).
  __device__ __forceinline__ void load(const uint16_t* p) { raw = *reinterpret_cast<const u32x4*>(p); }
  __device__ __forceinline__ void zero() { raw = u32x4{0u, 0u, 0u, 0u}; }
  // Zero the octet unless valid (a select, not a branch: guarded loads are
  // issued unconditionally from a clamped address so they all stay in flight).
  __device__ __forceinline__ void keep_if(bool valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) raw[j] = valid ? raw[j] : 0u;
  }
  // Exact widening: a bf16 is the top half of a binary32.
  __device__ __forceinline__ float get(int i) const {
    const uint32_t w = raw[i >> 1];
    return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
  }
  // max over the 8 elements of the |x| bit pattern (as binary32 bits); NaN
  // patterns exceed Inf, so NaN propagates.
  __device__ __forceinline__ uint32_t absmax_bits() const {
    // 16-bit lane-wise max of the |bf16| patterns (v_pk_max_u16), then the
    // larger half widened to binary32 bits.  Computed on the raw words so it
    // shares no value with the widening of get().
    u16x2 m = u16x2{0, 0};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, raw[j] & 0x7FFF7FFFu));
    return static_cast<uint32_t>(max(m[0], m[1])) << 16;
  }
};

template <> struct Octet<float> {
  u32x4 raw0, raw1;
  __device__ __forceinline__ void load_nt(const float* p) {
    raw0 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    raw1 = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p) + 1);
  }
  __device__ __forceinline__ void load(const float* p) {
    raw0 = *reinterpret_cast<const u32x4*>(p);
    raw1 = *(reinterpret_cast<const u32x4*>(p) + 1);
  }
  __device__ __forceinline__ void zero() {
    raw0 = u32x4{0u, 0u, 0u, 0u};
    raw1 = raw0;
  }
  __device__ __forceinline__ void keep_if(bool valid) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      raw0[j] = valid ? raw0[j] : 0u;
      raw1[j] = valid ? raw1[j] : 0u;
    }
  }
  __device__ __forceinline__ float get(int i) const {
    return __uint_as_float(i < 4 ? raw0[i] : raw1[i - 4]);
  }
  __device__ __forceinline__ uint32_t absmax_bits() const {
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(raw0[j] & kAbsMask, raw1[j] & kAbsMask));
    return m;
  }
};

// ---------------------------------------------------------------------------
// FP32 -> FP8 for 4 values, byte i of the result = code of value i.
// The clamp to +-F_max comes first, so the convert never sees an overflow;
// v_cvt_pk_fp8_f32 / v_cvt_pk_bf8_f32 round to nearest even onto the OCP
// grid (subnormals included), which the parity tests check exhaustively at
// every tie.  NaN needs the separate path below (the clamp does not keep it).
template <int F>
__device__ __forceinline__ uint32_t cvt4(float a, float b, float c, float d) {
  constexpr float M = Fmt<F>::kMax;
  a = __builtin_amdgcn_fmed3f(a, -M, M);
  b = __builtin_amdgcn_fmed3f(b, -M, M);
  c = __builtin_amdgcn_fmed3f(c, -M, M);
  d = __builtin_amdgcn_fmed3f(d, -M, M);
  int w;
  if constexpr (F == kE4M3) {
    w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  } else {
    w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
  }
  return static_cast<uint32_t>(w);
}

// Same, with NaN inputs mapped to the code 0x7F.
template <int F>
__device__ __forceinline__ uint32_t cvt4_nan(float a, float b, float c, float d) {
  const uint32_t w = cvt4<F>(a, b, c, d);
  const uint32_t m = (__builtin_isnan(a) ? 0x000000FFu : 0u) | (__builtin_isnan(b) ? 0x0000FF00u : 0u) |
                     (__builtin_isnan(c) ? 0x00FF0000u : 0u) | (__builtin_isnan(d) ? 0xFF000000u : 0u);
  return (w & ~m) | (0x7F7F7F7Fu & m);
}

// Exact decode of 4 FP8 codes (one dword, byte i = element i) to binary32.
template <int F>
__device__ __forceinline__ void decode4(uint32_t w, float* out) {
  if constexpr (F == kE4M3) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
  } else {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_bf8(static_cast<int>(w), true);
    out[0] = lo[0]; out[1] = lo[1]; out[2] = hi[0]; out[3] = hi[1];
  }
}

// ---------------------------------------------------------------------------
// Reductions (wave64).

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o)));
  return v;
}

// Max over aligned segments of L lanes (L a power of two <= 64); every lane of
// the segment receives the result.
template <int L>
__device__ __forceinline__ uint32_t segment_max_u32(uint32_t v) {
#pragma unroll
  for (int o = L / 2; o >= 1; o >>= 1)
    v = max(v, static_cast<uint32_t>(__shfl_xor(static_cast<int>(v), o)));
  return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    const uint32_t lo = static_cast<uint32_t>(v), hi = static_cast<uint32_t>(v >> 32);
    const uint32_t olo = static_cast<uint32_t>(__shfl_xor(static_cast<int>(lo), o));
    const uint32_t ohi = static_cast<uint32_t>(__shfl_xor(static_cast<int>(hi), o));
    v += (static_cast<unsigned long long>(ohi) << 32) | olo;
  }
  return v;
}

// Block-wide max of m and sums of s and u over NW waves; thread 0 writes
// {m, s, u, 0} to dst (16 bytes).  Called by every thread of the block.
template <int NW>
__device__ __forceinline__ void block_stats_store(u32x4* dst, uint32_t m, uint32_t s, uint32_t u) {
  __shared__ uint32_t sh_st[3][NW];
  m = wave_max_u32(m);
  s = static_cast<uint32_t>(wave_sum_u64(s));
  u = static_cast<uint32_t>(wave_sum_u64(u));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) {
    sh_st[0][w] = m;
    sh_st[1][w] = s;
    sh_st[2][w] = u;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t tm = 0, ts = 0, tu = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      tm = max(tm, sh_st[0][i]);
      ts += sh_st[1][i];
      tu += sh_st[2][i];
    }
    *dst = u32x4{tm, ts, tu, 0u};
  }
}

// ---------------------------------------------------------------------------
// Division of a 32-bit unsigned by a run-time invariant divisor d >= 1:
// q = (mulhi(n, m) + n) >> l with l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
  uint32_t d, m, l;
  __host__ FastDiv() : d(1), m(0), l(0) {}
  __host__ explicit FastDiv(uint32_t div) : d(div) {
    l = 0;
    while ((1ull << l) < div) ++l;
    m = static_cast<uint32_t>(((1ull << 32) * ((1ull << l) - div)) / div + 1);
  }
  __device__ __forceinline__ uint32_t div(uint32_t n) const {
    return static_cast<uint32_t>((static_cast<uint64_t>(__umulhi(n, m)) + n) >> l);
  }
};

}  // namespace fp8rt
