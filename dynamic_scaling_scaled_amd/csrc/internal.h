// internal.h -- declarations shared by the library's translation units (host
// side).  Not installed; the public interface is include/fp8rt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8rt.h"

namespace fp8rt {

// Per-block partial results of the quantize kernels (reduced by a finisher
// kernel into amax_out and the saturation / underflow counters).
struct BlockPartial {
  uint32_t amax_bits;
  uint32_t pad;
  unsigned long long sat;
  unsigned long long under;
};

// Stream-ordered scratch memory for one call (hipMallocAsync / hipFreeAsync
// on the caller's stream, so concurrent calls never share it).
class CallScratch {
 public:
  explicit CallScratch(hipStream_t s) : stream_(s) {}
  ~CallScratch() {
    if (ptr_) (void)hipFreeAsync(ptr_, stream_);
  }
  CallScratch(const CallScratch&) = delete;
  CallScratch& operator=(const CallScratch&) = delete;
  hipError_t alloc(size_t bytes) {
    if (bytes == 0) bytes = 256;
    return hipMallocAsync(&ptr_, bytes, stream_);
  }
  void* get() const { return ptr_; }

 private:
  void* ptr_ = nullptr;
  hipStream_t stream_;
};

// Effective group extent of a granularity: 0 or >= n means the whole dimension.
inline int64_t group_extent(int64_t n, int32_t g) { return (g <= 0 || g >= n) ? n : g; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct QuantArgs {
  const void* x;
  int xt;  // fp8rt_dtype
  int64_t rows, cols, ldx;
  int64_t er, ec;  // effective group extents
  int fmt;
  int mode;  // fp8rt_mode
  float eps;
  int pow2;
  float* scale;
  float* inv_scale;
  uint8_t* q;
  int64_t ldq;
  float* amax_out;
  unsigned long long* counts;
  bool amax_only;  // fp8_amax: write amax_out only
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
hipError_t launch_compute_scale(const float* amax, int64_t n, int fmt, float eps, int pow2,
                                float* scale, float* inv_scale, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                             int64_t er, int64_t ec, const float* scale, void* y, int yt,
                             int64_t ldy, hipStream_t stream);
hipError_t launch_history_update(float* history, int32_t len, int32_t* head, const float* amax_new,
                                 int fmt, float eps, int pow2, float* scale_next,
                                 float* inv_scale_next, hipStream_t stream);

struct GemmArgs {
  const uint8_t* a;
  int fa;
  int64_t lda;
  int64_t era, eca;  // effective scale-group extents of A (rows, K)
  const float* sa;
  const uint8_t* b;
  int fb;
  int64_t ldb;
  int64_t erb, ecb;
  const float* sb;
  int64_t M, N, K;
  const void* bias;
  int bias_t;
  void* y;
  int yt;
  int64_t ldy;
  bool pow2_mx;  // 1x32 power-of-two scales through the scaled MFMA
};

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);

}  // namespace fp8rt
