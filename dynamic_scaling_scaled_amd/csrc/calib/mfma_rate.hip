// mfma_rate.hip -- a measurement aid beside the library, not part of the FP8
// chain: the sustained rate of the gfx950 FP8 matrix-core instructions with
// their operands held in registers, so that no memory traffic, LDS read or
// barrier sits in the loop.  It gives the ceiling the GEMM kernels are
// measured against on this chip: the instruction rate at the clock the chip
// holds for the operands' switching activity (zero bytes against random ones).
//
// Each wave keeps 16 independent accumulators (4 x 4 tiles: 256 FP32
// registers of 32x32x64, or 64 of 16x16x128; far more independent chains than
// either instruction's latency needs) and issues 16 MFMAs per iteration on 4 A
// and 4 B operand registers loaded once.  The sum
// of the accumulators is written per thread so the work cannot be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves, one per SIMD
constexpr int kOpInts = 8 * 8 * 64;  // 8 operand registers of 8 dwords for 64 lanes

template <int SHAPE>
__global__ __launch_bounds__(kThreads) void k_mfma_rate(const int* __restrict__ ops, int iters,
                                                        float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  i32x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      a[i][j] = ops[(i * 8 + j) * 64 + lane];
      b[i][j] = ops[((i + 4) * 8 + j) * 64 + lane];
    }
  float s = 0.f;
  if constexpr (SHAPE == 32) {
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 16; ++k) s += acc[i][j][k];
  } else {
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(b[j], a[i], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k) s += acc[i][j][k];
  }
  out[static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// Number of int32 operand words the kernel reads (the caller fills them with
// zeros or random FP8 bytes).
int fp8rt_calib_mfma_operand_ints(void) { return kOpInts; }

// Runs `blocks` workgroups of 256 threads, each wave issuing 16 * iters FP8
// MFMAs of the given shape (32: 32x32x64, 16: 16x16x128) on E4M3 operands.
// ops: device, kOpInts int32; out: device, blocks * 256 floats.  Returns the
// hipError_t of the launch (0 on success); an unknown shape or a
// non-positive count returns hipErrorInvalidValue without launching.
int fp8rt_calib_mfma_rate(int shape, const int* ops, int blocks, int iters, float* out, hipStream_t st) {
  if (!ops || !out || blocks <= 0 || iters <= 0 || (shape != 32 && shape != 16)) return hipErrorInvalidValue;
  if (shape == 32)
    hipLaunchKernelGGL(k_mfma_rate<32>, dim3(blocks), dim3(kThreads), 0, st, ops, iters, out);
  else
    hipLaunchKernelGGL(k_mfma_rate<16>, dim3(blocks), dim3(kThreads), 0, st, ops, iters, out);
  return hipGetLastError();
}

}  // extern "C"
