// internal.h -- declarations shared by the library's translation units (host
// side).  Not installed; the public interface is include/fp8rt.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fp8rt.h"

namespace fp8rt {

// Per-block partial results of the quantize kernels, combined by the next
// kernel on the stream (plain stores and loads: the kernel boundary orders
// them; no device-scope fences or same-address atomics, which are slow on a
// GPU whose L2 caches are per XCD).
// 16 bytes, moved as one vector; a block handles fewer than 2^32 elements, so
// its counts fit 32 bits (the finisher sums them in 64).
struct BlockPartial {
  uint32_t amax_bits;
  uint32_t sat;
  uint32_t under;
  uint32_t pad;
};

constexpr int kMaxBlocks = 8192;  // upper bound of every quantize grid

// Device workspace of one (device, stream) pair.  Calls on one stream are
// ordered, so they never share it concurrently.
struct DevWorkspace {
  BlockPartial pass1[kMaxBlocks];  // per-tensor amax partials of the first pass
  BlockPartial pass2[kMaxBlocks];  // per-block counters / observed amax of a cast pass
};

// Returns the workspace of (current device, stream), allocating it on first
// use (hipMalloc; nothing in it is zeroed: every partial is written before it
// is read).
hipError_t get_workspace(hipStream_t stream, DevWorkspace** ws);

// Returns a scratch buffer of at least `bytes` for (current device, stream).
// It grows on demand: a larger buffer replaces it and the old one is kept,
// never freed, so an address a captured graph holds stays valid; buffers live
// for the life of the process and their contents do not persist between
// calls.
hipError_t get_scratch(hipStream_t stream, size_t bytes, void** ptr);

// Compute units of the current device (256 on MI355X).
int device_cus();

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
  int64_t img;  // 0: q row-major (ldq); else q is the weight image of cols = 128 img
  float* amax_out;
  unsigned long long* counts;
  bool amax_only;  // fp8_amax: write amax_out only
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t stream);
// Cast-transpose: the quantize of a (tensor, row or column groups), codes also
// written transposed to qt [cols x rows] (ldqt).
hipError_t launch_quantize_transpose(const QuantArgs& a, uint8_t* qt, int64_t ldqt, hipStream_t stream);
hipError_t launch_compute_scale(const float* amax, int64_t n, int fmt, float eps, int pow2,
                                float* scale, float* inv_scale, hipStream_t stream);
hipError_t launch_dequantize(const uint8_t* q, int fmt, int64_t rows, int64_t cols, int64_t ldq,
                             int64_t er, int64_t ec, const float* scale, void* y, int yt,
                             int64_t ldy, hipStream_t stream);
// fn: 0 = window maximum, 1 = latest amax; margin: scale from f * 2^margin.
hipError_t launch_history_update(float* history, int32_t len, int32_t* head, const float* amax_new,
                                 int fmt, float eps, int pow2, int fn, int margin, float* scale_next,
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
  bool b_packed = false;  // b is fragment-ordered (launch_pack_weights16)
  bool exact_products = false;  // decode kernel: codes widened to bf16, bf16 MFMA
  // FP8 output (fp8_scaled_gemm_fp8out) when yq_fmt >= 0: y then holds codes
  // of y_fp32 * r_y, r_y = ry[0] or fl32(1 / sy[0]); per-block partials of
  // max |y| and the saturation / underflow counts go to part.
  int yq_fmt = -1;
  const float* sy = nullptr;
  const float* ry = nullptr;
  float* amax_y = nullptr;
  unsigned long long* counts_y = nullptr;
  BlockPartial* part = nullptr;
  // When set, the GEMM's scratch comes from this fixed buffer instead of the
  // stream's growable one (the allocation-free entry point): scale repacks
  // must fit (gemm_required_scratch), a split last wave takes fewer K parts,
  // or none, to fit.
  void* fixed_scratch = nullptr;
  size_t fixed_scratch_bytes = 0;
};

// Scratch for a GEMM call: the fixed buffer when g has one (an error if it is
// smaller than `bytes`), else the stream's buffer (get_scratch).
hipError_t gemm_scratch(const GemmArgs& g, hipStream_t stream, size_t bytes, void** ptr);
// Bytes of scratch the kernel that launch_gemm picks for g cannot do without
// (the repacked 1x32 exponents, the transposed 1x128 A scales); the FP32
// parts of a split last wave are optional and not counted.
size_t gemm_required_scratch(const GemmArgs& g);
size_t gemm_big_required_scratch(const GemmArgs& g);
size_t gemm_kblock_required_scratch(const GemmArgs& g);

// The allocation-free GEMM's scratch: a fixed device array of the library
// (noalloc.hip) of kNoAllocScratchBytes; its address on the current device.
constexpr size_t kNoAllocScratchBytes = FP8RT_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// Output kinds of the GEMM kernels' epilogues.
constexpr int kOutF32 = 0, kOutBF16 = 1, kOutE4M3 = 2, kOutE5M2 = 3;
inline int gemm_out_kind(const GemmArgs& g) {
  if (g.yq_fmt >= 0) return g.yq_fmt == FP8RT_E4M3 ? kOutE4M3 : kOutE5M2;
  return g.yt == FP8RT_BF16 ? kOutBF16 : kOutF32;
}

// Combines n per-block partials into amax_out[0] / counts[0..1] (nullable).
hipError_t launch_finish(const BlockPartial* part, int n, float* amax_out, unsigned long long* counts,
                         hipStream_t stream);

hipError_t launch_gemm(const GemmArgs& g, hipStream_t stream);
bool gemm_big_eligible(const GemmArgs& g);
// nparts (nullable) receives the number of FP8-output statistics partials
// written to g.part.
hipError_t launch_gemm_big(const GemmArgs& g, hipStream_t stream, int* nparts = nullptr);
bool gemm_kblock_eligible(const GemmArgs& g);
hipError_t launch_gemm_kblock(const GemmArgs& g, hipStream_t stream);
// Adds the FP32 K-parts of the split 256 x 256 tiles t_main, t_main + 1, ...
// (part[k split + p], tile order of the large kernels), then applies
// s_a(row) s_b(col) (a null table: already applied), the bias and g's output
// type.
hipError_t launch_split_reduce(const GemmArgs& g, hipStream_t st, const float* part, int t_main, int split,
                               int tiles_m, int tiles_n, const float* sa, const float* sb, int vec);
bool gemm_skinny_eligible(const GemmArgs& g);
// Workgroups of the decode kernel's grid for g (one statistics partial each
// with an FP8 output).
int64_t skinny_blocks(const GemmArgs& g);

// Weight-only FP8 GEMM (gemm_wonly.hip): bf16 activations x [M x K] (ldx in
// elements), FP8 weights w [N x K] (ldw bytes) with fp32 scales
// [ceil(N/erw)][ceil(K/ecw)]; ecw >= K or a multiple of 128.
struct WonlyArgs {
  const uint16_t* x = nullptr;
  int64_t ldx = 0;
  const uint8_t* w = nullptr;
  int fw = 0;
  int64_t ldw = 0;
  const float* sw = nullptr;
  int64_t erw = 1, ecw = 1;
  int64_t M = 0, N = 0, K = 0;
  const void* bias = nullptr;
  int bias_t = 0;
  void* y = nullptr;
  int yt = 0;
  int64_t ldy = 0;
  bool w_packed = false;  // w is fragment-ordered (launch_pack_weights16)
};
hipError_t launch_gemm_wonly(const WonlyArgs& g, hipStream_t stream);

// Quantization error statistics (ledger.hip): w [N x K] (fp32 / bf16, ldw),
// codes q (ldq) with scales [ceil(N/er)][ceil(K/ec)], optional bf16 x [M x K]
// (ldx); stats: 7 device doubles.  partials: quant_error_partials_bytes(N).
struct QuantErrorArgs {
  const void* w = nullptr;
  int wt = 0;
  int64_t ldw = 0;
  const uint8_t* q = nullptr;
  int f = 0;
  int64_t ldq = 0;
  int64_t N = 0, K = 0;
  const float* scale = nullptr;
  int64_t er = 1, ec = 1;
  const uint16_t* x = nullptr;
  int64_t M = 0, ldx = 0;
  double* stats = nullptr;
};
size_t quant_error_partials_bytes(int64_t N);
hipError_t launch_quant_error(const QuantErrorArgs& g, void* partials, hipStream_t stream);
hipError_t launch_gemm_skinny(const GemmArgs& g, hipStream_t stream);
// Fragment-ordered copy of row-major codes q [N x K] (ldq; K % 128 == 0) into
// qp: 2 KB per (16-row group, 128-byte K step), groups zero-padded past N.
hipError_t launch_pack_weights16(const uint8_t* q, int64_t N, int64_t K, int64_t ldq, uint8_t* qp,
                                 hipStream_t stream);

}  // namespace fp8rt
