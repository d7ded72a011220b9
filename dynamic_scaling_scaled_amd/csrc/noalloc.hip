// noalloc.hip -- the fixed device scratch of the allocation-free GEMM entry
// point (fp8_scaled_gemm_noalloc): a file-scope device array, one copy per
// GPU, that lives as long as the process.
//
// In host code `scratch` names a host-side stand-in, not device memory, so
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to kernels.
#include <mutex>

#include "internal.h"

namespace fp8rt {

// kNoAllocScratchBytes = 16 MiB: the repacked 1x32 exponents of a
// 8192 x 18432 x 7168 GEMM take 6.0 MB and its transposed 1x128 A scales
// 1.8 MB; a split last wave takes as many K parts as fit (256 KB per part and
// split tile).
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex* mu = new std::mutex;  // never destroyed: no work at exit
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(*mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace fp8rt
