// workspace.hip -- per-(device, stream) device workspace for the cross-block
// results of the quantize kernels (the per-block partials of an amax pass and
// of a cast pass).  Allocated and zeroed once per pair on first use and kept
// for the life of the process.  Also a growable per-pair scratch buffer for
// the GEMM's repacked block scales, and the compute-unit count of a device.
#include <mutex>
#include <utility>
#include <map>

#include "internal.h"

namespace fp8rt {

hipError_t get_workspace(hipStream_t stream, DevWorkspace** ws) {
  static std::mutex mu;
  static std::map<std::pair<int, uintptr_t>, DevWorkspace*> table;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(stream));
  std::lock_guard<std::mutex> lock(mu);
  auto it = table.find(key);
  if (it != table.end()) {
    *ws = it->second;
    return hipSuccess;
  }
  void* p = nullptr;
  e = hipMalloc(&p, sizeof(DevWorkspace));
  if (e != hipSuccess) return e;
  e = hipMemset(p, 0, sizeof(DevWorkspace));
  if (e == hipSuccess) e = hipDeviceSynchronize();  // zeroed before any stream uses it
  if (e != hipSuccess) {
    (void)hipFree(p);
    return e;
  }
  *ws = static_cast<DevWorkspace*>(p);
  table.emplace(key, *ws);
  return hipSuccess;
}

hipError_t get_scratch(hipStream_t stream, size_t bytes, void** ptr) {
  static std::mutex mu;
  static std::map<std::pair<int, uintptr_t>, std::pair<void*, size_t>> table;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const auto key = std::make_pair(dev, reinterpret_cast<uintptr_t>(stream));
  std::lock_guard<std::mutex> lock(mu);
  auto& slot = table[key];
  if (slot.second >= bytes) {
    *ptr = slot.first;
    return hipSuccess;
  }
  if (slot.first) {
    e = hipStreamSynchronize(stream);  // earlier work on this stream may still read it
    if (e != hipSuccess) return e;
    e = hipFree(slot.first);
    slot = {nullptr, 0};
    if (e != hipSuccess) return e;
  }
  const size_t want = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);  // whole MiB
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) return e;
  slot = {p, want};
  *ptr = p;
  return hipSuccess;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  (void)hipGetDevice(&dev);
  if (dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

}  // namespace fp8rt
