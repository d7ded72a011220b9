// workspace.hip -- per-(device, stream) device workspace for the cross-block
// results of the quantize kernels (the per-block partials of an amax pass and
// of a cast pass).  Allocated and zeroed once per pair on first use and kept
// for the life of the process.
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

}  // namespace fp8rt
