// workspace.hip -- per-(device, stream) device memory of the library: the
// per-block partials of the quantize kernels (a fixed 256 KB workspace) and a
// scratch buffer for the GEMM's repacked block scales, the FP32 parts of a
// split last wave and the cast-transpose's per-group arrays.
//
// Lifetime rules, chosen so that a HIP graph captured after warm-up stays
// valid:
//   - memory is allocated on first use and never freed or moved while the
//     process runs: when the scratch of a pair must grow, the new buffer is
//     allocated and the old one is kept, so a graph that captured the old
//     address replays into live memory (the superseded buffers cost at most
//     as much again as the current one, since each growth at least doubles);
//   - nothing is zeroed or synchronized on first use (every partial is written
//     by the kernel that produces it before the kernel that reads it runs), so
//     no call waits on the device;
//   - the tables live on the heap and are never destroyed, so no destructor
//     runs (and no HIP call is made) at process exit.
// Calls on one stream are ordered and share that stream's memory; a graph
// replayed on another stream while eager calls run on its capture stream
// would share it concurrently, so graphs are replayed on the capture stream
// or with no overlapping calls on it.
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "internal.h"

namespace fp8rt {

namespace {

struct Slot {
  DevWorkspace* ws = nullptr;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  std::vector<void*> retired;  // superseded scratch buffers, kept alive
};

std::mutex& table_mutex() {
  static std::mutex* mu = new std::mutex;
  return *mu;
}

Slot& slot_of(int dev, hipStream_t stream) {
  static auto* table = new std::map<std::pair<int, uintptr_t>, Slot>;
  return (*table)[std::make_pair(dev, reinterpret_cast<uintptr_t>(stream))];
}

}  // namespace

hipError_t get_workspace(hipStream_t stream, DevWorkspace** ws) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(table_mutex());
  Slot& s = slot_of(dev, stream);
  if (!s.ws) {
    void* p = nullptr;
    e = hipMalloc(&p, sizeof(DevWorkspace));
    if (e != hipSuccess) return e;
    s.ws = static_cast<DevWorkspace*>(p);
  }
  *ws = s.ws;
  return hipSuccess;
}

hipError_t get_scratch(hipStream_t stream, size_t bytes, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(table_mutex());
  Slot& s = slot_of(dev, stream);
  if (s.scratch_bytes >= bytes) {
    *ptr = s.scratch;
    return hipSuccess;
  }
  size_t want = (bytes + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);  // whole MiB
  if (want < 2 * s.scratch_bytes) want = 2 * s.scratch_bytes;
  void* p = nullptr;
  e = hipMalloc(&p, want);
  if (e != hipSuccess) return e;
  if (s.scratch) s.retired.push_back(s.scratch);
  s.scratch = p;
  s.scratch_bytes = want;
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
