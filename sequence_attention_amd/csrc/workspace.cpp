// Per-device and per-stream resources shared by the launchers.
#include <map>
#include <mutex>
#include <utility>

#include "dit_internal.h"

namespace dit {

hipError_t device_cu_count(int* cus) {
  static int cached[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  if (cached[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    cached[dev] = n > 0 ? n : 1;
  }
  *cus = cached[dev];
  return hipSuccess;
}

namespace {

struct Buffer {
  void* ptr = nullptr;
  size_t bytes = 0;
};

struct StreamBuffers {
  Buffer zeroed;   // kept all-zero between kernels by its users
  Buffer scratch;  // contents undefined
};

std::mutex g_mutex;
std::map<std::pair<int, hipStream_t>, StreamBuffers> g_buffers;

// Grow `buf` to at least `bytes`; a fresh allocation is zero-filled when
// `zero` is set.  Growth first waits for the stream, whose earlier kernels
// may still use the old allocation.
hipError_t ensure(Buffer& buf, size_t bytes, bool zero, hipStream_t stream) {
  if (buf.bytes >= bytes) return hipSuccess;
  hipError_t e;
  if (buf.ptr != nullptr) {
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return e;
    if ((e = hipFree(buf.ptr)) != hipSuccess) return e;
    buf = Buffer();
  }
  const size_t want = bytes + bytes / 4;  // headroom against repeated growth
  void* p = nullptr;
  if ((e = hipMalloc(&p, want)) != hipSuccess) return e;
  if (zero && (e = hipMemsetAsync(p, 0, want, stream)) != hipSuccess) {
    (void)hipFree(p);
    return e;
  }
  buf.ptr = p;
  buf.bytes = want;
  return hipSuccess;
}

}  // namespace

hipError_t stream_workspace(hipStream_t stream, size_t zeroed_bytes, size_t scratch_bytes,
                            void** zeroed, void** scratch) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mutex);
  StreamBuffers& sb = g_buffers[{dev, stream}];
  if ((e = ensure(sb.zeroed, zeroed_bytes, true, stream)) != hipSuccess) return e;
  if ((e = ensure(sb.scratch, scratch_bytes, false, stream)) != hipSuccess) return e;
  *zeroed = sb.zeroed.ptr;
  *scratch = sb.scratch.ptr;
  return hipSuccess;
}

}  // namespace dit
