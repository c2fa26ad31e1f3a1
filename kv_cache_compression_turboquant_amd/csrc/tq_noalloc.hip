// Static device scratch for the entry point that allocates nothing (tq_scores_noalloc): callers
// that cannot allocate device memory (code under graph capture, tight serving loops) get the
// query-prologue workspace of the score path from a fixed array in the library's image instead
// of a caller buffer.  Each device holds its own copy of the array for the life of the process.
#include <hip/hip_runtime.h>

#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

constexpr size_t kScratchBytes = size_t(4) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// The device address of the current device's copy of `scratch`, looked up once per device with
// that device current (the host-side name is only a stand-in and must never reach a kernel).
hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace tq
