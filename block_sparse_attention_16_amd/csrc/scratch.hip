// Device-resident scratch for the narrowing entry point that takes no
// workspace (bsa_select_from_mass_noalloc), for callers that cannot allocate
// device memory.  The array and the lookup of its device address sit in this
// file; the kernels receive the address as an ordinary argument.
#include "bsa_internal.h"

#include <mutex>

namespace bsa {

// The narrowing kernels' counts and bitmask.  One copy per GPU, held until
// the process ends; every call on a GPU shares it, so calls that overlap on
// one GPU race.  Both kernels overwrite what they use (every row's count and
// every bitmask word), so nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_for_stream(hipStream_t stream, void** ptr) {
  int dev = 0;
  hipError_t e = hipSuccess;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    dev = (int)d;
  } else {
    e = hipGetDevice(&dev);
  }
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    // The array's host-side name is only a stand-in: its device address is
    // looked up once per device, with that device current (made current for
    // the lookup only; the caller's current device is restored).
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bsa
