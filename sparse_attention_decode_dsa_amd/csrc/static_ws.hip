// The fused layer entry without a caller workspace: its scores, top-k and split-MLA
// scratch live in one fixed device array of this library, so the call allocates nothing
// (for code under HIP graph capture, serving loops and harnesses that cannot allocate).
//
// The array is a file-scope device variable.  Its name is a host-side stand-in in host
// code, never a device address: the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept per device; only that address
// is handed to kernels.  Every GPU the library runs on holds its own copy of the array
// until the process ends.  Calls on one GPU share that GPU's array, so calls that overlap
// in time on one GPU (different streams, or host threads without ordering) race; each
// call's kernels write every scratch byte they later read, so no clearing is needed.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ml4_launch.h"
#include "ml4dsa.h"

static __device__ __align__(256) unsigned char scratch[ML4_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

namespace ml4 {

// Looked up once per device, with that device current (each device holds its own copy of
// the array at its own address); kernels only ever receive this address.
hipError_t static_scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
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

}  // namespace ml4
