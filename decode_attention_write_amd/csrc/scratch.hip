// Device scratch for the allocation-free decode step (oscar_decode_step_noalloc): the split
// partials, prepared queries and page-group counters that oscar_decode_step keeps in the
// caller's workspace live here instead, in a file-scope device array.  Each GPU the library runs
// on holds its own copy of the array (at its own address) from the moment the code object is
// loaded until the process ends.
//
// The array's name is only a host-side stand-in: its device address on the current device is
// looked up once per device with hipGetSymbolAddress and cached; host code passes that address
// to the kernels, never the name.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"
#include "oscar.h"

namespace oscar {

static __device__ __align__(256) uint8_t scratch[OSCAR_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace oscar
