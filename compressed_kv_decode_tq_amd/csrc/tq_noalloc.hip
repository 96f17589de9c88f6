// Static device scratch for the decode entry point that allocates nothing
// (tq_decode_attn_noalloc): the same workspace tq_decode_attn takes as an
// argument (query digits and constants, split partials), held in a file-scope
// device array instead, for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code `scratch` names a host-side stand-in, not the
// device address: the address is taken once per device with
// hipGetSymbolAddress and only that pointer is ever handed to kernels.
#include <mutex>

#include "tq_internal.h"

namespace tq {
namespace {

static __device__ __align__(256) uint8_t scratch[TQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  // first call on this device, with the device current: look the array's
  // device address up once and keep it
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_status[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_status[dev] == hipSuccess ? p : nullptr;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *ptr = g_ptr[dev];
  *bytes = TQ_NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace tq
