// The static device buffer of mla_decode_fwd_noalloc: the split schedule and
// the partials of a no-allocation decode live here instead of in caller
// buffers. Each device that loads the library holds its own copy of the array
// until the process ends. In host code the array's name is only a host-side
// stand-in: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to a kernel or a copy.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "mla_decode.h"
#include "mla_internal.h"

static __device__ __align__(256) uint8_t scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};
}  // namespace

namespace mla {

hipError_t scratch_address(int dev, void** out) {
  *out = nullptr;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev) return hipErrorInvalidDevice;   // the lookup needs `dev` current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace mla
