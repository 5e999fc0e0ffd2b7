// Static device scratch of cp_attn_rank_forward_static: the two receive slots
// and the running state of one rank forward, in a file-scope device array of
// CP_STATIC_SCRATCH_BYTES, so that callers who cannot allocate device memory
// (code under stream capture, tight serving loops, harnesses that forbid
// allocation) can run the forward without a workspace.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code `scratch` names a host-side stand-in, not a
// device address; its device address is looked up once per device with that
// device current, and only that address is ever handed to kernels or copies.
#include "launch.h"
#include "cpattn.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

__device__ __align__(256) unsigned char scratch[CP_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_addr[kMaxDevices];   // device address of `scratch` per device, once looked up

}  // namespace

namespace cpattn {

hipError_t static_scratch(void** addr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || reinterpret_cast<uintptr_t>(p) % 256 != 0) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  *bytes = CP_STATIC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace cpattn
