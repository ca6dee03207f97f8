// clsa_step_no_alloc: clsa_step with its workspace taken from a library-owned static device array
// instead of a caller allocation, for callers that cannot allocate device memory (code under graph
// capture, serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this file's device code object: each GPU the library runs on holds its own
// copy (kNoAllocScratchBytes) from the first call on that GPU until the process ends.  Its device
// address is looked up once per device with hipGetSymbolAddress and kept; host code never passes
// the array's own name to a kernel (in host code that name is a stand-in, not a device address).
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "clsa_internal.h"

namespace clsa {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int no_alloc_scratch(void** ptr, std::string& err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    err = std::string("hipGetDevice: ") + hipGetErrorString(e);
    return (int)e;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    err = "device ordinal beyond the devices this library tracks";
    return (int)hipErrorInvalidDevice;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      err = std::string("hipGetSymbolAddress of the static scratch: ") + hipGetErrorString(e);
      return e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return 0;
}

}  // namespace clsa
