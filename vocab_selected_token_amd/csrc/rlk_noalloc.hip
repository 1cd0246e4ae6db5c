// rlk_noalloc.hip -- the library's own device scratch, for the entry point that
// allocates nothing (rlk_logp_fwd_noalloc).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy until the process ends.  In host code the array's name stands for
// a host-side placeholder, not a device address, so it is never passed to a
// kernel or a copy.  Its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and kept per device; the entry
// point hands that address to the kernels as the workspace.  Every call on one
// GPU shares the array, and the last call's contents stay in it: the kernels
// write every partial they later read, and the status words are cleared by the
// forward itself when it validates.  Calls that overlap on one GPU (two host
// threads, or two streams) race on it.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "rlk_internal.h"

namespace rlk {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace rlk
