// Library-owned device scratch for callers that cannot allocate: code being
// captured into a HIP graph, serving loops or harnesses that forbid
// hipMalloc.  The split-K decode's partial states (u_c, m_c, l_c) go into a
// file-scope device array instead of a caller workspace.
//
// Every GPU the library runs on holds its own copy of the array (loaded with
// the code object, kept until the process ends).  In host code the array's
// name is only a host-side stand-in: its device address is looked up once
// per device with hipGetSymbolAddress, with that device current, and that
// address is what the kernels receive.  All calls on one GPU share the
// array, so calls that overlap in time on one GPU (two streams, two host
// threads) race on it; calls ordered on one stream do not.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/fa.h"
#include "launch.h"

namespace fa {
namespace {

static __device__ __align__(256) float scratch[FA_STATIC_SCRATCH_BYTES / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
