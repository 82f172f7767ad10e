// Static device scratch of the allocation-free forward entry point.
//
// mosaic_bsa_forward_noalloc serves callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc).  Its workspace (pooled q̄, k̄, v̄, o_CG, the per-block
// largest key norms, k̄'s bf16 pieces and |k̄_j|^2) lives in the file-scope
// array below instead of a caller buffer.  Each GPU gets its own copy when this code object is loaded
// on it and keeps it until the process ends.  Host code never uses the
// array's name as a device address: the address comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept in a per-device table.  Every call on a GPU shares that GPU's
// array, so calls that overlap on one GPU (different streams or threads
// without ordering) race.
#include <hip/hip_runtime.h>

#include <mutex>
#include <unordered_map>

#include "bsa_launch.h"

namespace mosaic {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;   // device ordinal -> that device's copy of `scratch`
}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    it = g_scratch_ptr.emplace(dev, p).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace mosaic
