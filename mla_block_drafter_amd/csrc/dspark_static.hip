// Device-resident scratch for dspark_draft_block_static: the draft pass for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope __device__ array: each GPU the library runs on
// holds its own copy, allocated when the code object is loaded and kept until
// the process ends.  In host code the array's name is only a stand-in, not a
// device address, so it is never passed to a kernel or a copy: the address is
// looked up once per device with hipGetSymbolAddress, with that device
// current, and that pointer is what the pass uses.
#include <mutex>

#include "../../include/dspark.h"
#include "kernels.h"

namespace dspark {

namespace {

__device__ __align__(256) unsigned char scratch[DSPARK_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device is current
    if (e != hipSuccess) return e;
    if (!p || (uintptr_t)p % 256) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = DSPARK_STATIC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace dspark
