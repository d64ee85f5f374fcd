// The library's static device scratch: the workspace of the allocation-free
// decode entry point (ds4q_moe_decode_static), for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid the allocator).
//
// One array of DS4Q_SCRATCH_BYTES per device, part of the code object: the
// loader reserves it on each device the library runs on, and it stays until
// the process ends.  In host code the array's name only stands for the
// symbol; its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is
// ever handed to kernels or runtime calls.  Every call on a device uses the
// same array, so calls that overlap in time on one device race; each call
// leaves its contents behind and nothing in the decode path reads a byte of
// the workspace that the same call did not write first.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/ds4q.h"
#include "launch.h"

static __device__ __align__(256) unsigned char scratch[DS4Q_SCRATCH_BYTES];

namespace ds4q {

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void *g_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t scratch_address(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace ds4q
