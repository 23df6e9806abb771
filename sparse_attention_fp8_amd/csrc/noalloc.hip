// Device scratch of dsa_sparse_mla_decode_noalloc: the split partials live in
// a file-scope device array instead of a caller workspace, so the call needs
// no allocation at all (for callers that cannot allocate: code under HIP
// graph capture, tight serving loops, harnesses that forbid it).
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and only that address is ever handed to a kernel.
// Every call on one device shares its copy of the array (each device that
// runs the library holds one until the process ends), so calls that overlap
// on one device race; the array keeps whatever the last call wrote.
#include <hip/hip_runtime.h>

#include <mutex>

#include "dsa.h"
#include "kernels.h"

namespace dsa {

namespace {

static __device__ __align__(256) unsigned char scratch[DSA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device (null until looked up)

}  // namespace

size_t static_scratch_bytes() { return sizeof(scratch); }

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // the current device's copy
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dsa
