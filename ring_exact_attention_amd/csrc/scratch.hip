// Library-owned scratch memory for the entry point that allocates nothing.
//
// One file-scope device array per GPU (every device the library runs on gets
// its own copy, held until the process ends).  In host code the array's name
// is only a host-side stand-in, so its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; that
// address, never the name, is what kernels and copies receive.
#include <mutex>

#include "common.h"

namespace bwa {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // BWA_NOALLOC_SCRATCH_BYTES
constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device, once looked up
}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

// Device address of the current device's scratch array.
hipError_t scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bwa
