// scratch.hip - the library-owned scratch of mla_decode_noalloc: one static
// device array, which every GPU the library runs on holds once (its own copy,
// at its own address) until the process ends.  The address is looked up once
// per device with hipGetSymbolAddress, with that device current, and host
// code uses only that address: in host code the array's name is a stand-in,
// not device memory.
#include "../../include/mla.h"
#include "mla_internal.h"

#include <mutex>

static __device__ __align__(256) unsigned char scratch[MLA_DECODE_SCRATCH_BYTES];

namespace mla {

namespace {
constexpr int kMaxDevices = 64;
}  // namespace

hipError_t decode_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = MLA_DECODE_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace mla
