// Library-held scratch for callers that cannot allocate (bca_decode_noalloc).
//
// One file-scope device array per GPU the library runs on, held until the
// process ends.  In host code the array's name is only a host-side stand-in,
// so its device address is fetched once per device with hipGetSymbolAddress
// (with that device current) and cached; every use in host code -- kernel
// arguments, fills -- goes through that cached pointer.
#include <mutex>

#include "bca_kernels.hpp"

namespace bca {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace bca
