// The fixed device scratch of the entry points that allocate nothing
// (qwattn_decode_noalloc): a file-scope array of kNoAllocScratchBytes in every
// device's global memory, held from the code object's load until the process
// ends.  Host code must never pass the array's name to a kernel or a copy: on
// the host it names a stand-in, not the device memory.  decode_scratch looks
// the device address up once per device (hipGetSymbolAddress with that device
// current) and hands out that address from then on.
#include <mutex>

#include "kernels.h"

namespace qw {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t decode_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace qw
