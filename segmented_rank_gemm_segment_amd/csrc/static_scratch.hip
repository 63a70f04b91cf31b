// Device scratch of the allocation-free layer call (lora_linear_fused_static).
//
// The call keeps what lora_linear_fused takes as workspace arguments -- the
// segment metadata and H -- in one file-scope device array instead, so that
// its caller passes only inputs and outputs and nothing is allocated.  Each
// GPU the library runs on holds its own copy of the array (at its own
// address) until the process ends.  Host code never uses the array's name as
// an address: the device address is looked up once per device with
// hipGetSymbolAddress and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/lora.h"
#include "lora_kernels.h"

namespace lora {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace lora
