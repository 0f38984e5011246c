// Scratch memory of the no-allocation entry point (qlora_linear_fwd_noalloc),
// for callers that cannot allocate: code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc.
//
// The buffer is a file-scope device array, so every GPU the library runs on
// holds its own copy from module load until the process ends. On the host,
// the array's name only stands in for the symbol: it is never passed to a
// kernel, a copy or a fill. Host code uses the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device with that device current and kept below.
#include <mutex>

#include "common.hpp"
#include "kernels.hpp"

namespace qlora {

namespace {
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_device_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace qlora
