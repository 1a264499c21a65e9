// Static device scratch for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc): nt_pair_block_noalloc keeps the block's workspace (the fp32
// projections a and b and the fp32 column mean m) in a file-scope device
// array instead of a caller buffer. Each GPU the library runs on holds its
// own copy, at its own address, until the process ends; calls on one GPU
// share it, so calls that overlap in time on one GPU race.
#include <mutex>

#include "nt_internal.hpp"

namespace nt {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];  // the device address of `scratch`, per device
std::mutex g_scratch_mu;

}  // namespace

// The array's device address on the current device, looked up once per
// device (with that device current) and cached. In host code the array's
// name is a host-side stand-in, never a device address: kernels only ever
// receive the pointer returned here.
hipError_t static_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace nt
