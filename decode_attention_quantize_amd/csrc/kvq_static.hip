// kvq_static.hip -- the library's static decode scratch: one fixed-size
// device array per GPU, for the decode entry point that allocates nothing.
//
// The array is a file-scope __device__ object, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host
// code never passes the array's name to a kernel (on the host that name is a
// stand-in, not a device address): the device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and cached.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "kvq_internal.h"

namespace kvq {
namespace {

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

struct DeviceScratch {
  void* ptr = nullptr;
  bool ready = false;
};
DeviceScratch g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void zero_words_kernel(uint32_t* p, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

}  // namespace

// Device address of the current device's scratch array.  Layout: split
// partials in the first kStaticPartialsBytes, then a fixed tail of
// kStaticCounterBytes holding one arrival counter per unit (LDS-staged
// decode) and, in its last word, the non-finite output row count.  The first
// call on a device looks the address up and zeroes that tail (every decode
// leaves its counters at zero again; the row count is reset when it is
// read); it synchronizes the device.  Later calls only read the cached
// pointer.
hipError_t static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  DeviceScratch& d = g_scratch[dev];
  if (!d.ready) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255)) return hipErrorInvalidValue;
    // the fixed tail: per-unit arrival counters, then the non-finite count
    uint32_t* tail = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p) + kStaticPartialsBytes);
    const int64_t words = static_cast<int64_t>(kStaticCounterBytes / 4);
    hipLaunchKernelGGL(zero_words_kernel, dim3(16), dim3(256), 0, nullptr, tail, words);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    d.ptr = p;
    d.ready = true;
  }
  *out = d.ptr;
  return hipSuccess;
}

}  // namespace kvq
