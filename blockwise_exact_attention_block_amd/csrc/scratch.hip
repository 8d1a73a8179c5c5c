// Library-owned device scratch for the one entry point that must not allocate
// (ra_splitkv_decode_noalloc): a fixed-size file-scope device array. Every GPU the
// library runs on holds its own copy of it at its own address until the process
// ends. In host code the array's name is only a host-side stand-in, so its device
// address is looked up with hipGetSymbolAddress, once per device with that device
// current, and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

namespace ra {

constexpr size_t kScratchBytes = size_t(16) << 20;   // 16 MiB per device

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device ordinal
}  // namespace

size_t scratch_bytes() { return kScratchBytes; }

// The current device's copy of the scratch array. The first call on a device looks
// its address up (with that device current, as the caller's device is) and keeps
// it; later calls return the kept address.
hipError_t device_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace ra
