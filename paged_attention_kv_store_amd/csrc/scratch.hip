// Library-owned device scratch for the decode entry point that allocates
// nothing (pkv_paged_attention_decode_static), and a fill kernel that clears
// counters without a memset node (so a captured graph replays it correctly).
//
// The scratch is one file-scope device array. Its name, used in host code,
// is only a host-side stand-in for the symbol, not a device address: the
// address comes from hipGetSymbolAddress, looked up once per device with
// that device current, and only that address is ever handed to kernels.
#include "common.h"

#include <mutex>

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

__global__ __launch_bounds__(256) void zero_ints_kernel(int32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0;
}

hipError_t launch_zero_ints(int32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (n + threads - 1) / threads;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_ints_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, p, n);
  return hipGetLastError();
}

}  // namespace pkv
