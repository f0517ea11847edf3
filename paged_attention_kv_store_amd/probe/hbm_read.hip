// Streaming HBM read, the bandwidth ceiling a read-only kernel reaches on
// this GPU: every byte of a buffer is read once with 16-byte vector loads,
// each workgroup streaming one contiguous range, several loads in flight per
// lane. The values are folded into one word per workgroup so that the loads
// are not removed. Measurement aid for the benchmark; not part of the
// attention library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 256;

template <int kInFlight>   // 16-byte loads in flight per lane
__global__ __launch_bounds__(kThreads) void hbm_read_kernel(const uint4* __restrict__ src, int64_t n16,
                                                            int64_t per_wg, uint32_t* __restrict__ sink) {
  const int64_t begin = (int64_t)blockIdx.x * per_wg;
  const int64_t end = begin + per_wg < n16 ? begin + per_wg : n16;
  uint32_t acc = 0;
  int64_t i = begin + threadIdx.x;
  for (; i + (kInFlight - 1) * kThreads < end; i += kInFlight * kThreads) {
    uint4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = src[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < end; i += kThreads) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  // one word per workgroup: the xor of all its lanes (lane 0 of each wave
  // contributes through an atomic, so the result is order-independent)
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if ((threadIdx.x & 63) == 0) atomicXor(sink + blockIdx.x, acc);
}

}  // namespace

// Read `bytes` (a multiple of 16) of device memory at `src` once, with
// `workgroups` workgroups of 256 lanes each streaming a contiguous range and
// `in_flight` (4, 8 or 16) loads in flight per lane; sink: device
// uint32[workgroups], xor-accumulated. Returns a hipError_t.
extern "C" int pkv_probe_hbm_read(const void* src, size_t bytes, int32_t workgroups, int32_t in_flight, void* sink,
                                  void* stream) {
  if (!src || !sink || workgroups <= 0 || bytes % 16 != 0) return (int)hipErrorInvalidValue;
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t per_wg = (n16 + workgroups - 1) / workgroups;
  const dim3 grid((unsigned)workgroups), block(kThreads);
  const hipStream_t st = (hipStream_t)stream;
  const uint4* s = reinterpret_cast<const uint4*>(src);
  uint32_t* k = reinterpret_cast<uint32_t*>(sink);
  switch (in_flight) {
    case 4: hipLaunchKernelGGL(hbm_read_kernel<4>, grid, block, 0, st, s, n16, per_wg, k); break;
    case 8: hipLaunchKernelGGL(hbm_read_kernel<8>, grid, block, 0, st, s, n16, per_wg, k); break;
    case 16: hipLaunchKernelGGL(hbm_read_kernel<16>, grid, block, 0, st, s, n16, per_wg, k); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
