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

namespace {

// Paged gather read: the K and V bytes of one decode layer, read in the
// decode's pattern -- 16-row tiles of one kv-head's slice of the cache rows,
// at the cache's row pitch, listed by their first row's byte offset -- with
// the tiles split evenly over the waves and nothing computed: the rate that
// access pattern allows when every wave has the same work. Waves are
// numbered contiguously per XCD (workgroups go to the 8 XCDs round robin),
// so a list ordered kv-head first gives each XCD one kv-head's tiles when
// there are 8. Lane l reads quarter l % 4 of row l / 4 of a tile.
template <int kSliceBytes>   // one kv-head's part of a row: 256 (bf16, head_dim 128) or 128 (E4M3)
__global__ __launch_bounds__(kThreads) void paged_read_kernel(const char* __restrict__ k, const char* __restrict__ v,
                                                              const int64_t* __restrict__ tiles, int32_t ntiles,
                                                              int64_t pitch, uint32_t* __restrict__ sink) {
  constexpr int kLoads = kSliceBytes / 4 / 16;   // 16-byte loads per lane, tile and tensor
  constexpr int kWaves = kThreads / 64;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int nwg = gridDim.x;   // a multiple of 8
  const int wave = ((int)(blockIdx.x % 8) * (nwg / 8) + (int)(blockIdx.x / 8)) * kWaves + w;
  const int share = (ntiles + nwg * kWaves - 1) / (nwg * kWaves);
  const int a = min(wave * share, ntiles), b = min(a + share, ntiles);
  const int64_t lane_off = (int64_t)(lane >> 2) * pitch + (lane & 3) * (kSliceBytes / 4);
  uint32_t acc = 0;
  uint4 r0[2 * kLoads], r1[2 * kLoads];
  auto load = [&](int64_t off, uint4 (&r)[2 * kLoads]) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      r[i] = *reinterpret_cast<const uint4*>(k + off + lane_off + 16 * i);
      r[kLoads + i] = *reinterpret_cast<const uint4*>(v + off + lane_off + 16 * i);
    }
  };
  auto fold = [&](const uint4 (&r)[2 * kLoads]) {
#pragma unroll
    for (int i = 0; i < 2 * kLoads; ++i) acc ^= r[i].x ^ r[i].y ^ r[i].z ^ r[i].w;
  };
  for (int c = a; c < b; c += 64) {
    // the offsets of up to 64 tiles of the share, one per lane
    const int n = min(64, b - c);
    const int64_t my = lane < n ? tiles[c + lane] : 0;
    auto off = [&](int j) { return (int64_t)__shfl(my, j, 64); };
    load(off(0), r0);
    int j = 0;
    for (; j + 1 < n; j += 2) {
      load(off(j + 1), r1);
      fold(r0);
      if (j + 2 < n) load(off(j + 2), r0);
      fold(r1);
    }
    if (j < n) fold(r0);
  }
  for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, 64);
  if (lane == 0) atomicXor(sink + blockIdx.x, acc);
}

}  // namespace

// Read the tiles listed in `tiles` (device int64[ntiles]: byte offset, within
// k and v, of a tile's first row slice) from both k and v: 16 rows of
// slice_bytes (256 or 128) each, rows `pitch` bytes apart, with `workgroups`
// (a multiple of 8) workgroups of 4 waves sharing the tiles evenly; sink:
// device uint32[workgroups], xor-accumulated. Returns a hipError_t.
extern "C" int pkv_probe_paged_read(const void* k, const void* v, const int64_t* tiles, int32_t ntiles, int64_t pitch,
                                    int32_t slice_bytes, int32_t workgroups, void* sink, void* stream) {
  if (!k || !v || !tiles || !sink || ntiles < 0 || workgroups <= 0 || workgroups % 8 != 0 || pitch <= 0)
    return (int)hipErrorInvalidValue;
  if (ntiles == 0) return (int)hipSuccess;
  const dim3 grid((unsigned)workgroups), block(kThreads);
  const hipStream_t st = (hipStream_t)stream;
  const char* kc = reinterpret_cast<const char*>(k);
  const char* vc = reinterpret_cast<const char*>(v);
  uint32_t* s = reinterpret_cast<uint32_t*>(sink);
  switch (slice_bytes) {
    case 256: hipLaunchKernelGGL(paged_read_kernel<256>, grid, block, 0, st, kc, vc, tiles, ntiles, pitch, s); break;
    case 128: hipLaunchKernelGGL(paged_read_kernel<128>, grid, block, 0, st, kc, vc, tiles, ntiles, pitch, s); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}
