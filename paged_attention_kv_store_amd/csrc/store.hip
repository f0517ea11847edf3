// kv_cache_store: scatter new K/V token rows into their cache slots.
//
// A token's row (all kv-heads x head_dim) is contiguous both in the new-row
// tensors [T, Hkv, D] and in the cache [NB, bs, Hkv, D], because a slot names
// one (block, row) pair: slot = block * block_size + row. The store is thus a
// scatter of contiguous rows, done as 16-byte vector copies with each lane
// moving one 16-byte piece of K and the same piece of V.
// Pure data movement: bit-exact for every dtype. The E4M3 variant below
// quantises on the way.
#include "common.h"
#include "device_utils.h"

namespace pkv {

__global__ __launch_bounds__(256) void kv_store_kernel(StoreParams p) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)p.num_tokens * p.row_vec16;
  if (idx >= total) return;
  const int64_t t = idx / p.row_vec16;
  const int64_t piece = idx - t * p.row_vec16;
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // padding / outside the pool
  const uint4* ks = reinterpret_cast<const uint4*>(p.k) + t * p.row_vec16 + piece;
  const uint4* vs = reinterpret_cast<const uint4*>(p.v) + t * p.row_vec16 + piece;
  uint4* kd = reinterpret_cast<uint4*>(p.k_cache) + (int64_t)slot * p.row_vec16 + piece;
  uint4* vd = reinterpret_cast<uint4*>(p.v_cache) + (int64_t)slot * p.row_vec16 + piece;
  const uint4 kv = *ks;
  const uint4 vv = *vs;
  *kd = kv;
  *vd = vv;
}

hipError_t launch_store(const StoreParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_tokens * p.row_vec16;
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const int64_t blocks = (total + threads - 1) / threads;
  hipLaunchKernelGGL(kv_store_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// E4M3 store: each lane quantises (quantize4 in device_utils.h) 8
// consecutive elements of one token row of K and the same 8 of V, with the
// scale of their kv-head.
// ---------------------------------------------------------------------------
template <bool kF32>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float* x) {
  if constexpr (kF32) {
    const float4* p = reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + elem);
    const float4 a = p[0], b = p[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + elem);
    x[0] = bf16_lo(v.x); x[1] = bf16_hi(v.x); x[2] = bf16_lo(v.y); x[3] = bf16_hi(v.y);
    x[4] = bf16_lo(v.z); x[5] = bf16_hi(v.z); x[6] = bf16_lo(v.w); x[7] = bf16_hi(v.w);
  }
}

template <bool kF32>
__global__ __launch_bounds__(256) void kv_store_fp8_kernel(StoreFp8Params p) {
  const int pieces = p.row_elems / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)p.num_tokens * pieces) return;
  const int64_t t = idx / pieces;
  const int e0 = (int)(idx - t * pieces) * 8;
  const int32_t slot = p.slot_mapping[t];
  if (slot < 0 || (int64_t)slot >= p.num_slots) return;  // padding / outside the pool
  const int g = e0 / p.head_dim;
  float kx[8], vx[8];
  load8<kF32>(p.k, t * p.row_elems + e0, kx);
  load8<kF32>(p.v, t * p.row_elems + e0, vx);
  const float ks = p.k_scale[g], vs = p.v_scale[g];
  const int64_t dst = (int64_t)slot * p.row_elems + e0;
  *reinterpret_cast<uint2*>(p.k_cache + dst) = make_uint2(quantize4(kx, ks), quantize4(kx + 4, ks));
  *reinterpret_cast<uint2*>(p.v_cache + dst) = make_uint2(quantize4(vx, vs), quantize4(vx + 4, vs));
}

hipError_t launch_store_fp8(const StoreFp8Params& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.num_tokens * (p.row_elems / 8);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  const dim3 grid((unsigned)((total + threads - 1) / threads));
  if (p.src_f32)
    hipLaunchKernelGGL(kv_store_fp8_kernel<true>, grid, dim3(threads), 0, stream, p);
  else
    hipLaunchKernelGGL(kv_store_fp8_kernel<false>, grid, dim3(threads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
