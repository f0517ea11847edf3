// kv_cache_store: scatter new K/V token rows into their cache slots.
//
// A token's row (all kv-heads x head_dim) is contiguous both in the new-row
// tensors [T, Hkv, D] and in the cache [NB, bs, Hkv, D], because a slot names
// one (block, row) pair: slot = block * block_size + row. The store is thus a
// scatter of contiguous rows, done as 16-byte vector copies with each lane
// moving one 16-byte piece of K and the same piece of V.
// Pure data movement: bit-exact for every dtype.
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

}  // namespace pkv
