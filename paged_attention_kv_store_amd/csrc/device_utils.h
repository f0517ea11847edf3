// Device helpers shared by the kernels: bf16 conversions, vector types,
// cross-lane reductions for 64-wide wavefronts.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// bf16 is the upper half of an IEEE fp32: widening is a 16-bit shift.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to bf16 (nearest even, the hardware default mode;
// v_cvt_pk_bf16_f32) and packed low/high into one 32-bit word.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// One fp32 value rounded to bf16 (nearest even).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) { return (uint16_t)pack_bf16x2(f, 0.f); }

template <typename T>
__device__ __forceinline__ T bit_cast_to(const uint4& v) {
  static_assert(sizeof(T) == sizeof(uint4), "size mismatch");
  return __builtin_bit_cast(T, v);
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) { return __shfl_xor(x, mask, 64); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// 16-byte global load that bypasses nothing special; kept as a single
// dwordx4 access.
__device__ __forceinline__ uint4 load16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint2 load8(const void* p) { return *reinterpret_cast<const uint2*>(p); }

// Max of v over the four lanes l, l^16, l^32, l^48 (the 16-lane rows of the
// wave), with the gfx950 row-swap instructions instead of LDS permutes:
// permlane16_swap(x, x) leaves rows (0,0,2,2) in one result and (1,1,3,3) in
// the other, permlane32_swap(x, x) the lower and the upper halves.
// NaN-propagating (IEEE maximum, v_maximum3_f32 on gfx950: no canonicalising
// moves as with fmaxf).
__device__ __forceinline__ float max_across_rows(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// NaN-propagating maximum of eight values (three v_maximum3_f32 on gfx950)
__device__ __forceinline__ float max8(const float (&x)[8]) {
  const auto mx = [](float a, float b) { return __builtin_elementwise_maximum(a, b); };
  return mx(mx(mx(x[0], x[1]), mx(x[2], x[3])), mx(mx(x[4], x[5]), mx(x[6], x[7])));
}

// Two bf16 words holding the exact values of the four E4M3 codes of w (every
// E4M3 value is a bf16 value). gfx950's scaled conversion goes straight to
// packed bf16, scale 1; checked on the GPU to give, for all 256 codes, the
// bits of the E4M3 -> f32 conversion followed by the nearest-even bf16 pack.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
}

// ---- E4M3 quantisation (the cache format's reading) ------------------------
// t = x / scale as one IEEE float32 division, clamped to +-448 (a NaN passes
// through), rounded to the nearest E4M3 code with ties to even by the
// hardware conversion; a NaN becomes the canonical code 0x7f (the conversion
// would set the sign bit). Used by the store and by the store fused into
// decode, so both write the same bytes.
__device__ __forceinline__ float clamp_e4m3(float t) {
  return t > 448.f ? 448.f : (t < -448.f ? -448.f : t);
}

// codes of x[0..3] / s, packed little-endian
__device__ __forceinline__ uint32_t quantize4(const float* x, float s) {
  float t[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) t[i] = clamp_e4m3(x[i] / s);
  uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
  w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], (int)w, true);
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (t[i] != t[i]) w = (w & ~(0xffu << (8 * i))) | (0x7fu << (8 * i));
  return w;
}

// codes of the 8 bf16 values in v, divided by s
__device__ __forceinline__ uint2 quantize8_bf16(const uint4& v, float s) {
  const float x[8] = {bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y),
                      bf16_lo(v.z), bf16_hi(v.z), bf16_lo(v.w), bf16_hi(v.w)};
  return make_uint2(quantize4(x, s), quantize4(x + 4, s));
}

// ---- items in order of cost ------------------------------------------------
// The item of the given rank when items 0 .. n_items-1 are ordered by cost,
// highest first, ties by index; -1 past the last rank. cost_of(j) is an
// integer in [0, kBuckets). Called by the whole workgroup of kThreads
// threads (rank and n_items workgroup-uniform): a histogram of the costs in
// LDS gives the cost of the rank and its place among the items of that
// cost, then a scan in index order picks the item. hist (kBuckets ints) and
// cost (n_items entries) are LDS the caller does not use again until after
// the barrier this ends with. O(n_items / kThreads) per thread.
template <int kThreads, int kBuckets, typename CostFn>
__device__ int item_of_rank(int rank, int n_items, CostFn cost_of, int* hist, uint16_t* cost) {
  static_assert(kBuckets % kThreads == 0 && kThreads % 64 == 0, "bucket split");
  constexpr int kWaves = kThreads / 64;
  constexpr int kPerThread = kBuckets / kThreads;
  __shared__ int s_wave[kWaves];
  __shared__ int s_pick[2];
  if (rank >= n_items) return -1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < kBuckets; i += kThreads) hist[i] = 0;
  __syncthreads();
  for (int j = tid; j < n_items; j += kThreads) {
    const int b = cost_of(j);
    cost[j] = (uint16_t)b;
    atomicAdd(&hist[b], 1);
  }
  __syncthreads();
  // items in this thread's buckets, and in all higher buckets (a suffix sum
  // over threads: lanes above within the wave, then the waves above)
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) mine += hist[kPerThread * tid + i];
  int suffix = mine;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int x = __shfl_down(suffix, d, 64);
    if (lane + d < 64) suffix += x;
  }
  if (lane == 0) s_wave[w] = suffix;
  __syncthreads();
  int above = suffix - mine;
  for (int v = w + 1; v < kWaves; ++v) above += s_wave[v];
  if (above <= rank && rank < above + mine) {
    for (int i = kPerThread - 1; i >= 0; --i) {
      const int cnt = hist[kPerThread * tid + i];
      if (rank < above + cnt) {
        s_pick[0] = kPerThread * tid + i;
        s_pick[1] = rank - above;
        break;
      }
      above += cnt;
    }
  }
  __syncthreads();
  // the k-th item (in index order) of the chosen bucket
  const int bucket = s_pick[0];
  int k = s_pick[1];
  int item = -1;
  for (int base = 0; base < n_items; base += kThreads) {
    const int j = base + tid;
    const bool hit = j < n_items && cost[j] == bucket;
    const uint64_t mask = __ballot(hit);
    __syncthreads();                        // s_wave of the previous pass is read
    if (lane == 0) s_wave[w] = __popcll(mask);
    __syncthreads();
    int before = 0, total = 0;
    for (int v = 0; v < kWaves; ++v) {
      before += v < w ? s_wave[v] : 0;
      total += s_wave[v];
    }
    if (k < total) {
      if (hit && before + __popcll(mask & ((1ull << lane) - 1)) == k) s_pick[0] = j;
      __syncthreads();
      item = s_pick[0];
      break;
    }
    k -= total;
  }
  __syncthreads();                          // hist, cost and s_pick are free again
  return item;
}

}  // namespace pkv
