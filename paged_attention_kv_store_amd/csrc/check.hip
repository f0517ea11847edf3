// Debugging checks of the values the caller keeps in device memory, which
// the attention and store entry points never read on the host: context
// lengths, block-table entries, chunk boundaries and store slots. Each check
// counts the violations into a small device report; nothing is changed and
// nothing out of bounds is touched, so a check can run before a suspect call.
//
// The pool holds blocks 0 .. num_blocks-1 ("Implementation Details", section
// "PagedAttention -- BlockPool"), a sequence uses the first
// ceil(context_len / block_size) entries of its block table ("Building a
// minimal vLLM implementation", section sequence.py), and a slot names one
// row of the pool (block * block_size + row).
#include "common.h"

#include <algorithm>

namespace pkv {

namespace {
constexpr int kCheckThreads = 256;

__device__ __forceinline__ int block_sum(int v, int* s_part) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_part[w] = v;
  __syncthreads();
  int t = 0;
  for (int i = 0; i < kCheckThreads / 64; ++i) t += s_part[i];
  __syncthreads();
  return t;
}
}  // namespace

// report[0..2] = 0, report[3] = none; bits[0 .. words) = 0.
__global__ __launch_bounds__(kCheckThreads) void check_init_kernel(int32_t* report, int32_t none,
                                                                   uint32_t* bits, int64_t words) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 3) report[i] = 0;
  if (i == 3) report[3] = none;
  for (int64_t j = i; j < words; j += (int64_t)gridDim.x * blockDim.x) bits[j] = 0u;
}

// One workgroup per sequence (grid-stride): its length, the table entries
// it uses, and (chunks) its row count.
__global__ __launch_bounds__(kCheckThreads) void check_tables_kernel(CheckParams p) {
  __shared__ int s_part[kCheckThreads / 64];
  for (int s = blockIdx.x; s < p.num_seqs; s += gridDim.x) {
    const int ctx_raw = p.context_lens[s];
    const bool bad_len = ctx_raw < 0 || ctx_raw > p.max_ctx;
    const int ctx = min(max(ctx_raw, 0), p.max_ctx);
    const int used = (ctx + p.block_size - 1) / p.block_size;   // <= max_blocks by the host bound
    const int32_t* row = p.block_tables + (int64_t)s * p.max_blocks;
    int bad = 0;
    for (int j = threadIdx.x; j < used; j += kCheckThreads) bad += (unsigned)row[j] >= (unsigned)p.num_blocks;
    bad = block_sum(bad, s_part);
    bool bad_chunk = false;
    if (p.cu_seqlens_q != nullptr) {
      const int lo = p.cu_seqlens_q[s], hi = p.cu_seqlens_q[s + 1];
      const int rows = hi - lo;
      bad_chunk = rows < 0 || rows > p.max_q_len || rows > ctx_raw || (s == 0 && lo != 0) ||
                  (s == p.num_seqs - 1 && hi != p.total_q);
    }
    if (threadIdx.x == 0) {
      if (bad_len) atomicAdd(&p.report[0], 1);
      if (bad) atomicAdd(&p.report[1], bad);
      if (bad_chunk) atomicAdd(&p.report[2], 1);
      if (bad_len || bad || bad_chunk) atomicMin(&p.report[3], s);
    }
  }
}

// Tokens (grid-stride): slots past the pool, and claims of a slot that an
// earlier-arriving token already claimed (the first claim is not counted, so
// a slot named k times adds k - 1). seen / dup: one bit per pool row.
__global__ __launch_bounds__(kCheckThreads) void check_slots_mark_kernel(SlotCheckParams p) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < p.num_tokens;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int32_t slot = p.slot_mapping[t];
    if (slot < 0) {
      atomicAdd(&p.report[2], 1);
      continue;
    }
    if ((int64_t)slot >= p.num_slots) {
      atomicAdd(&p.report[0], 1);
      atomicMin(&p.report[3], (int32_t)t);
      continue;
    }
    const uint32_t bit = 1u << (slot & 31);
    const uint32_t old = atomicOr(&p.seen[slot >> 5], bit);
    if (old & bit) {
      atomicAdd(&p.report[1], 1);
      atomicOr(&p.dup[slot >> 5], bit);
    }
  }
}

// Every token whose slot is claimed more than once counts for the lowest
// offending index (so the index does not depend on which claim came first).
__global__ __launch_bounds__(kCheckThreads) void check_slots_find_kernel(SlotCheckParams p) {
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < p.num_tokens;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int32_t slot = p.slot_mapping[t];
    if (slot < 0 || (int64_t)slot >= p.num_slots) continue;
    if (p.dup[slot >> 5] & (1u << (slot & 31))) atomicMin(&p.report[3], (int32_t)t);
  }
}

static unsigned grid_for(int64_t items, int64_t per_block) {
  const int64_t g = (items + per_block - 1) / per_block;
  return (unsigned)std::min<int64_t>(std::max<int64_t>(g, 1), 65535);
}

hipError_t launch_check_tables(const CheckParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(check_init_kernel, dim3(1), dim3(kCheckThreads), 0, stream, p.report, p.num_seqs,
                     (uint32_t*)nullptr, (int64_t)0);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (p.num_seqs == 0) return hipSuccess;
  hipLaunchKernelGGL(check_tables_kernel, dim3(grid_for(p.num_seqs, 1)), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_check_slots(const SlotCheckParams& p, hipStream_t stream) {
  const int64_t words = (p.num_slots + 31) / 32;
  hipLaunchKernelGGL(check_init_kernel, dim3(grid_for(2 * words, kCheckThreads)), dim3(kCheckThreads), 0, stream,
                     p.report, p.num_tokens, p.seen, 2 * words);   // seen and dup are adjacent
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  if (p.num_tokens == 0) return hipSuccess;
  const unsigned g = grid_for(p.num_tokens, kCheckThreads);
  hipLaunchKernelGGL(check_slots_mark_kernel, dim3(g), dim3(kCheckThreads), 0, stream, p);
  if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
  hipLaunchKernelGGL(check_slots_find_kernel, dim3(g), dim3(kCheckThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
