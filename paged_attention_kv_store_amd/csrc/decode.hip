// Decode attention over a paged KV cache: one query row per (sequence, q-head).
//
// Per-item kernels (decode_valu_kernel, decode_mfma_kernel):
// one workgroup of 4 wavefronts per (kv-head, partition, sequence).
// The grid is one-dimensional; decode_item maps a workgroup to its item in
// index order, and sized_item (the single-pass matrix-core kernel) by item
// size, so that the two workgroups sharing a compute unit pair a long item
// with a short one. A workgroup serves all G = Hq/Hkv q-heads that share the kv-head, so each K/V byte is
// read once for the whole group. The partition's tokens are cut into 16-token
// tiles; wave w takes tiles w, w+4, w+8, ... Every tile lies inside one
// physical block (block_size is a multiple of 16 and tiles start at multiples
// of 16), so one block-table entry gives the tile's 16 cache rows. Each wave
// keeps an online-softmax state (reference max in log2 units, sum, fp32
// output accumulator); the four states are merged through LDS at the end.
// A partition that is the sequence's only one writes the normalised output;
// otherwise it writes (max, sum, unnormalised output) to the split-K
// workspace and the last partition of the sequence to finish merges them
// (merge_and_write), in the same launch.
//
// Two kernel families compute the same thing:
//  * decode_valu_kernel: lanes split a cache row into 16-byte pieces; q.k dot
//    products are vector FMAs finished by xor-shuffle sums across the lanes of
//    a row; P.V is vector FMAs. Any dtype; G <= 8 for bf16, G <= 16 for fp32.
//  * decode_mfma_kernel (bf16): q.k for the 16 tile tokens x the G heads is a
//    16x16x32 bf16 matrix-core product per 32 dims of head_dim (the G heads
//    are padded to 16 columns); P.V is 16x16x16 bf16 matrix-core steps with
//    P rounded to bf16 and the B operand built in-lane from whole V rows, so
//    no transposition of V is needed.
//
// decode_balanced_kernel (bf16) computes the same with the work spread
// evenly over a grid that fills the GPU once (see its own comment).
#include "common.h"
#include "device_utils.h"

#include <algorithm>
#include <atomic>

namespace pkv {

#ifndef PKV_DECODE_WAVES
#define PKV_DECODE_WAVES 4
#endif
constexpr int kWaves = PKV_DECODE_WAVES;   // wavefronts per decode workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 16;
#ifndef PKV_DECODE_STAGES
#define PKV_DECODE_STAGES 2
#endif
// Tiles in flight per wave in the matrix-core decode (register ring depth).
constexpr int kStages = PKV_DECODE_STAGES;
// The same for E4M3 caches, whose tiles are half as many bytes.
#ifndef PKV_DECODE_STAGES_FP8
#define PKV_DECODE_STAGES_FP8 2
#endif
// Work-balanced decode: resident workgroups per compute unit (= waves per
// SIMD) and tiles in flight per wave.
#ifndef PKV_BAL_WG_PER_CU
#define PKV_BAL_WG_PER_CU 1
#endif
#ifndef PKV_BAL_STAGES
#define PKV_BAL_STAGES 3
#endif
#ifndef PKV_DECODE_WAVES_PER_SIMD
#define PKV_DECODE_WAVES_PER_SIMD 2
#endif

template <typename T>
__device__ __forceinline__ void store_out(void* out, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_out<float>(void* out, int64_t idx, float v) {
  reinterpret_cast<float*>(out)[idx] = v;
}
template <>
__device__ __forceinline__ void store_out<uint16_t>(void* out, int64_t idx, float v) {
  reinterpret_cast<uint16_t*>(out)[idx] = f32_to_bf16_rne(v);
}

// Rows of q-heads g*G .. g*G+G-1 of sequence s set to zero (empty context),
// or to NaN (poisoned).
template <typename T, int D>
__device__ void write_zero_rows(const DecodeParams& p, int s, int g, bool poisoned = false) {
  const int G = p.group;
  const float v = poisoned ? __builtin_nanf("") : 0.f;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    store_out<T>(p.out, ((int64_t)s * p.num_q_heads + g * G + h) * D + d, v);
  }
}

// Relaxed agent-scope atomic accesses of partial results: written through
// to, and read from, the point where all XCDs see the same memory (each XCD
// has its own L2), without a whole-cache write-back or invalidation.
__device__ __forceinline__ void coherent_store(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float coherent_load(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge the per-wave softmax states held in LDS and write the output of a
// sequence's only partition. With several partitions, write this partition's
// (max, sum, unnormalised output) with agent-coherent stores, wait for them
// to complete, and count the partition's arrival on the (sequence, kv-head)
// counter; the workgroup that arrives last merges all partitions
// (log-sum-exp: out = sum_k 2^(m_k - M) o_k / sum_k 2^(m_k - M) l_k) and
// resets the counter. No workgroup waits for another.
//   s_m[w*16 + h], s_l[w*16 + h]: wave w's reference max (log2) and sum
//   s_o[(w*GP + h)*D + d]: wave w's unnormalised output
template <typename T, int D, int GP>
__device__ void merge_and_write(const DecodeParams& p, int s, int g, int part, int n_parts,
                                const float* s_m, const float* s_l, const float* s_o,
                                bool poisoned) {
  const int G = p.group;
  const int64_t head0 = (int64_t)s * p.num_q_heads + g * G;   // first q-head of the group
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    // a shared-prefix partial joins the waves' states as one more term
    const bool pre = p.pre_m != nullptr;
    const float mp = pre ? p.pre_m[head0 + h] : neg_inf();
    float M = mp;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w * 16 + h]);
    float L = 0.f, O = 0.f;
    if (pre && mp != neg_inf()) {
      const float f = fast_exp2(mp - M);
      L = p.pre_l[head0 + h] * f;
      O = p.pre_o[(head0 + h) * D + d] * f;
    }
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = s_m[w * 16 + h];
      const float f = (mw == neg_inf()) ? 0.f : fast_exp2(mw - M);
      L += s_l[w * 16 + h] * f;
      O += s_o[(w * GP + h) * D + d] * f;
    }
    if (poisoned) L = __builtin_nanf("");
    if (n_parts <= 1) {
      // with a shared prefix, a row with no key at all (an empty context) is
      // zero, as the decode without one writes it
      store_out<T>(p.out, (head0 + h) * D + d, (pre && M == neg_inf() && !poisoned) ? 0.f : O / L);
    } else {
      const int64_t base = (head0 + h) * p.num_partitions + part;
      coherent_store(p.ws_o + base * D + d, O);
      if (d == 0) {
        coherent_store(p.ws_m + base, M);
        coherent_store(p.ws_l + base, L);
      }
    }
  }
  if (n_parts <= 1) return;

  __shared__ int s_last;
  // every thread's partial stores have completed before the arrival counts
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int* counter = p.part_counters + (int64_t)s * p.num_kv_heads + g;
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n_parts - 1;
  __syncthreads();
  if (!s_last) return;
  asm volatile("" ::: "memory");
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, d = idx - h * D;
    const int64_t base = (head0 + h) * p.num_partitions;
    float M = neg_inf(), L = 0.f, O = 0.f;
    // eight partitions' loads in flight at a time, then their online merge
    constexpr int kBatch = 8;
    for (int k0 = 0; k0 < n_parts; k0 += kBatch) {
      float mv[kBatch], lv[kBatch], ov[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int64_t k = base + min(k0 + u, n_parts - 1);
        mv[u] = coherent_load(p.ws_m + k);
        lv[u] = coherent_load(p.ws_l + k);
        ov[u] = coherent_load(p.ws_o + k * D + d);
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        if (k0 + u >= n_parts) break;
        if (mv[u] > M) {
          const float f = (M == neg_inf()) ? 0.f : fast_exp2(M - mv[u]);
          L *= f;
          O *= f;
          M = mv[u];
        }
        const float f = (mv[u] == neg_inf()) ? 0.f : fast_exp2(mv[u] - M);
        L += f * lv[u];
        O += f * ov[u];
      }
    }
    store_out<T>(p.out, (head0 + h) * D + d, O / L);
  }
  if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Context length as read from device memory, kept inside [0, max_ctx]: the
// grid, the block-table row and the split-K workspace are sized by the host
// bound, so a longer (invalid) length must not index past them.
__device__ __forceinline__ int clamp_ctx(int ctx, int max_ctx) { return min(max(ctx, 0), max_ctx); }

// Physical block of the tile starting at logical position tok0; an entry
// outside the pool is replaced by block 0 and flags the result as invalid.
__device__ __forceinline__ int64_t tile_row0(const int32_t* bt, int tok0, int bs, int num_blocks,
                                             bool& poisoned) {
  const int lb = tok0 / bs;
  int blk = bt[lb];
  if ((unsigned)blk >= (unsigned)num_blocks) {
    blk = 0;
    poisoned = true;
  }
  return (int64_t)blk * bs + (tok0 - lb * bs);
}

// The sequence's new row in a fused store + decode: stored at `slot` and
// standing for logical position `pos` = ctx-1; `mine` marks the wave of the
// workgroup whose tiles include that position (tile (pos - t0)/16 belongs to
// wave tile % kWaves).
struct NewRow {
  bool mine;
  int slot;
  int pos;
};

__device__ __forceinline__ NewRow new_row_of(const DecodeParams& p, int slot, int ctx, int t0, int t1,
                                             int w) {
  NewRow r{false, -1, ctx - 1};
  if (p.new_slots == nullptr) return r;
  if (slot < 0 || (int64_t)slot >= (int64_t)p.num_blocks * p.block_size) return r;  // padding / outside
  if (r.pos < t0 || r.pos >= t1) return r;                                            // another partition
  r.slot = slot;
  r.mine = ((r.pos - t0) / kTile) % kWaves == w;
  return r;
}

// Work item of a decode workgroup. Items are numbered partition fastest,
// then kv-head, then sequence: i = part + P * (g + Hkv * s). Workgroups go to
// the XCDs round robin (id % 8), each XCD with its own L2.
//  * One partition: item = workgroup id, so with 8 kv-heads each XCD serves
//    one kv-head of every sequence; blocks shared by consecutive sequences
//    are re-read from one L2.
//  * Several partitions: within each run of 8 consecutive items the XCD that
//    takes an item is rotated by the run index, so the partitions of a
//    sequence still spread over all XCDs but no XCD is tied to one partition
//    index (with 2 partitions and mostly short sequences, a fixed mapping
//    would leave half the XCDs nearly idle).
// Returns false for the grid's padding.
// The launchers keep the item count below 2^31, so 32-bit arithmetic holds.
constexpr int kXcds = 8;
__device__ __forceinline__ bool decode_item(const DecodeParams& p, int& g, int& part, int& s) {
  uint32_t item = blockIdx.x;
  const uint32_t np = (uint32_t)p.num_partitions, hkv = (uint32_t)p.num_kv_heads;
  if (np > 1) {
    const uint32_t x = item % kXcds, k = item / kXcds;
    item = k * kXcds + (x + k) % kXcds;
  }
  if (item >= (uint32_t)p.num_seqs * hkv * np) return false;
  const uint32_t r = np > 1 ? item / np : item;
  part = (int)(item - r * np);
  s = (int)(r / hkv);
  g = (int)(r - (uint32_t)s * hkv);
  return true;
}

// Work item by size (single pass; after a shared prefix, sized by the tokens
// past it, see stage_tiles). Two workgroups of this
// kernel fit a compute unit, and with C units workgroup b and workgroup
// b + C are placed on the same one (the dispatcher fills every unit once,
// then again in the same order). Item x = sequence * kv_heads + kv-head;
// its size is the sequence's 16-token tiles.
//  * At most 2C items: workgroup b < C takes item b at once (no ranking on
//    its path). Workgroup C + i, on the unit of item i, takes a second item
//    from x >= C so that the two groups pair in opposite order of size: if
//    item i is the r-th largest of the first C (r from 0), it takes the
//    (C - 1 - r)-th largest of the rest, or none when there are not that
//    many. The grid is then 2C workgroups.
//  * More items: workgroup b < 2C takes the item of rank b < C, or of rank
//    3C - 1 - b (the largest 2C items, each unit pairing a long one with a
//    short one); workgroups past 2C, started as earlier ones finish, take the
//    remaining ranks in order.
// Ranks are by size, largest first, ties by item index (a histogram and a
// selection scan in LDS; all kv-heads of a sequence are adjacent).
constexpr int kRankBuckets = 2048;     // tiles per sequence, capped
constexpr int kRankMaxSeqs = 4096;

// Tiles of every sequence (capped), staged in LDS once per ranking workgroup.
__device__ __forceinline__ void stage_tiles(const DecodeParams& p, uint16_t* tiles) {
  for (int i = threadIdx.x; i < p.num_seqs; i += kThreads) {
    int c = clamp_ctx(p.context_lens[i], p.max_ctx);
    // the shared-prefix decode's own pass reads only the tokens past the prefix
    if (p.seq_prefix != nullptr) c = max(c - p.seq_prefix[i], 0);
    tiles[i] = (uint16_t)min((c + kTile - 1) / kTile, kRankBuckets - 1);
  }
  __syncthreads();
}

// Rank of item i among items 0 .. n-1 (largest first, ties by index).
__device__ __forceinline__ int rank_among(int i, int n, int hkv, const uint16_t* tiles, int* s_sum) {
  const int ti = tiles[i / hkv];
  int cnt = 0;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    const int tj = tiles[j / hkv];
    cnt += (tj > ti || (tj == ti && j < i)) ? 1 : 0;
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) cnt += __shfl_xor(cnt, d, 64);
  if ((threadIdx.x & 63) == 0) s_sum[threadIdx.x >> 6] = cnt;
  __syncthreads();
  int r = 0;
#pragma unroll
  for (int v = 0; v < kWaves; ++v) r += s_sum[v];
  __syncthreads();                        // s_sum is free again
  return r;
}

__device__ __forceinline__ bool sized_item(const DecodeParams& p, int& g, int& s, int* hist, uint16_t* cost,
                                           uint16_t* tiles, int* s_sum) {
  const int hkv = p.num_kv_heads;
  const int n = p.num_seqs * hkv, c = p.pair_span;
  const int b = blockIdx.x;
  int x;
  if (n <= 2 * c) {
    if (b < c) {
      if (b >= n) return false;
      x = b;
    } else {
      const int m = n - c;               // items of the second group
      if (m <= 0) return false;
      stage_tiles(p, tiles);
      const int k = c - 1 - rank_among(b - c, c, hkv, tiles, s_sum);
      if (k >= m) return false;          // workgroup-uniform
      const int j = item_of_rank<kThreads, kRankBuckets>(
          k, m, [&](int i) { return (int)tiles[(c + i) / hkv]; }, hist, cost);
      if (j < 0) return false;
      x = c + j;
    }
  } else {
    const int f = 2 * c;
    const int r = b < c ? b : (b < f ? 3 * c - 1 - b : b);
    if (r >= n) return false;
    stage_tiles(p, tiles);
    const int q = r / hkv;
    const int sq = item_of_rank<kThreads, kRankBuckets>(
        q, p.num_seqs, [&](int i) { return (int)tiles[i]; }, hist, cost);
    if (sq < 0) return false;
    x = sq * hkv + (r - q * hkv);
  }
  s = x / hkv;
  g = x - s * hkv;
  return true;
}

// Work item from a plan (single pass): the same pairing as sized_item with
// the ranks already computed, once per step, by decode_plan_kernel. Workgroup
// b takes rank b < C, or rank 3C - 1 - b for C <= b < 2C (each unit pairs the
// r-th largest item with the (2C - 1 - r)-th), or rank b past 2C. Rank r is
// kv-head r % Hkv of the (r / Hkv)-th largest sequence. The plan entry also
// holds the sequence's length and the block of wave w's first tile, so the
// first K/V loads wait for one load, as in index order.
static_assert(kWaves <= kPlanEntryInts - 2, "plan entry holds one block per wave");
__device__ __forceinline__ bool planned_item(const DecodeParams& p, int w, int& g, int& s, int& ctx_raw,
                                             int& blk0) {
  const int hkv = p.num_kv_heads, n = p.num_seqs * hkv, c = p.pair_span;
  const int b = blockIdx.x;
  const int r = b < c ? b : (b < 2 * c ? 3 * c - 1 - b : b);
  if (r >= n) return false;
  const int q = r / hkv;
  g = r - q * hkv;
  const int32_t* e = p.plan + (int64_t)q * kPlanEntryInts;
  s = e[0];
  ctx_raw = e[1];
  blk0 = e[2 + w];
  return (unsigned)s < (unsigned)p.num_seqs;   // a foreign plan never leads out of bounds
}

// The plan of a single-pass decode step (one workgroup): sequences in order
// of 16-token tiles (capped at kRankBuckets - 1), largest first, ties by
// index. A histogram gives each size's first rank; sequences then take
// their places chunk by chunk, counting equal sizes before them in the chunk.
__global__ __launch_bounds__(kThreads) void decode_plan_kernel(PlanParams p) {
  constexpr int kPer = kRankBuckets / kThreads;   // buckets per thread
  static_assert(kRankBuckets % kThreads == 0, "bucket split");
  __shared__ int s_first[kRankBuckets];   // counts, then the next rank of each size
  __shared__ int s_wave[kWaves];
  __shared__ int s_chunk[kThreads];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  auto bucket = [&](int i) {
    const int c = clamp_ctx(p.context_lens[i], p.max_ctx);
    return min((c + kTile - 1) / kTile, kRankBuckets - 1);
  };
  for (int i = tid; i < kRankBuckets; i += kThreads) s_first[i] = 0;
  __syncthreads();
  for (int i = tid; i < p.num_seqs; i += kThreads) atomicAdd(&s_first[bucket(i)], 1);
  __syncthreads();
  // sequences in this thread's buckets, and in all larger ones (a suffix sum
  // over threads: lanes above within the wave, then the waves above)
  int mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += s_first[kPer * tid + i];
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
  for (int i = kPer - 1; i >= 0; --i) {   // only this thread touches its buckets
    const int cnt = s_first[kPer * tid + i];
    s_first[kPer * tid + i] = above;
    above += cnt;
  }
  __syncthreads();
  for (int base = 0; base < p.num_seqs; base += kThreads) {
    const int i = base + tid;
    const int b = i < p.num_seqs ? bucket(i) : -1;
    s_chunk[tid] = b;
    __syncthreads();
    if (i < p.num_seqs) {
      int tie = 0;
      for (int j = 0; j < tid; ++j) tie += s_chunk[j] == b ? 1 : 0;
      const int r = s_first[b] + tie;
      const int32_t* bt = p.block_tables + (int64_t)i * p.max_blocks;
      int blk[kPlanEntryInts - 2];
#pragma unroll
      for (int v = 0; v < kPlanEntryInts - 2; ++v)
        blk[v] = v < kWaves ? bt[min((v * kTile) / p.block_size, p.max_blocks - 1)] : 0;
      int4* e = reinterpret_cast<int4*>(p.plan + (int64_t)r * kPlanEntryInts);
      e[0] = make_int4(i, p.context_lens[i], blk[0], blk[1]);
      e[1] = make_int4(blk[2], blk[3], blk[4], blk[5]);
    }
    __syncthreads();
    if (i < p.num_seqs) atomicAdd(&s_first[b], 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// Vector-ALU decode
// ---------------------------------------------------------------------------
template <typename T>
struct Widen;
template <>
struct Widen<float> {
  static constexpr int kEPL = 4;
  __device__ static void run(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
};
template <>
struct Widen<uint16_t> {
  static constexpr int kEPL = 8;
  __device__ static void run(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x);
    f[1] = bf16_hi(v.x);
    f[2] = bf16_lo(v.y);
    f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z);
    f[5] = bf16_hi(v.z);
    f[6] = bf16_lo(v.w);
    f[7] = bf16_hi(v.w);
  }
};

template <typename T, int D, int G>
__global__ __launch_bounds__(kThreads) void decode_valu_kernel(DecodeParams p) {
  constexpr int EPL = Widen<T>::kEPL;   // elements per 16-byte lane piece
  constexpr int LPR = D / EPL;          // lanes covering one cache row
  constexpr int RPI = 64 / LPR;         // rows per wave-wide load
  constexpr int LOADS = kTile / RPI;    // loads per 16-token tile
  static_assert(LPR >= 2 && LPR <= 64 && 64 % LPR == 0 && kTile % RPI == 0, "bad shape");

  __shared__ float s_m[kWaves * 16], s_l[kWaves * 16];
  __shared__ float s_o[kWaves * G * D];

  int g, part, s;
  if (!decode_item(p, g, part, s)) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int c = lane % LPR, rg = lane / LPR;
  const int ctx = clamp_ctx(p.context_lens[s], p.max_ctx);
  const int P = p.partition_size;
  const int t0 = part * P;
  if (t0 >= ctx) {
    if (part == 0) write_zero_rows<T, D>(p, s, g);
    return;
  }
  const int n_parts = (ctx + P - 1) / P;
  const int t1 = min(ctx, t0 + P);
  const int n_tiles = (t1 - t0 + kTile - 1) / kTile;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  const int bs = p.block_size;

  float qf[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const T* qrow = reinterpret_cast<const T*>(p.q) + ((int64_t)s * p.num_q_heads + g * G + h) * D;
    Widen<T>::run(load16(qrow + c * EPL), qf[h]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[h][e] *= p.scale_log2;
  }

  const T* kc = reinterpret_cast<const T*>(p.k_cache) + g * D + c * EPL;
  const T* vc = reinterpret_cast<const T*>(p.v_cache) + g * D + c * EPL;
  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;

  float m_ref[G], l_part[G], acc[G][EPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_ref[h] = neg_inf();
    l_part[h] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[h][e] = 0.f;
  }
  bool poisoned = false;

  // Fused store: the sequence's new row (position ctx-1) goes to its slot,
  // and the wave that owns the tile holding ctx-1 uses it from registers.
  const NewRow nr = new_row_of(p, p.new_slots != nullptr ? p.new_slots[s] : -1, ctx, t0, t1, w);
  uint4 nk = make_uint4(0, 0, 0, 0), nv = make_uint4(0, 0, 0, 0);
  if (nr.mine) {
    const int64_t src = ((int64_t)s * p.num_kv_heads + g) * D + c * EPL;
    nk = load16(reinterpret_cast<const T*>(p.k_new) + src);
    nv = load16(reinterpret_cast<const T*>(p.v_new) + src);
    if (rg == 0) {   // the LPR lanes of row group 0 cover the row
      const int64_t dst = (int64_t)nr.slot * row_elems + g * D + c * EPL;
      *reinterpret_cast<uint4*>(const_cast<T*>(reinterpret_cast<const T*>(p.k_cache)) + dst) = nk;
      *reinterpret_cast<uint4*>(const_cast<T*>(reinterpret_cast<const T*>(p.v_cache)) + dst) = nv;
    }
  }

  for (int it = w; it < n_tiles; it += kWaves) {
    const int tok0 = t0 + it * kTile;
    const int64_t row0 = tile_row0(bt, tok0, bs, p.num_blocks, poisoned);
    uint4 kr[LOADS], vr[LOADS];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) kr[i] = load16(kc + (row0 + rg + RPI * i) * row_elems);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) vr[i] = load16(vc + (row0 + rg + RPI * i) * row_elems);
    // in the tile holding the new row, that row comes from registers
    const bool ov = nr.mine && tok0 <= nr.pos && nr.pos < tok0 + kTile;

    float x[LOADS][G];
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      float kf[EPL];
      uint4 kq = kr[i];
      if (ov && tok0 + rg + RPI * i == nr.pos) kq = nk;
      Widen<T>::run(kq, kf);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) a = fmaf(qf[h][e], kf[e], a);
#pragma unroll
        for (int m = 1; m < LPR; m <<= 1) a += shfl_xor_f(a, m);
        x[i][h] = (tok0 + rg + RPI * i < t1) ? a : neg_inf();
      }
    }
    bool grow = false;
    float mt[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float v = x[0][h];
#pragma unroll
      for (int i = 1; i < LOADS; ++i) v = fmaxf(v, x[i][h]);
#pragma unroll
      for (int m = LPR; m < 64; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
      mt[h] = v;
      grow |= v > m_ref[h] + kRescaleThreshold;
    }
    if (__any(grow)) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float m_new = fmaxf(m_ref[h], mt[h]);
        const float alpha = fast_exp2(m_ref[h] - m_new);
        l_part[h] *= alpha;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] *= alpha;
        m_ref[h] = m_new;
      }
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      float vf[EPL];
      uint4 vq = vr[i];
      if (ov && tok0 + rg + RPI * i == nr.pos) vq = nv;
      Widen<T>::run(vq, vf);
      const bool live = tok0 + rg + RPI * i < t1;
#pragma unroll
      for (int e = 0; e < EPL; ++e) vf[e] = live ? vf[e] : 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pr = fast_exp2(x[i][h] - m_ref[h]);
        l_part[h] += pr;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[h][e] = fmaf(pr, vf[e], acc[h][e]);
      }
    }
  }

  // fold the row groups of the wave together
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1) {
      l_part[h] += shfl_xor_f(l_part[h], m);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[h][e] += shfl_xor_f(acc[h][e], m);
    }
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[(w * G + h) * D + c * EPL + e] = acc[h][e];
    }
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      s_m[w * 16 + h] = m_ref[h];
      s_l[w * 16 + h] = l_part[h];
    }
  }
  poisoned = __any(poisoned);
  __shared__ int s_poison;
  if (threadIdx.x == 0) s_poison = 0;
  __syncthreads();
  if (poisoned && lane == 0) s_poison = 1;
  __syncthreads();
  merge_and_write<T, D, G>(p, s, g, part, n_parts, s_m, s_l, s_o, s_poison != 0);
}

// ---------------------------------------------------------------------------
// Matrix-core decode (bf16)
// ---------------------------------------------------------------------------
// Per wave: tiles w, w+4, w+8, ... of the partition. Loads run kStages-1
// tiles ahead of the math in a ring of register buffers, and each tile's
// physical block id comes from a scalar load issued kStages tiles ahead. The
// prefetch is unconditional (past the wave's last tile it re-reads that tile,
// an L2 hit) so that the wait before a tile's math covers only its own loads.
//
// q.k: 16x16x32 bf16 MFMA, A = the tile's 16 K rows, B = q^T with the G heads
// as columns (padded to 16). Its output gives lane l the scores of tokens
// 4*(l/16)+r, r=0..3, for head l%16 -- exactly the A operand (P, heads as
// rows, 4 tokens per lane) of the 16x16x16 bf16 MFMA used for P.V. For the
// B operand (4 consecutive tokens of one column per lane) each 16-lane group
// reads its 4 V rows whole (lane n holds columns EPL*n .. EPL*n+EPL-1 of all
// 4 tokens), so step i of P.V takes column EPL*n+i of the 4 rows with two
// in-lane byte permutes: no lane exchange, and every V load reads full rows.
//
// E4M3 caches (FP8): a lane holds the D/4 contiguous bytes [qg*D/4, +D/4) of
// its K row, so step c of q.k pairs elements qg*D/4 + 8c .. +7 (q is loaded
// in the same order), and EPL bytes of each of its 4 V rows. Codes become
// bf16 at the point of use (exact: every E4M3 value is a bf16 value); the K
// scale joins the logit multiplier and the V scale the accumulator.
template <int D, bool FP8>
struct MfmaTile;
template <int D>
struct MfmaTile<D, false> {
  static constexpr int KCH = D / 32;   // 16-byte K pieces per lane
  static constexpr int EPL = D / 16;   // V columns per lane
  uint4 k[KCH];
  uint4 v[4];                          // rows 4*qg + 0..3 (EPL bf16 each, rest unused)
};
template <int D>
struct MfmaTile<D, true> {
  static constexpr int KCH = D / 32;
  static constexpr int EPL = D / 16;
  uint4 k[D / 64];                     // D/4 bytes of the K row
  uint2 v[4];                          // EPL bytes of each V row (D = 64: .x only)
};

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

#ifndef PKV_DECODE_WAVES_PER_SIMD_FP8
#define PKV_DECODE_WAVES_PER_SIMD_FP8 2
#endif
template <bool FP8>
constexpr int kMfmaWavesPerSimd = FP8 ? PKV_DECODE_WAVES_PER_SIMD_FP8 : PKV_DECODE_WAVES_PER_SIMD;

template <int D, int GP, bool FP8>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kMfmaWavesPerSimd<FP8>, kMfmaWavesPerSimd<FP8>)))
void decode_mfma_kernel(DecodeParams p) {
  using Tile = MfmaTile<D, FP8>;
  constexpr int kStages = FP8 ? PKV_DECODE_STAGES_FP8 : ::pkv::kStages;
  constexpr int KCH = Tile::KCH;
  constexpr int EPL = Tile::EPL;   // also the number of 16x16x16 P.V steps

  __shared__ float s_m[kWaves * 16], s_l[kWaves * 16];
  __shared__ float s_o[kWaves * GP * D];
  __shared__ int s_poison;
  __shared__ int s_rank_hist[kRankBuckets];
  __shared__ uint16_t s_rank_cost[kRankMaxSeqs];
  __shared__ uint16_t s_rank_tiles[kRankMaxSeqs];
  __shared__ int s_rank_sum[kWaves];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int g, part = 0, s;
  int plan_ctx = 0, plan_blk = 0;
  const bool planned = p.plan != nullptr;
  if (planned) {
    if (!planned_item(p, w, g, s, plan_ctx, plan_blk)) return;
  } else if (p.pair_span > 0) {
    if (!sized_item(p, g, s, s_rank_hist, s_rank_cost, s_rank_tiles, s_rank_sum)) return;
  } else if (!decode_item(p, g, part, s)) {
    return;
  }
  const int n = lane & 15, qg = lane >> 4;
  const int G = p.group;
  const int P = p.partition_size;
  const int bs = p.block_size;
  const int32_t* bt = p.block_tables + (int64_t)s * p.max_blocks;

  // The loads that depend only on the work item are issued together, before
  // any of them is waited for: the context length, the new row's slot and
  // pieces (fused store), the shared prefix, the q rows, and the block of
  // the wave's first tile as it is without a shared prefix (index kept
  // inside the table row; used only when it is the right entry).
  // With several partitions most workgroups of short sequences have nothing
  // to do; those leave before loading anything else.
  // With a plan, the length and the first block come from it; the kernel
  // still reads both from context_lens and the table, off the path of the
  // first loads, and poisons the row if the plan does not match them.
  const int ctx_raw = planned ? plan_ctx : p.context_lens[s];
  if (p.num_partitions > 1 && p.seq_prefix == nullptr && part * P >= clamp_ctx(ctx_raw, p.max_ctx)) {
    if (part == 0) write_zero_rows<uint16_t, D>(p, s, g);
    return;
  }
  const int slot_raw = p.new_slots != nullptr ? p.new_slots[s] : -1;
  const int prefix_raw = p.seq_prefix != nullptr ? p.seq_prefix[s] : 0;
  const int blk_idx = min((part * P + w * kTile) / bs, p.max_blocks - 1);
  const int blk_first = planned ? plan_blk : bt[blk_idx];
  const int ctx_check = planned ? p.context_lens[s] : 0;
  const int blk_check = planned ? bt[blk_idx] : 0;

  // B operand of q.k^T: column n is q-head g*G+n (zero past the group). In
  // step c, lane group qg holds head_dim elements [32c + 8qg, 32c + 8qg + 8),
  // so the four lanes of a K row read 64 contiguous bytes per load. The K
  // operand uses the same element order, so the contraction pairs matching
  // elements whatever order the hardware sums them in.
  // (E4M3 caches: elements qg*D/4 + 8c .. +7 instead, see MfmaTile.)
  bf16x8_t qb[KCH];
  {
    const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) +
                           ((int64_t)s * p.num_q_heads + g * G + n) * D + (FP8 ? qg * (D / 4) : 8 * qg);
#pragma unroll
    for (int j = 0; j < KCH; ++j) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (n < G) v = load16(qrow + (FP8 ? 8 : 32) * j);
      qb[j] = bit_cast_to<bf16x8_t>(v);
    }
  }
  // The new row's pieces as this lane uses them (bf16), loaded whether or
  // not this wave turns out to hold the new row's position.
  constexpr int kNewK = FP8 ? 2 * (D / 64) : KCH;
  uint4 nkr[kNewK], nvr = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int c = 0; c < kNewK; ++c) nkr[c] = make_uint4(0, 0, 0, 0);
  if (p.new_slots != nullptr) {
    const uint16_t* kn = reinterpret_cast<const uint16_t*>(p.k_new) + ((int64_t)s * p.num_kv_heads + g) * D;
    const uint16_t* vn = reinterpret_cast<const uint16_t*>(p.v_new) + ((int64_t)s * p.num_kv_heads + g) * D;
#pragma unroll
    for (int c = 0; c < kNewK; ++c) nkr[c] = load16(kn + (FP8 ? qg * (D / 4) + 8 * c : 8 * qg + 32 * c));
    if constexpr (EPL == 8) {
      nvr = load16(vn + EPL * n);
    } else {
      const uint2 h = load8(vn + EPL * n);
      nvr = make_uint4(h.x, h.y, 0, 0);
    }
  }

  const int ctx = clamp_ctx(ctx_raw, p.max_ctx);
  // Shared-prefix second pass: the tokens before `start` are covered by the
  // first pass's partials (a prefix that is not a multiple of 16 or exceeds
  // the context breaks the contract: the row is poisoned and no token read).
  int start = 0;
  bool bad_prefix = false;
  if (p.seq_prefix != nullptr) {
    start = prefix_raw;
    if (start < 0 || start > ctx || (start & (kTile - 1)) != 0) {
      bad_prefix = true;
      start = ctx;
    }
  }
  const int t0 = start + part * P;
  if (t0 >= ctx && p.pre_m == nullptr) {
    if (part == 0) write_zero_rows<uint16_t, D>(p, s, g, planned && ctx_check != ctx_raw);
    return;
  }
  const int n_parts = (ctx + P - 1) / P;
  const int t1 = min(ctx, t0 + P);
  const int n_tiles = (t1 - t0 + kTile - 1) / kTile;
  const int my_tiles = w < n_tiles ? (n_tiles - w + kWaves - 1) / kWaves : 0;
  const int64_t row_elems = (int64_t)p.num_kv_heads * D;
  // logit multiplier (with the K scale for E4M3 caches) and V scale
  const float logit_scale = FP8 ? p.scale_log2 * p.k_scale[g] : p.scale_log2;

  constexpr int kElt = FP8 ? 1 : 2;   // bytes per cache element
  const char* kc = reinterpret_cast<const char*>(p.k_cache) + (g * D + (FP8 ? qg * (D / 4) : 8 * qg)) * kElt;
  // V: lane reads rows 4*qg + st (st = 0..3), columns EPL*n .. EPL*n+EPL-1
  const char* vc = reinterpret_cast<const char*>(p.v_cache) + (g * D + EPL * n) * kElt;

  float m_ref = neg_inf();   // reference max of head n (replicated over qg)
  float l_part = 0.f;        // sum over this lane's tokens for head n
  f32x4_t acc[EPL];          // acc[i][r] = O[head 4*qg + r][EPL*n + i]
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  bool bad = false;

  // Fused store: the sequence's new row (position ctx-1) goes to its slot,
  // and the wave that owns the tile holding ctx-1 uses it from registers.
  // E4M3 caches: the new row is quantised here exactly as the store kernel
  // does, and its codes stand in for the cache's.
  // (bf16 caches use nkr / nvr as they are.)
  const NewRow nr = new_row_of(p, slot_raw, ctx, t0, t1, w);
  uint4 nk8[D / 64];                               // E4M3: codes of elements qg*D/4 ..
  uint2 nv8 = make_uint2(0u, 0u);                  // E4M3: codes of columns EPL*n ..
#pragma unroll
  for (int c = 0; c < D / 64; ++c) nk8[c] = make_uint4(0, 0, 0, 0);
  if (FP8 && nr.mine) {
    const float ks = p.k_scale[g], vs = p.v_scale[g];
#pragma unroll
    for (int c = 0; c < D / 64; ++c) {
      const uint2 a = quantize8_bf16(nkr[2 * c], ks);
      const uint2 b = quantize8_bf16(nkr[2 * c + 1], ks);
      nk8[c] = make_uint4(a.x, a.y, b.x, b.y);
    }
    if constexpr (EPL == 8) {
      nv8 = quantize8_bf16(nvr, vs);
    } else {
      const float x[4] = {bf16_lo(nvr.x), bf16_hi(nvr.x), bf16_lo(nvr.y), bf16_hi(nvr.y)};
      nv8 = make_uint2(quantize4(x, vs), 0u);
    }
  }

  // Logical position of the first token of the wave's j-th tile (j clamped
  // to the wave's last tile) and its physical block.
  auto tile_tok0 = [&](int j) { return t0 + (w + kWaves * min(j, my_tiles - 1)) * kTile; };
  auto block_of = [&](int j) { return bt[tile_tok0(j) / bs]; };

  // Issue the loads of the wave's j-th tile, whose physical block is blk (an
  // id outside the pool reads block 0 and poisons the result).
  auto issue = [&](int j, int blk, Tile& t) {
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      blk = 0;
      bad = true;
    }
    const int tok0 = tile_tok0(j);
    const int64_t row0 = (int64_t)blk * bs + (tok0 % bs);
    const int64_t row_bytes = row_elems * kElt;
    const char* kp = kc + (row0 + n) * row_bytes;
    const char* vp = vc + (row0 + 4 * qg) * row_bytes;
    if constexpr (FP8) {
#pragma unroll
      for (int c = 0; c < D / 64; ++c) t.k[c] = load16(kp + 16 * c);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if constexpr (EPL == 8) t.v[st] = load8(vp + st * row_bytes);
        else t.v[st] = make_uint2(*reinterpret_cast<const uint32_t*>(vp + st * row_bytes), 0u);
      }
    } else {
#pragma unroll
      for (int c = 0; c < KCH; ++c) t.k[c] = load16(kp + 64 * c);
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        if constexpr (EPL == 8) {
          t.v[st] = load16(vp + st * row_bytes);
        } else {
          const uint2 h = load8(vp + st * row_bytes);
          t.v[st] = make_uint4(h.x, h.y, 0, 0);
        }
      }
    }
  };

  // Scores, online softmax and P.V of the wave's j-th tile.
  auto compute = [&](int j, const Tile& t) {
    const int tok0 = tile_tok0(j);
    // in the tile holding the new row, that row comes from registers
    const bool ov = nr.mine && tok0 <= nr.pos && nr.pos < tok0 + kTile;
    const int rn = nr.pos - tok0;
    // S[token 4*qg + r][head n] in sc[r]
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KCH; ++c) {
      uint4 kq;
      if constexpr (FP8) {
        uint32_t w0 = word_of(t.k[(2 * c) / 4], (2 * c) % 4);
        uint32_t w1 = word_of(t.k[(2 * c + 1) / 4], (2 * c + 1) % 4);
        if (ov && n == rn) {
          w0 = word_of(nk8[(2 * c) / 4], (2 * c) % 4);
          w1 = word_of(nk8[(2 * c + 1) / 4], (2 * c + 1) % 4);
        }
        const uint2 lo = e4m3x4_to_bf16(w0);
        const uint2 hi = e4m3x4_to_bf16(w1);
        kq = make_uint4(lo.x, lo.y, hi.x, hi.y);
      } else {
        kq = t.k[c];
        if (ov && n == rn) kq = nkr[c];
      }
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast_to<bf16x8_t>(kq), qb[c], sc, 0, 0, 0);
    }

    const int tokq = tok0 + 4 * qg;
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (tokq + r < t1) ? sc[r] * logit_scale : neg_inf();
    // max over the tile's 16 tokens: the lane's four, then across the lane
    // groups qg (row swaps, no LDS round trip); NaN-propagating. A head's
    // maximum clears the threshold exactly when one of its four lanes'
    // maxima does, so the reduction across lanes runs only when a
    // reference rises.
    const float lane_max = __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]),
                                                         __builtin_elementwise_maximum(x[2], x[3]));
    if (__any(lane_max > m_ref + kRescaleThreshold)) {
      const float mt = max_across_rows(lane_max);
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float a = __shfl(alpha, 4 * qg + r, 64);   // factor of head 4*qg + r
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e][r] *= a;
      }
      m_ref = m_new;
    }
    // P in bf16 (rounded to nearest even); the sum uses the rounded weights
    // so numerator and denominator see the same values.
    uint32_t pw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pw[h] = pack_bf16x2(fast_exp2(x[2 * h] - m_ref), fast_exp2(x[2 * h + 1] - m_ref));
      l_part += bf16_lo(pw[h]) + bf16_hi(pw[h]);
    }
    const short4_t pa = __builtin_bit_cast(short4_t, make_uint2(pw[0], pw[1]));

    // V rows past the context may hold anything (NaN included): zero them
    // before they meet a zero weight (only the last tile can be partial).
    uint32_t vd[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if constexpr (FP8) {
        uint2 c8 = t.v[st];
        if (ov && 4 * qg + st == rn) c8 = nv8;
        const uint2 a = e4m3x4_to_bf16(c8.x);
        const uint2 b = EPL == 8 ? e4m3x4_to_bf16(c8.y) : make_uint2(0u, 0u);
        vd[st][0] = a.x;
        vd[st][1] = a.y;
        vd[st][2] = b.x;
        vd[st][3] = b.y;
      } else {
        uint4 v = t.v[st];
        if (ov && 4 * qg + st == rn) v = nvr;
        vd[st][0] = v.x;
        vd[st][1] = v.y;
        vd[st][2] = v.z;
        vd[st][3] = v.w;
      }
    }
    if (tok0 + kTile > t1) {
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bool live = tokq + st < t1;
#pragma unroll
        for (int i = 0; i < 4; ++i) vd[st][i] = live ? vd[st][i] : 0u;
      }
    }
    // step i: B column n = V[tokens 4*qg + 0..3][EPL*n + i]
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b0 = __builtin_amdgcn_perm(vd[1][i / 2], vd[0][i / 2], sel);
      const uint32_t b1 = __builtin_amdgcn_perm(vd[3][i / 2], vd[2][i / 2], sel);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(
          pa, __builtin_bit_cast(short4_t, make_uint2(b0, b1)), acc[i], 0, 0, 0);
    }
  };

  if (my_tiles > 0) {
    // kStages register buffers in a ring; the loop is unrolled by the ring
    // size so every buffer index is a compile-time constant and no register
    // copy (which would wait on its pending load) is needed.
    Tile buf[kStages];
    int blk_ahead = start == 0 ? blk_first : block_of(0);
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) {
      const int b = blk_ahead;
      blk_ahead = block_of(i + 1);
      issue(i, b, buf[i]);
    }
    for (int j = 0; j < my_tiles; j += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        const int b = blk_ahead;
        blk_ahead = block_of(j + u + kStages);
        issue(j + u + kStages - 1, b, buf[(u + kStages - 1) % kStages]);
        if (j + u < my_tiles) compute(j + u, buf[u]);
      }
    }
  }

  // The new row goes to its cache slot after the loop, so that no store is
  // in flight while the loop's loads are being waited for.
  if (FP8 && nr.mine) {
    uint8_t* kd = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.k_cache)) +
                  (int64_t)nr.slot * row_elems + g * D;
    uint8_t* vd = const_cast<uint8_t*>(reinterpret_cast<const uint8_t*>(p.v_cache)) +
                  (int64_t)nr.slot * row_elems + g * D;
    if (n == 0) {   // lanes n == 0 (qg = 0..3) hold the codes of the whole K row
#pragma unroll
      for (int c = 0; c < D / 64; ++c) *reinterpret_cast<uint4*>(kd + qg * (D / 4) + 16 * c) = nk8[c];
    }
    if (qg == 0) {  // lanes qg == 0 (n = 0..15) hold the codes of all V columns
      if constexpr (EPL == 8) {
        *reinterpret_cast<uint2*>(vd + EPL * n) = nv8;
      } else {
        *reinterpret_cast<uint32_t*>(vd + EPL * n) = nv8.x;
      }
    }
  } else if (nr.mine) {
    uint16_t* kd = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(p.k_cache)) +
                   (int64_t)nr.slot * row_elems + g * D;
    uint16_t* vd = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(p.v_cache)) +
                   (int64_t)nr.slot * row_elems + g * D;
    if (n == 0) {   // lanes n == 0 (qg = 0..3) hold all K pieces of the row
#pragma unroll
      for (int c = 0; c < KCH; ++c) *reinterpret_cast<uint4*>(kd + 8 * qg + 32 * c) = nkr[c];
    }
    if (qg == 0) {  // lanes qg == 0 (n = 0..15) hold all V columns
      if constexpr (EPL == 8) {
        *reinterpret_cast<uint4*>(vd + EPL * n) = nvr;
      } else {
        *reinterpret_cast<uint2*>(vd + EPL * n) = make_uint2(nvr.x, nvr.y);
      }
    }
  }

  l_part += shfl_xor_f(l_part, 16);
  l_part += shfl_xor_f(l_part, 32);
  if (lane < 16) {
    s_m[w * 16 + lane] = m_ref;
    s_l[w * 16 + lane] = l_part;
  }
  const float v_scale = FP8 ? p.v_scale[g] : 1.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * qg + r;
    if (h < G) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_o[(w * GP + h) * D + EPL * n + e] = acc[e][r] * v_scale;
    }
  }
  const bool stale = planned && (ctx_check != ctx_raw || (my_tiles > 0 && blk_check != blk_first));
  const bool poisoned = __any(bad) || bad_prefix || stale;
  if (threadIdx.x == 0) s_poison = 0;
  __syncthreads();
  if (poisoned && lane == 0) s_poison = 1;
  __syncthreads();
  merge_and_write<uint16_t, D, GP>(p, s, g, part, n_parts, s_m, s_l, s_o, s_poison != 0);
}

// ---------------------------------------------------------------------------
// Work-balanced matrix-core decode (bf16)
// ---------------------------------------------------------------------------
// The batch's 16-token tiles form one list, kv-head slowest, then sequence,
// then tile: kv-head g's tiles are a contiguous run of C = sum_s ceil(ctx_s/16)
// tiles. A grid sized to fill the GPU once gives every wave an equal,
// contiguous share of the list, so waves finish together however unequal the
// context lengths are. A wave walks its share with the register ring of the
// per-item kernel, switching sequence and kv-head as it crosses items (each
// ring slot carries its own q rows). An item that lies wholly inside one
// share is finished by that wave. An item cut by share boundaries leaves one
// piece (max, sum, unnormalised output) per wave that touched it; the wave
// that completes its piece last, as counted by an arrival counter (one per
// wave index: that of the item's first wave), merges the pieces and writes
// the output. No wave ever waits for another.
// Waves are numbered contiguously per XCD (workgroups go to the 8 XCDs round
// robin), so each XCD walks a contiguous part of the list: with 8 kv-heads,
// one kv-head per XCD, and blocks shared between sequences are re-read from
// one L2.
namespace {
constexpr int kBalThreads = 64 * kBalWavesPerWorkgroup;
constexpr int kBalMinShare = 4;         // fewest tiles a wave is given
constexpr int kInfoRows = 31;           // tile descriptor: live rows (1..16)
constexpr int kInfoLast = 1 << 5;       //   last tile of its item
constexpr int kInfoNewRow = 1 << 6;     //   its last row comes from the new K/V rows
constexpr int kInfoBad = 1 << 7;        //   block id outside the pool

template <int D>
struct BalSlot {
  uint4 k[D / 32];
  uint4 v[4];
  uint4 q[D / 32];
  int s, g, t, info;
};
}  // namespace

template <int D>
__global__ __launch_bounds__(kBalThreads) __attribute__((amdgpu_waves_per_eu(PKV_BAL_WG_PER_CU, PKV_BAL_WG_PER_CU)))
void decode_balanced_kernel(DecodeParams p) {
  constexpr int kStages = PKV_BAL_STAGES;
  constexpr int KCH = D / 32;
  constexpr int EPL = D / 16;
  __shared__ int s_cum[kBalMaxSeqs + 1];     // tiles of sequences before s
  __shared__ uint8_t s_last[kBalMaxSeqs];    // rows in a sequence's last tile
  __shared__ int s_wsum[kBalWavesPerWorkgroup];

  const int S = p.num_seqs, Hkv = p.num_kv_heads, Hq = p.num_q_heads, G = p.group;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15, qg = lane >> 4;
  const int bs = p.block_size;
  const int64_t row_elems = (int64_t)Hkv * D;
  const int64_t num_slots = (int64_t)p.num_blocks * bs;

  // Wave position in the list order: XCD-contiguous.
  const int nwg = gridDim.x;   // a multiple of kXcds
  const int pos = ((int)(blockIdx.x % kXcds) * (nwg / kXcds) + (int)(blockIdx.x / kXcds)) *
                      kBalWavesPerWorkgroup + w;
  const int NW = nwg * kBalWavesPerWorkgroup;

  // New rows of the fused store: kRowLanes lanes move one item's K and V
  // rows, 16 bytes each; the first pass is loaded now and stored at the end.
  constexpr int kRowLanes = D / 4;              // 16-byte pieces of a K row and a V row
  constexpr int kRowsPerPass = 64 / kRowLanes;
  const int row_sub = lane % kRowLanes;
  const bool row_is_v = row_sub >= kRowLanes / 2;
  const int row_piece = row_sub % (kRowLanes / 2);
  int new_item = pos * kRowsPerPass + lane / kRowLanes;
  int new_slot = -1;
  uint4 new_data = make_uint4(0, 0, 0, 0);
  auto load_new_row = [&](int item) {
    const int s = item / Hkv, g = item - (item / Hkv) * Hkv;
    const int64_t off = ((int64_t)s * Hkv + g) * D + 8 * row_piece;
    new_data = load16(reinterpret_cast<const uint16_t*>(row_is_v ? p.v_new : p.k_new) + off);
    new_slot = p.new_slots[s];
  };
  auto store_new_row = [&](int item) {
    const int s = item / Hkv, g = item - (item / Hkv) * Hkv;
    // a sequence with an empty context has no new row in it
    if (new_slot < 0 || new_slot >= num_slots || s_cum[s + 1] == s_cum[s]) return;
    uint16_t* dst = const_cast<uint16_t*>(reinterpret_cast<const uint16_t*>(row_is_v ? p.v_cache : p.k_cache)) +
                    (int64_t)new_slot * row_elems + g * D + 8 * row_piece;
    *reinterpret_cast<uint4*>(dst) = new_data;
  };
  const bool fused = p.new_slots != nullptr;
  if (fused && new_item < S * Hkv) load_new_row(new_item);

  // ---- tiles per sequence and their exclusive prefix sums ------------------
  for (int i = tid; i < S; i += kBalThreads) {
    const int c = clamp_ctx(p.context_lens[i], p.max_ctx);
    const int nt = (c + kTile - 1) / kTile;
    s_cum[i] = nt;
    s_last[i] = (uint8_t)(nt > 0 ? c - (nt - 1) * kTile : 0);
  }
  __syncthreads();
  {
    const int per = (S + kBalThreads - 1) / kBalThreads;
    const int lo = min(tid * per, S), hi = min(lo + per, S);
    int run = 0;
    for (int i = lo; i < hi; ++i) run += s_cum[i];
    int incl = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    if (lane == 63) s_wsum[w] = incl;
    __syncthreads();
    int base = incl - run;
    for (int i = 0; i < w; ++i) base += s_wsum[i];
    for (int i = lo; i < hi; ++i) {
      const int nt = s_cum[i];
      s_cum[i] = base;
      base += nt;
    }
    if (tid == kBalThreads - 1) s_cum[S] = base;   // the last thread's running sum is the total
    __syncthreads();
  }
  const int C = s_cum[S];          // tiles per kv-head
  const int T = C * Hkv;           // the host bounds this below 2^30
  const int share = max((T + NW - 1) / NW, kBalMinShare);
  const int a = min(pos * share, T);
  const int cnt = min(T - a, share);

  // ---- tile descriptors: lane l describes tile `base + l` of the share -----
  int d_s = 0, d_g = 0, d_t = 0, d_info = 0, d_blk = 0;
  auto describe = [&](int base) {
    const int x = a + min(base + lane, cnt - 1);
    const int g = x / C;
    const int r = x - g * C;
    int lo = 0, hi = S - 1;   // last sequence whose first tile is <= r (never an empty one)
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_cum[mid] <= r) lo = mid;
      else hi = mid - 1;
    }
    const int s = lo, t = r - s_cum[s];
    const bool last = t == s_cum[s + 1] - s_cum[s] - 1;
    int info = last ? (int)s_last[s] | kInfoLast : kTile;
    if (last && fused) {
      const int slot = p.new_slots[s];
      if (slot >= 0 && slot < num_slots) info |= kInfoNewRow;
    }
    d_blk = p.block_tables[(int64_t)s * p.max_blocks + (t * kTile) / bs];
    d_s = s;
    d_g = g;
    d_t = t;
    d_info = info;
  };

  const uint16_t* kc = reinterpret_cast<const uint16_t*>(p.k_cache);
  const uint16_t* vc = reinterpret_cast<const uint16_t*>(p.v_cache);
  const uint16_t* qbase = reinterpret_cast<const uint16_t*>(p.q);
  const int head_in_group = n % G;   // padding columns repeat a real head (finite, never written)

  // Loads of the share's j-th tile (j clamped to the last one) into a slot.
  auto issue = [&](int j, BalSlot<D>& sl) {
    if (j < cnt && j > 0 && (j & 63) == 0) describe(j);
    const int idx = min(j, cnt - 1) & 63;
    const int s = __builtin_amdgcn_readlane(d_s, idx);
    const int g = __builtin_amdgcn_readlane(d_g, idx);
    const int t = __builtin_amdgcn_readlane(d_t, idx);
    int info = __builtin_amdgcn_readlane(d_info, idx);
    int blk = __builtin_amdgcn_readlane(d_blk, idx);
    if ((unsigned)blk >= (unsigned)p.num_blocks) {
      blk = 0;
      info |= kInfoBad;
    }
    sl.s = s;
    sl.g = g;
    sl.t = t;
    sl.info = info;
    const int64_t row0 = (int64_t)blk * bs + (t * kTile) % bs;
    const uint16_t* kp = kc + (row0 + n) * row_elems + g * D + 8 * qg;
    const uint16_t* vp = vc + (row0 + 4 * qg) * row_elems + g * D + EPL * n;
    // the tile's last row is the new token: read it from the new rows
    const int rn = (info & kInfoRows) - 1;
    const bool ovr = (info & kInfoNewRow) != 0;
    const int64_t nrow = ((int64_t)s * Hkv + g) * D;
    if (ovr && n == rn) kp = reinterpret_cast<const uint16_t*>(p.k_new) + nrow + 8 * qg;
    const uint16_t* qp = qbase + ((int64_t)s * Hq + g * G + head_in_group) * D + 8 * qg;
#pragma unroll
    for (int c = 0; c < KCH; ++c) sl.k[c] = load16(kp + 32 * c);
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const uint16_t* src = (ovr && 4 * qg + st == rn)
                                ? reinterpret_cast<const uint16_t*>(p.v_new) + nrow + EPL * n
                                : vp + st * row_elems;
      if constexpr (EPL == 8) {
        sl.v[st] = load16(src);
      } else {
        const uint2 h = load8(src);
        sl.v[st] = make_uint4(h.x, h.y, 0, 0);
      }
    }
#pragma unroll
    for (int c = 0; c < KCH; ++c) sl.q[c] = load16(qp + 32 * c);
  };

  // softmax state of the current item
  float m_ref = neg_inf(), l_part = 0.f;
  f32x4_t acc[EPL];
  bool item_bad = false, seg_full = false, seg_first = true;
  // items this wave left a piece of (at most its first and its last)
  int pend_s0 = 0, pend_g0 = 0, pend_s1 = 0, pend_g1 = 0, npend = 0;
  float* pieces = p.bal_pieces;
  const int stride = p.bal_piece_stride;

  auto flush = [&](int s, int g, bool complete) {
    float l_tot = l_part;
    l_tot += shfl_xor_f(l_tot, 16);
    l_tot += shfl_xor_f(l_tot, 32);
    if (complete) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * qg + r;
        const float l = __shfl(l_tot, h, 64);
        const float inv = item_bad ? __builtin_nanf("") : 1.f / l;
        if (h < G) {
          uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)s * Hq + g * G + h) * D + EPL * n;
          if constexpr (EPL == 8) {
            uint32_t pk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) pk[e] = pack_bf16x2(acc[2 * e][r] * inv, acc[2 * e + 1][r] * inv);
            *reinterpret_cast<uint4*>(o) = make_uint4(pk[0], pk[1], pk[2], pk[3]);
          } else {
            *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(acc[0][r] * inv, acc[1][r] * inv),
                                                     pack_bf16x2(acc[2][r] * inv, acc[3][r] * inv));
          }
        }
      }
    } else {
      // agent-coherent stores: complete means visible to every XCD
      float* pc = pieces + (int64_t)(2 * pos + (seg_first ? 0 : 1)) * stride;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 4 * qg + r;
        if (h < G) {
          float* o = pc + h * D + EPL * n;
#pragma unroll
          for (int e = 0; e < EPL; ++e) coherent_store(o + e, acc[e][r]);
        }
      }
      if (qg == 0 && n < G) {
        coherent_store(pc + G * D + n, m_ref);
        coherent_store(pc + G * D + G + n, item_bad ? __builtin_nanf("") : l_tot);
      }
      if (npend == 0) {
        pend_s0 = s;
        pend_g0 = g;
      } else {
        pend_s1 = s;
        pend_g1 = g;
      }
      ++npend;
    }
    seg_first = false;
  };

  // Scores, online softmax and P.V of one tile (the same arithmetic as the
  // per-item kernel), then the end-of-item bookkeeping.
  auto compute = [&](int j, const BalSlot<D>& sl) {
    const int info = sl.info;
    if (j == 0 || sl.t == 0) {
      m_ref = neg_inf();
      l_part = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[e] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      item_bad = false;
      seg_full = sl.t == 0;
    }
    item_bad |= (info & kInfoBad) != 0;
    const int valid = info & kInfoRows;
    f32x4_t sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < KCH; ++c)
      sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bit_cast_to<bf16x8_t>(sl.k[c]), bit_cast_to<bf16x8_t>(sl.q[c]),
                                                   sc, 0, 0, 0);
    float x[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] = (4 * qg + r < valid) ? sc[r] * p.scale_log2 : neg_inf();
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = fmaxf(mt, shfl_xor_f(mt, 16));
    mt = fmaxf(mt, shfl_xor_f(mt, 32));
    if (__any(mt > m_ref + kRescaleThreshold)) {
      const float m_new = fmaxf(m_ref, mt);
      const float alpha = fast_exp2(m_ref - m_new);
      l_part *= alpha;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float f = __shfl(alpha, 4 * qg + r, 64);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e][r] *= f;
      }
      m_ref = m_new;
    }
    uint32_t pw[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pw[h] = pack_bf16x2(fast_exp2(x[2 * h] - m_ref), fast_exp2(x[2 * h + 1] - m_ref));
      l_part += bf16_lo(pw[h]) + bf16_hi(pw[h]);
    }
    const short4_t pa = __builtin_bit_cast(short4_t, make_uint2(pw[0], pw[1]));
    uint32_t vd[4][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const bool live = 4 * qg + st < valid;   // rows past the context may hold anything
      vd[st][0] = live ? sl.v[st].x : 0u;
      vd[st][1] = live ? sl.v[st].y : 0u;
      vd[st][2] = live ? sl.v[st].z : 0u;
      vd[st][3] = live ? sl.v[st].w : 0u;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      const uint32_t sel = (i & 1) ? 0x07060302u : 0x05040100u;
      const uint32_t b0 = __builtin_amdgcn_perm(vd[1][i / 2], vd[0][i / 2], sel);
      const uint32_t b1 = __builtin_amdgcn_perm(vd[3][i / 2], vd[2][i / 2], sel);
      acc[i] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(short4_t, make_uint2(b0, b1)),
                                                         acc[i], 0, 0, 0);
    }
    if ((info & kInfoLast) || j == cnt - 1) flush(sl.s, sl.g, seg_full && (info & kInfoLast));
  };

  if (cnt > 0) {
    describe(0);
    BalSlot<D> buf[kStages];
#pragma unroll
    for (int i = 0; i < kStages - 1; ++i) issue(i, buf[i]);
    for (int j = 0; j < cnt; j += kStages) {
#pragma unroll
      for (int u = 0; u < kStages; ++u) {
        issue(j + u + kStages - 1, buf[(u + kStages - 1) % kStages]);
        if (j + u < cnt) compute(j + u, buf[u]);
      }
    }
  }

  // ---- items cut by share boundaries: arrive, and merge if last ------------
  for (int i = 0; i < npend; ++i) {
    const int s = i == 0 ? pend_s0 : pend_s1, g = i == 0 ? pend_g0 : pend_g1;
    const int A = g * C + s_cum[s];
    const int B = A + (s_cum[s + 1] - s_cum[s]);
    const int np = (B - 1) / share - A / share + 1;
    // The item's first wave holds the item's start and, the item running past
    // its share, ends with it: no other cut item starts in that wave, so the
    // wave's index names the item's counter.
    int* counter = p.bal_counters + A / share;
    // The piece's stores have completed (at the agent coherence point) before
    // the arrival is counted; the memory clobber keeps the compiler from
    // moving memory accesses across.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    int old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != np - 1) continue;
    // Last arrival: every other piece completed before its arrival was counted,
    // and the coherent loads below are issued after this one's count returned.
    asm volatile("" ::: "memory");
    const int w0 = A / share;
    for (int idx = lane; idx < G * (D / 4); idx += 64) {
      const int h = idx / (D / 4), d4 = idx - h * (D / 4);
      float M = neg_inf(), L = 0.f;
      float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
      // eight pieces' loads in flight at a time, then their online merge
      constexpr int kBatch = 8;
      for (int k0 = 0; k0 < np; k0 += kBatch) {
        float mv[kBatch], lv[kBatch];
        float4 ov[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int pw = w0 + min(k0 + u, np - 1);
          const float* pc = pieces + (int64_t)(2 * pw + (pw * share < A ? 1 : 0)) * stride;
          const float* po = pc + h * D + 4 * d4;
          mv[u] = coherent_load(pc + G * D + h);
          lv[u] = coherent_load(pc + G * D + G + h);
          ov[u] = make_float4(coherent_load(po), coherent_load(po + 1), coherent_load(po + 2),
                              coherent_load(po + 3));
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (k0 + u >= np) break;   // clamped repeats of the last piece are not counted
          const float m = mv[u];
          if (m > M) {
            const float f = (M == neg_inf()) ? 0.f : fast_exp2(M - m);
            L *= f;
            O.x *= f;
            O.y *= f;
            O.z *= f;
            O.w *= f;
            M = m;
          }
          const float f = (m == neg_inf()) ? 0.f : fast_exp2(m - M);
          L += f * lv[u];
          O.x += f * ov[u].x;
          O.y += f * ov[u].y;
          O.z += f * ov[u].z;
          O.w += f * ov[u].w;
        }
      }
      const float inv = 1.f / L;
      uint16_t* o = reinterpret_cast<uint16_t*>(p.out) + ((int64_t)s * Hq + g * G + h) * D + 4 * d4;
      *reinterpret_cast<uint2*>(o) = make_uint2(pack_bf16x2(O.x * inv, O.y * inv), pack_bf16x2(O.z * inv, O.w * inv));
    }
    if (lane == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);   // for the next call
  }

  // ---- sequences with an empty context: zero output rows -------------------
  for (int s = pos; s < S; s += NW) {
    if (s_cum[s + 1] != s_cum[s]) continue;
    uint4* o = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + (int64_t)s * Hq * D);
    for (int i = lane; i < Hq * D / 8; i += 64) o[i] = make_uint4(0, 0, 0, 0);
  }

  // ---- fused store: the new rows go to their cache slots --------------------
  if (fused) {
    if (new_item < S * Hkv) store_new_row(new_item);
    for (new_item += NW * kRowsPerPass; new_item < S * Hkv; new_item += NW * kRowsPerPass) {
      load_new_row(new_item);
      store_new_row(new_item);
    }
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static bool decode_grid_fits(const DecodeParams& p) {
  return (int64_t)p.num_seqs * p.num_kv_heads * p.num_partitions <= 0x7fffffff - kXcds;
}

static dim3 decode_grid(const DecodeParams& p) {
  const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads * p.num_partitions;
  return dim3((unsigned)((items + kXcds - 1) / kXcds * kXcds));
}

template <typename T, int D>
static hipError_t launch_valu_g(const DecodeParams& p, hipStream_t stream) {
  if (!decode_grid_fits(p)) return hipErrorInvalidValue;
  const dim3 grid = decode_grid(p);
  switch (p.group) {
#define PKV_G(GV) \
  case GV: hipLaunchKernelGGL((decode_valu_kernel<T, D, GV>), grid, dim3(kThreads), 0, stream, p); break;
    PKV_G(1) PKV_G(2) PKV_G(3) PKV_G(4) PKV_G(5) PKV_G(6) PKV_G(7) PKV_G(8)
#undef PKV_G
    default:
      // groups 9..16 for fp32 caches (bf16 ones use the MFMA kernel there);
      // the per-head state of 16 heads fits the registers at 4 elements per
      // lane, not at the 8 of bf16
      if constexpr (sizeof(T) == 4) {
        switch (p.group) {
#define PKV_G(GV) \
  case GV: hipLaunchKernelGGL((decode_valu_kernel<T, D, GV>), grid, dim3(kThreads), 0, stream, p); break;
          PKV_G(9) PKV_G(10) PKV_G(11) PKV_G(12) PKV_G(13) PKV_G(14) PKV_G(15) PKV_G(16)
#undef PKV_G
          default:
            return hipErrorInvalidValue;
        }
        break;
      }
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 0) return head_dim == 64 ? launch_valu_g<float, 64>(p, stream) : launch_valu_g<float, 128>(p, stream);
  return head_dim == 64 ? launch_valu_g<uint16_t, 64>(p, stream) : launch_valu_g<uint16_t, 128>(p, stream);
}

template <int D, bool FP8>
static hipError_t launch_mfma_d(const DecodeParams& p, hipStream_t stream) {
  if (!decode_grid_fits(p)) return hipErrorInvalidValue;
  dim3 grid = decode_grid(p);
  DecodeParams q = p;
  const int cus = device_compute_units();
  if (p.plan != nullptr)
    q.pair_span = cus;   // the plan holds the ranks: no limit from ranking in LDS
  else
    q.pair_span = (p.num_partitions == 1 && p.num_seqs <= kRankMaxSeqs && cus <= kRankMaxSeqs) ? cus : 0;
  const int64_t items = (int64_t)p.num_seqs * p.num_kv_heads;
  if (q.pair_span > 0 && items > q.pair_span && items <= 2 * (int64_t)q.pair_span)
    grid = dim3((unsigned)(2 * q.pair_span));   // a second workgroup on every unit
  if (p.group <= 4)
    hipLaunchKernelGGL((decode_mfma_kernel<D, 4, FP8>), grid, dim3(kThreads), 0, stream, q);
  else if (p.group <= 8)
    hipLaunchKernelGGL((decode_mfma_kernel<D, 8, FP8>), grid, dim3(kThreads), 0, stream, q);
  else
    hipLaunchKernelGGL((decode_mfma_kernel<D, 16, FP8>), grid, dim3(kThreads), 0, stream, q);
  return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_mfma_d<64, false>(p, stream) : launch_mfma_d<128, false>(p, stream);
}

hipError_t launch_decode_mfma_fp8(const DecodeParams& p, int head_dim, hipStream_t stream) {
  return head_dim == 64 ? launch_mfma_d<64, true>(p, stream) : launch_mfma_d<128, true>(p, stream);
}

hipError_t launch_decode_plan(const PlanParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(decode_plan_kernel, dim3(1), dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

// Compute units of the current device (queried once per device).
int device_compute_units() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
  int cus = cache[dev].load(std::memory_order_relaxed);
  if (cus > 0) return cus;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

// PKV_BAL_WG_PER_CU workgroups per compute unit (at most the kernel's
// occupancy of two), so the whole grid is resident at once; fewer when the
// batch has too few tiles to give every wave kBalMinShare of them.
hipError_t launch_decode_balanced(const DecodeParams& p, int head_dim, hipStream_t stream) {
  const int64_t tiles = (int64_t)p.num_seqs * p.num_kv_heads * ((p.max_ctx + kTile - 1) / kTile);
  const int64_t per_wg = (int64_t)kBalMinShare * kBalWavesPerWorkgroup;
  int64_t nwg = std::min<int64_t>(PKV_BAL_WG_PER_CU * (int64_t)device_compute_units(), kBalMaxWorkgroups);
  nwg = std::min<int64_t>(nwg, std::max<int64_t>((tiles + per_wg - 1) / per_wg, 1));
  nwg = std::min<int64_t>((nwg + kXcds - 1) / kXcds * kXcds, kBalMaxWorkgroups);
  const dim3 grid((unsigned)nwg);
  if (head_dim == 64)
    hipLaunchKernelGGL(decode_balanced_kernel<64>, grid, dim3(kBalThreads), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_balanced_kernel<128>, grid, dim3(kBalThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace pkv
