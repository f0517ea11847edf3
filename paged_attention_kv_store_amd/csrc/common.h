// Shared declarations of the HIP kernels' launchers and small device helpers.
// Internal to the library: the public interface is include/pkv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// log2(e): softmax runs in base 2 (v_exp_f32 computes 2^x), so logits are
// pre-multiplied by scale * log2(e); exp(a - b) == exp2(log2e*a - log2e*b).
constexpr float kLog2e = 1.4426950408889634f;

// Lazy rescaling threshold, in log2 units. The running max used as the
// softmax reference is raised only when a new logit exceeds it by more than
// this, so exp2(logit - reference) <= 2^8 and the fp32 sums stay far from
// overflow; the final division by the sum removes the reference exactly.
constexpr float kRescaleThreshold = 8.0f;

struct StoreParams {
  const void* k;
  const void* v;
  void* k_cache;
  void* v_cache;
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int64_t num_slots;     // num_blocks * block_size
  int32_t row_vec16;     // bytes of one token row (kv_heads * head_dim * elt) / 16
};

// E4M3 store: new rows (bf16 or fp32) quantised with one scale per kv-head.
struct StoreFp8Params {
  const void* k;
  const void* v;
  uint8_t* k_cache;
  uint8_t* v_cache;
  const int32_t* slot_mapping;
  const float* k_scale;      // [num_kv_heads]
  const float* v_scale;
  int32_t num_tokens;
  int64_t num_slots;
  int32_t row_elems;         // num_kv_heads * head_dim (a multiple of 8)
  int32_t head_dim;
  int32_t src_f32;           // 1: fp32 rows, 0: bf16 rows
};

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t max_blocks;        // block table row length
  int32_t num_blocks;
  int32_t block_size;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;             // num_q_heads / num_kv_heads
  float scale_log2;          // scale * log2(e)
  int32_t max_ctx;           // host bound; a larger device length is truncated to it
  int32_t partition_size;    // tokens per partition (single pass: >= max context)
  int32_t num_partitions;    // partitions per (sequence, kv-head) in the grid
  float* ws_m;               // [num_seqs, num_q_heads, num_partitions]
  float* ws_l;               // same
  float* ws_o;               // [num_seqs, num_q_heads, num_partitions, head_dim]
  int32_t* part_counters;    // [num_seqs * num_kv_heads] arrival counters, zero between calls
  // Fused store of one new row per sequence at position ctx-1 (all null when
  // not fused): k_new/v_new [num_seqs, num_kv_heads, head_dim], new_slots [num_seqs].
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
  // Shared-prefix decode, second pass (null otherwise): the sequence's
  // tokens before seq_prefix[s] are covered by partials of the first pass,
  // merged into the output.
  const int32_t* seq_prefix;   // [num_seqs]
  const float* pre_m;          // [num_seqs, num_q_heads]
  const float* pre_l;
  const float* pre_o;          // [num_seqs, num_q_heads, head_dim]
  // E4M3 caches only (null otherwise): dequantisation scales [num_kv_heads].
  const float* k_scale;
  const float* v_scale;
  // Work-balanced decode only: arrival counters [kBalMaxWaves] (zero between
  // calls; the start of the counter block) and per-wave pieces
  // [2 * kBalMaxWaves][piece_stride] (after the counter block).
  int32_t* bal_counters;
  float* bal_pieces;
  int32_t bal_piece_stride;  // floats per piece
  // Set by the per-item launcher: the compute units, when workgroups are
  // given their items by size (0: in index order).
  int32_t pair_span;
  // Planned single-pass decode (null otherwise): kPlanEntryInts int32 per
  // sequence, largest first, written by decode_plan_kernel.
  const int32_t* plan;
};

// A decode plan lists the sequences of a step largest first. Entry r:
// {sequence, its context_lens value, the table entries of the first tiles of
// waves 0..3 (16-token tiles w, i.e. block (16 w) / block_size), 0, 0}.
constexpr int kPlanEntryInts = 8;

struct PlanParams {
  int32_t* plan;             // [num_seqs, kPlanEntryInts]
  const int32_t* block_tables;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t block_size;
};

// Split-K: the workspace starts with this many arrival counters (one per
// (sequence, kv-head)), at a fixed place so that calls of any sizes can share
// a workspace; the partial results follow.
constexpr int kSplitMaxItems = 65536;
// Every decode mode that merges partial results keeps its arrival counters
// in this block at the start of the workspace (split-K: one per (sequence,
// kv-head); work-balanced: one per wave) and its partial results after it.
// Every call leaves the whole block zero, so one workspace serves calls of
// any mode and size in turn.
constexpr int64_t kCounterBytes = (int64_t)kSplitMaxItems * 4;

// Work-balanced decode limits. Every workgroup keeps the per-sequence tile
// prefix sums in LDS, which bounds the batch; the piece area is sized for
// the largest grid the launcher uses.
constexpr int kBalMaxSeqs = 8192;
constexpr int kBalMaxWorkgroups = 1024;
constexpr int kBalWavesPerWorkgroup = 4;
constexpr int kBalMaxWaves = kBalMaxWorkgroups * kBalWavesPerWorkgroup;
static_assert((int64_t)kBalMaxWaves * 4 <= kCounterBytes, "work-balanced counters fit the counter block");

// Floats of one piece: unnormalised output [G][D], then max [G] and sum [G],
// rounded up to 16 bytes.
inline int64_t bal_piece_stride(int group, int head_dim) {
  return ((int64_t)group * head_dim + 2 * group + 3) / 4 * 4;
}

struct PrefillParams {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* cu_seqlens_q;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t total_q;
  int32_t max_q_len;
  int32_t num_q_tiles;       // set by the launcher
  int32_t longest_first;     // set by the launcher: items start in order of cost
  int32_t pair_span;         // set by the launcher: compute units, when ids C .. 2C-1 are mirrored
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t block_size;
  int32_t block_size_log2;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_ctx;
  float scale_log2;
  int32_t causal;
  // Shared-prefix decode, first pass (all null / 0 otherwise): chunk c is a
  // group of sequences whose block-table row is that of its first query row
  // (cu_seqlens_q[c]), and instead of normalised rows the kernel writes
  // fp32 partials (log2 max, sum, unnormalised output) per (row, q-head),
  // plus the chunk's context length for each of its rows in seq_prefix.
  int32_t table_row_is_first_q;
  float* part_m;             // [total_q, num_q_heads]
  float* part_l;
  float* part_o;             // [total_q, num_q_heads, head_dim]
  int32_t* seq_prefix;       // [total_q]
  // E4M3 caches only (null otherwise): dequantisation scales [num_kv_heads].
  const float* k_scale;
  const float* v_scale;
};

// Checks of device-held inputs (debugging aids; see check.hip).
//   report[0] lengths outside [0, max_ctx], [1] used table entries outside
//   the pool, [2] chunks with an impossible row count, [3] the lowest
//   offending sequence (num_seqs if none).
struct CheckParams {
  const int32_t* block_tables;
  const int32_t* context_lens;
  const int32_t* cu_seqlens_q;   // null: decode (no chunks)
  int32_t num_seqs;
  int32_t max_blocks;
  int32_t max_ctx;
  int32_t num_blocks;
  int32_t block_size;
  int32_t total_q;
  int32_t max_q_len;
  int32_t* report;
};
//   report[0] slots past the pool, [1] repeated claims of a slot, [2]
//   negative (padding) slots, [3] the lowest offending token (num_tokens if
//   none). seen, dup: bitmaps of ceil(num_slots / 32) words each, dup = seen + words.
struct SlotCheckParams {
  const int32_t* slot_mapping;
  int32_t num_tokens;
  int64_t num_slots;
  uint32_t* seen;
  uint32_t* dup;
  int32_t* report;
};

// Compute units of the current device (queried once per device).
int device_compute_units();

// Bytes of the library-owned decode scratch (one array per device, held
// until the process ends), and its device address on the current device.
constexpr size_t kStaticScratchBytes = (size_t)64 << 20;
hipError_t static_scratch(void** ptr);

// p[0 .. n-1] = 0 with a kernel on `stream`.
hipError_t launch_zero_ints(int32_t* p, int64_t n, hipStream_t stream);

// dtype codes match pkv_dtype
hipError_t launch_store(const StoreParams& p, hipStream_t stream);
hipError_t launch_store_fp8(const StoreFp8Params& p, hipStream_t stream);
hipError_t launch_decode_valu(const DecodeParams& p, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_mfma_fp8(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_balanced(const DecodeParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_plan(const PlanParams& p, hipStream_t stream);
hipError_t launch_prefill(const PrefillParams& p, int head_dim, hipStream_t stream);
hipError_t launch_prefill_fp8(const PrefillParams& p, int head_dim, hipStream_t stream);
hipError_t launch_check_tables(const CheckParams& p, hipStream_t stream);
hipError_t launch_check_slots(const SlotCheckParams& p, hipStream_t stream);

}  // namespace pkv
