// C ABI of the library: argument validation, launch configuration, dispatch.
// The contract of every entry point is documented in include/pkv.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "common.h"
#include "pkv.h"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_EHIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

int elt_size(int dt) { return dt == PKV_F32 ? 4 : dt == PKV_BF16 ? 2 : 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Partitions per (sequence, kv-head) and the tokens in each; single pass
// (partition_size 0) is one partition spanning the longest context.
void partitioning(int32_t max_ctx, int32_t partition_size, int32_t* part, int64_t* nparts) {
  if (partition_size == 0) {
    *part = (int32_t)(ceil_div(max_ctx > 16 ? max_ctx : 16, 16) * 16);
    *nparts = 1;
  } else {
    *part = partition_size;
    *nparts = max_ctx > 0 ? ceil_div(max_ctx, partition_size) : 1;
  }
}

// The partition size PKV_PARTITION_AUTO stands for. Single pass when the
// (sequence, kv-head) items give every compute unit two workgroups, or when
// contexts are short enough that the longest item is not the tail; otherwise
// split-K with 1024-token partitions (halved down to 256 while the longest
// context's partitions still could not fill two workgroups per unit).
// Measured on one MI355X: 256 items of up to 32K tokens take 384 us in one
// pass and 213 us with 1024- or 2048-token partitions; 1024 and 2048 items of
// up to 4K tokens are fastest in one pass (split-K at 2048 tokens adds 12-14%).
// The split-K partition for a batch too small to fill the GPU in one pass:
// about one partition per compute unit, as a power of two within
// [512, 2048] tokens (fewer, longer partitions leave fewer partials to
// merge; shorter ones leave compute units idle). 0 when one partition holds
// the longest context.
int32_t auto_split(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx) {
  const int64_t items = (int64_t)num_seqs * num_kv_heads;
  const int64_t per_unit = ceil_div(items * max_ctx, (int64_t)pkv::device_compute_units());
  int32_t part = 512;
  while (part < 2048 && part < per_unit) part *= 2;
  return ceil_div(max_ctx, part) > 1 ? part : 0;
}

// PKV_PARTITION_AUTO (measured on full-size batches of 1 to 64 sequences of
// up to 32K tokens, uniform, log-uniform and equal lengths): one pass when
// the items give every compute unit two workgroups or contexts are short;
// the work-balanced decode for mid-sized batches (from half a workgroup per
// compute unit), whose equal shares absorb the spread of lengths that the
// host cannot see; split-K (auto_split) for the smallest batches, where the
// work-balanced decode would split each item between too many waves.
int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx) {
  const int64_t items = (int64_t)num_seqs * num_kv_heads;
  const int64_t cus = pkv::device_compute_units();
  if (items >= 2 * cus || max_ctx <= 2048 || items > pkv::kSplitMaxItems) return 0;
  if (2 * items >= cus && num_seqs <= pkv::kBalMaxSeqs &&
      items * ceil_div(max_ctx, 16) < ((int64_t)1 << 30))
    return PKV_PARTITION_BALANCED;
  return auto_split(num_seqs, num_kv_heads, max_ctx);
}

int check_common(const char* fn, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                 int32_t head_dim, int dtype) {
  if (elt_size(dtype) == 0) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (num_blocks <= 0 || block_size <= 0 || num_kv_heads <= 0 || head_dim <= 0)
    return fail(PKV_EINVAL, "%s: num_blocks, block_size, num_kv_heads and head_dim must be positive", fn);
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_version(void) { return 100; }

extern "C" const char* pkv_last_error(void) { return g_last_error.c_str(); }

extern "C" int pkv_kv_cache_store(const void* k, const void* v, void* k_cache, void* v_cache,
                                  const int32_t* slot_mapping, int32_t num_tokens,
                                  int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                                  int32_t head_dim, pkv_dtype dtype, void* stream) {
  const char* fn = "pkv_kv_cache_store";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens < 0", fn);
  if (int rc = check_common(fn, num_blocks, block_size, num_kv_heads, head_dim, dtype)) return rc;
  const int64_t row_bytes = (int64_t)num_kv_heads * head_dim * elt_size(dtype);
  if (row_bytes % 16 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: a token row (%lld bytes) must be a multiple of 16 bytes", fn,
                (long long)row_bytes);
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(slot_mapping, 4))
    return fail(PKV_EINVAL, "%s: K/V pointers must be 16-byte aligned, slots 4-byte aligned", fn);
  pkv::StoreParams p;
  p.k = k;
  p.v = v;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_slots = (int64_t)num_blocks * block_size;
  p.row_vec16 = (int32_t)(row_bytes / 16);
  return hip_status(pkv::launch_store(p, (hipStream_t)stream), fn);
}


extern "C" size_t pkv_decode_plan_size(int32_t num_seqs) {
  if (num_seqs <= 0) return 0;
  return (size_t)num_seqs * pkv::kPlanEntryInts * sizeof(int32_t);
}

extern "C" int pkv_decode_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int32_t block_size, void* stream) {
  const char* fn = "pkv_decode_plan";
  if (num_seqs < 0 || num_seqs > 65535) return fail(PKV_EINVAL, "%s: num_seqs %d outside [0, 65535]", fn, num_seqs);
  if (block_size % 16 != 0 || block_size <= 0 || block_size > 256)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d must be a multiple of 16 up to 256", fn, block_size);
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "%s: max_blocks_per_seq must be positive", fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_context_len %d outside [0, max_blocks_per_seq * block_size = %lld]", fn,
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (num_seqs == 0) return PKV_OK;
  if (!plan || !block_tables || !context_lens) return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (plan_bytes < pkv_decode_plan_size(num_seqs))
    return fail(PKV_EWORKSPACE, "%s: the plan needs %zu bytes, got %zu", fn, pkv_decode_plan_size(num_seqs),
                plan_bytes);
  if (!aligned(plan, 16) || !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_EINVAL, "%s: plan must be 16-byte aligned, index arrays 4-byte", fn);
  pkv::PlanParams p;
  p.plan = reinterpret_cast<int32_t*>(plan);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.max_ctx = max_context_len;
  p.block_size = block_size;
  return hip_status(pkv::launch_decode_plan(p, (hipStream_t)stream), fn);
}

extern "C" size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, int32_t max_context_len,
                                            int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  if (partition_size == PKV_PARTITION_AUTO) {
    // a work-balanced choice falls back to split-K for calls the
    // work-balanced decode does not take (fp32, E4M3): room for either
    const int32_t a = auto_partition(num_seqs, num_kv_heads, max_context_len);
    const size_t wa = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, a);
    if (a != PKV_PARTITION_BALANCED) return wa;
    const size_t ws = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                                                auto_split(num_seqs, num_kv_heads, max_context_len));
    return wa > ws ? wa : ws;
  }
  if (partition_size == PKV_PARTITION_BALANCED) {
    // the counter block (its first kBalMaxWaves counters: one per wave), then
    // two pieces per wave, for the largest grid
    const int64_t stride = pkv::bal_piece_stride(num_q_heads / num_kv_heads, head_dim);
    return (size_t)(pkv::kCounterBytes + 2 * (int64_t)pkv::kBalMaxWaves * stride * (int64_t)sizeof(float));
  }
  if (partition_size == PKV_PARTITION_PLANNED) return pkv_decode_plan_size(num_seqs);
  if (partition_size <= 0) return 0;
  int32_t part;
  int64_t nparts;
  partitioning(max_context_len, partition_size, &part, &nparts);
  if (nparts <= 1) return 0;
  // the counter block (one counter per (sequence, kv-head)), then m, l, o of
  // every (sequence, q-head, partition)
  return (size_t)pkv::kCounterBytes + (size_t)num_seqs * num_q_heads * nparts * (head_dim + 2) * sizeof(float);
}

extern "C" int32_t pkv_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len) {
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_context_len < 0) return 0;
  return auto_partition(num_seqs, num_kv_heads, max_context_len);
}

extern "C" int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_decode_workspace_init";
  if (workspace_bytes == 0) return PKV_OK;
  if (!workspace) return fail(PKV_EINVAL, "%s: null workspace", fn);
  if (!aligned(workspace, 4)) return fail(PKV_EINVAL, "%s: workspace must be 4-byte aligned", fn);
  // the counter block shared by the split-K and the work-balanced layouts
  const size_t bytes = workspace_bytes < (size_t)pkv::kCounterBytes ? workspace_bytes : (size_t)pkv::kCounterBytes;
  return hip_status(pkv::launch_zero_ints(reinterpret_cast<int32_t*>(workspace), (int64_t)(bytes / 4),
                                          (hipStream_t)stream), fn);
}

namespace {

// Shared by the plain and the store-fused decode entry points; k_new, v_new
// and new_slots are null for the plain one.
int decode_impl(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens, const void* k_new,
                const void* v_new, const int32_t* new_slots, int32_t num_seqs,
                int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks,
                int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                int dtype, int32_t algo, void* stream, bool fp8 = false,
                const float* k_scale = nullptr, const float* v_scale = nullptr,
                bool clear_counters = false) {
  if (num_seqs < 0) return fail(PKV_EINVAL, "%s: num_seqs < 0", fn);
  if (int rc = check_common(fn, num_blocks, block_size, num_kv_heads, head_dim, dtype)) return rc;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                num_q_heads, num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d not in {64, 128}", fn, head_dim);
  if (block_size % 16 != 0 || block_size > 256)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d must be a multiple of 16 up to 256", fn, block_size);
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "%s: max_blocks_per_seq must be positive", fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_context_len %d outside [0, max_blocks_per_seq * block_size = %lld]", fn,
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (partition_size == PKV_PARTITION_AUTO) {
    partition_size = auto_partition(num_seqs, num_kv_heads, max_context_len);
    const bool mfma = algo == PKV_DECODE_MFMA || (algo == PKV_DECODE_AUTO && dtype == PKV_BF16);
    if (partition_size == PKV_PARTITION_BALANCED && (fp8 || !mfma || dtype != PKV_BF16))
      partition_size = auto_split(num_seqs, num_kv_heads, max_context_len);
  }
  const bool balanced = partition_size == PKV_PARTITION_BALANCED;
  const bool planned = partition_size == PKV_PARTITION_PLANNED;
  if (!balanced && !planned && (partition_size < 0 || partition_size % 16 != 0))
    return fail(PKV_EINVAL, "%s: partition_size %d must be 0, a positive multiple of 16, "
                "PKV_PARTITION_BALANCED, PKV_PARTITION_PLANNED or PKV_PARTITION_AUTO", fn, partition_size);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
  if (algo == PKV_DECODE_AUTO) algo = dtype == PKV_BF16 ? PKV_DECODE_MFMA : PKV_DECODE_VALU;
  if (fp8) {
    if (dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "%s: q and out must be bf16", fn);
    if (algo != PKV_DECODE_MFMA)
      return fail(PKV_EUNSUPPORTED, "%s: E4M3 caches are read by the MFMA kernel only", fn);
    if (balanced)
      return fail(PKV_EUNSUPPORTED, "%s: no work-balanced decode over E4M3 caches", fn);
  }
  if (algo == PKV_DECODE_MFMA) {
    if (dtype != PKV_BF16) return fail(PKV_EUNSUPPORTED, "%s: the MFMA kernel needs bf16", fn);
    if (group > 16) return fail(PKV_EUNSUPPORTED, "%s: GQA group %d > 16", fn, group);
  } else if (algo == PKV_DECODE_VALU) {
    const int max_group = dtype == PKV_F32 ? 16 : 8;   // per-head state in registers: 4 or 8 elements a lane
    if (group > max_group)
      return fail(PKV_EUNSUPPORTED, "%s: the VALU kernel supports GQA groups up to %d for this dtype", fn,
                  max_group);
  } else {
    return fail(PKV_EINVAL, "%s: unknown algo %d", fn, algo);
  }
  if (num_seqs > 65535 || num_kv_heads > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs and num_kv_heads are limited to 65535", fn);
  if (planned && algo != PKV_DECODE_MFMA)
    return fail(PKV_EUNSUPPORTED, "%s: the planned decode runs on the MFMA kernel (bf16)", fn);
  if (balanced) {
    if (algo != PKV_DECODE_MFMA)
      return fail(PKV_EUNSUPPORTED, "%s: the work-balanced decode runs on the MFMA kernel (bf16)", fn);
    if (num_seqs > pkv::kBalMaxSeqs)
      return fail(PKV_EUNSUPPORTED, "%s: the work-balanced decode takes at most %d sequences", fn,
                  pkv::kBalMaxSeqs);
    if ((int64_t)num_seqs * num_kv_heads * ceil_div(max_context_len, 16) >= ((int64_t)1 << 30))
      return fail(PKV_EUNSUPPORTED, "%s: more than 2^30 tiles for the work-balanced decode", fn);
  }
  {
    int32_t part_probe;
    int64_t nparts_probe;
    partitioning(max_context_len, (balanced || planned) ? 0 : partition_size, &part_probe, &nparts_probe);
    if (nparts_probe > 1 && (int64_t)num_seqs * num_kv_heads > pkv::kSplitMaxItems)
      return fail(PKV_EUNSUPPORTED, "%s: split-K takes at most %d (sequence, kv-head) pairs", fn,
                  pkv::kSplitMaxItems);
  }
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (balanced && !aligned(out, 16))
    return fail(PKV_EINVAL, "%s: the work-balanced decode needs a 16-byte aligned out", fn);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4))
    return fail(PKV_EINVAL, "%s: q and caches must be 16-byte aligned; out and index arrays 4-byte", fn);
  const bool fused = new_slots != nullptr;
  if (fp8 && (!k_scale || !v_scale || !aligned(k_scale, 4) || !aligned(v_scale, 4)))
    return fail(PKV_EINVAL, "%s: k_scale and v_scale must be non-null, 4-byte aligned", fn);
  if (fused && (!k_new || !v_new || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(new_slots, 4)))
    return fail(PKV_EINVAL, "%s: k_new and v_new must be non-null and 16-byte aligned", fn);

  int32_t part;
  int64_t nparts;
  partitioning(max_context_len, (balanced || planned) ? 0 : partition_size, &part, &nparts);
  if ((int64_t)num_seqs * num_kv_heads * nparts > 0x7ffffff0)
    return fail(PKV_EUNSUPPORTED, "%s: %lld work items exceed the grid; use a larger partition_size", fn,
                (long long)num_seqs * num_kv_heads * nparts);
  pkv::DecodeParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.scale_log2 = scale * pkv::kLog2e;
  p.max_ctx = max_context_len;
  p.partition_size = part;
  p.num_partitions = (int32_t)nparts;
  p.ws_m = p.ws_l = p.ws_o = nullptr;
  p.part_counters = nullptr;
  p.k_new = fused ? k_new : nullptr;
  p.v_new = fused ? v_new : nullptr;
  p.new_slots = fused ? new_slots : nullptr;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.seq_prefix = nullptr;
  p.pre_m = p.pre_l = p.pre_o = nullptr;
  p.bal_counters = nullptr;
  p.bal_pieces = nullptr;
  p.bal_piece_stride = 0;
  p.pair_span = 0;
  p.plan = nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (planned) {
    const size_t need = pkv_decode_plan_size(num_seqs);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EWORKSPACE, "%s: the planned decode needs its plan (%zu bytes) as workspace, got %zu", fn,
                  need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(PKV_EINVAL, "%s: the plan must be 16-byte aligned", fn);
    p.plan = reinterpret_cast<const int32_t*>(workspace);
  }
  if (balanced) {
    const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len, partition_size);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EWORKSPACE, "%s: the work-balanced decode needs %zu workspace bytes, got %zu", fn,
                  need, workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 256)) return fail(PKV_EINVAL, "%s: workspace must be 256-byte aligned", fn);
    p.bal_counters = reinterpret_cast<int32_t*>(workspace);
    p.bal_pieces = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + pkv::kCounterBytes);
    p.bal_piece_stride = (int32_t)pkv::bal_piece_stride(group, head_dim);
    if (clear_counters)
      if (hipError_t e = pkv::launch_zero_ints(p.bal_counters, pkv::kBalMaxWaves, st); e != hipSuccess)
        return hip_status(e, fn);
    return hip_status(pkv::launch_decode_balanced(p, head_dim, st), fn);
  }
  if (nparts > 1) {
    const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                  max_context_len, partition_size);
    if (!workspace || workspace_bytes < need)
      return fail(PKV_EWORKSPACE, "%s: split-K needs %zu workspace bytes, got %zu", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(PKV_EINVAL, "%s: workspace must be 16-byte aligned", fn);
    const int64_t cells = (int64_t)num_seqs * num_q_heads * nparts;
    p.part_counters = reinterpret_cast<int32_t*>(workspace);
    float* ws = reinterpret_cast<float*>(reinterpret_cast<char*>(workspace) + pkv::kCounterBytes);
    p.ws_m = ws;
    p.ws_l = ws + cells;
    p.ws_o = ws + 2 * cells;
    if (clear_counters)
      if (hipError_t e = pkv::launch_zero_ints(p.part_counters, (int64_t)num_seqs * num_kv_heads, st);
          e != hipSuccess)
        return hip_status(e, fn);
  }
  hipError_t e = fp8 ? pkv::launch_decode_mfma_fp8(p, head_dim, st)
                 : algo == PKV_DECODE_MFMA ? pkv::launch_decode_mfma(p, head_dim, st)
                                           : pkv::launch_decode_valu(p, head_dim, dtype, st);
  if (e != hipSuccess) return hip_status(e, fn);
  return PKV_OK;
}

}  // namespace

extern "C" int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const int32_t* block_tables,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t max_blocks_per_seq, int32_t max_context_len,
                                          int32_t num_blocks, int32_t block_size,
                                          int32_t num_q_heads, int32_t num_kv_heads,
                                          int32_t head_dim, float scale, int32_t partition_size,
                                          void* workspace, size_t workspace_bytes,
                                          pkv_dtype dtype, int32_t algo, void* stream) {
  return decode_impl("pkv_paged_attention_decode", out, q, k_cache, v_cache, block_tables,
                     context_lens, nullptr, nullptr, nullptr, num_seqs, max_blocks_per_seq,
                     max_context_len, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim,
                     scale, partition_size, workspace, workspace_bytes, dtype, algo, stream);
}

extern "C" int pkv_paged_attention_decode_store(void* out, const void* q, void* k_cache,
                                                void* v_cache, const int32_t* block_tables,
                                                const int32_t* context_lens, const void* k_new,
                                                const void* v_new, const int32_t* slot_mapping,
                                                int32_t num_seqs, int32_t max_blocks_per_seq,
                                                int32_t max_context_len, int32_t num_blocks,
                                                int32_t block_size, int32_t num_q_heads,
                                                int32_t num_kv_heads, int32_t head_dim, float scale,
                                                int32_t partition_size, void* workspace,
                                                size_t workspace_bytes, pkv_dtype dtype, int32_t algo,
                                                void* stream) {
  const char* fn = "pkv_paged_attention_decode_store";
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  return decode_impl(fn, out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                     slot_mapping, num_seqs, max_blocks_per_seq, max_context_len, num_blocks,
                     block_size, num_q_heads, num_kv_heads, head_dim, scale, partition_size,
                     workspace, workspace_bytes, dtype, algo, stream);
}

static_assert(PKV_STATIC_SCRATCH_BYTES == pkv::kStaticScratchBytes, "header and library agree on the scratch");

extern "C" int pkv_paged_attention_decode_static(void* out, const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_tables,
                                                 const int32_t* context_lens, int32_t num_seqs,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t num_blocks, int32_t block_size,
                                                 int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, float scale, int32_t partition_size,
                                                 pkv_dtype dtype, int32_t algo, void* stream) {
  const char* fn = "pkv_paged_attention_decode_static";
  if (partition_size == PKV_PARTITION_PLANNED)
    return fail(PKV_EINVAL, "%s: the planned decode reads a caller's plan; use pkv_paged_attention_decode", fn);
  const size_t need = pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                max_context_len, partition_size);
  if (need > pkv::kStaticScratchBytes)
    return fail(PKV_EWORKSPACE, "%s: the call needs %zu bytes of scratch; the library's static scratch holds %zu",
                fn, need, pkv::kStaticScratchBytes);
  void* ws = nullptr;
  if (need > 0)
    if (hipError_t e = pkv::static_scratch(&ws); e != hipSuccess) return hip_status(e, fn);
  return decode_impl(fn, out, q, k_cache, v_cache, block_tables, context_lens, nullptr, nullptr, nullptr,
                     num_seqs, max_blocks_per_seq, max_context_len, num_blocks, block_size, num_q_heads,
                     num_kv_heads, head_dim, scale, partition_size, ws, ws ? pkv::kStaticScratchBytes : 0,
                     dtype, algo, stream, false, nullptr, nullptr, /*clear_counters=*/true);
}

extern "C" int pkv_kv_cache_store_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                                      const int32_t* slot_mapping, const float* k_scale,
                                      const float* v_scale, int32_t num_tokens, int32_t num_blocks,
                                      int32_t block_size, int32_t num_kv_heads, int32_t head_dim,
                                      pkv_dtype src_dtype, void* stream) {
  const char* fn = "pkv_kv_cache_store_fp8";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens < 0", fn);
  if (int rc = check_common(fn, num_blocks, block_size, num_kv_heads, head_dim, src_dtype)) return rc;
  if (head_dim % 8 != 0)
    return fail(PKV_EUNSUPPORTED, "%s: head_dim %d must be a multiple of 8", fn, head_dim);
  if ((int64_t)num_kv_heads * head_dim > 0x7fffffff)
    return fail(PKV_EUNSUPPORTED, "%s: token row too long", fn);
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping || !k_scale || !v_scale)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 8) || !aligned(v_cache, 8) ||
      !aligned(slot_mapping, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return fail(PKV_EINVAL, "%s: new rows must be 16-byte aligned, caches 8-byte, slots and scales 4-byte",
                fn);
  pkv::StoreFp8Params p;
  p.k = k;
  p.v = v;
  p.k_cache = reinterpret_cast<uint8_t*>(k_cache);
  p.v_cache = reinterpret_cast<uint8_t*>(v_cache);
  p.slot_mapping = slot_mapping;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.num_tokens = num_tokens;
  p.num_slots = (int64_t)num_blocks * block_size;
  p.row_elems = num_kv_heads * head_dim;
  p.head_dim = head_dim;
  p.src_f32 = src_dtype == PKV_F32 ? 1 : 0;
  return hip_status(pkv::launch_store_fp8(p, (hipStream_t)stream), fn);
}

extern "C" int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                              const void* v_cache, const float* k_scale,
                                              const float* v_scale, const int32_t* block_tables,
                                              const int32_t* context_lens, int32_t num_seqs,
                                              int32_t max_blocks_per_seq, int32_t max_context_len,
                                              int32_t num_blocks, int32_t block_size,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, float scale, int32_t partition_size,
                                              void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode_fp8";
  return decode_impl(fn, out, q, k_cache, v_cache, block_tables, context_lens, nullptr, nullptr,
                     nullptr, num_seqs, max_blocks_per_seq, max_context_len, num_blocks, block_size,
                     num_q_heads, num_kv_heads, head_dim, scale, partition_size, workspace,
                     workspace_bytes, PKV_BF16, PKV_DECODE_MFMA, stream, true, k_scale, v_scale);
}

extern "C" int pkv_paged_attention_decode_store_fp8(
    void* out, const void* q, void* k_cache, void* v_cache, const float* k_scale, const float* v_scale,
    const int32_t* block_tables, const int32_t* context_lens, const void* k_new, const void* v_new,
    const int32_t* slot_mapping, int32_t num_seqs, int32_t max_blocks_per_seq, int32_t max_context_len,
    int32_t num_blocks, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
    float scale, int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode_store_fp8";
  if (num_seqs > 0 && (!k_new || !v_new || !slot_mapping))
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  return decode_impl(fn, out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                     slot_mapping, num_seqs, max_blocks_per_seq, max_context_len, num_blocks, block_size,
                     num_q_heads, num_kv_heads, head_dim, scale, partition_size, workspace,
                     workspace_bytes, PKV_BF16, PKV_DECODE_MFMA, stream, true, k_scale, v_scale);
}

static int prefill_impl(const char* fn, void* out, const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* block_tables, const int32_t* cu_seqlens_q, const int32_t* context_lens,
                        int32_t num_seqs, int32_t total_q, int32_t max_q_len, int32_t max_blocks_per_seq,
                        int32_t max_context_len, int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, float scale, int32_t causal, pkv_dtype dtype,
                        bool fp8, const float* k_scale, const float* v_scale, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0)
    return fail(PKV_EINVAL, "%s: negative size", fn);
  if (int rc = check_common(fn, num_blocks, block_size, num_kv_heads, head_dim, dtype)) return rc;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                num_q_heads, num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (dtype != PKV_BF16)
    return fail(PKV_EUNSUPPORTED, fp8 ? "%s: q and out must be bf16" : "%s: prefill supports bf16 only", fn);
  if (head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: prefill supports head_dim 128 only", fn);
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return fail(PKV_EUNSUPPORTED, "%s: GQA group %d not in {1, 2, 4, 8, 16}", fn, group);
  if (block_size < 16 || block_size > 256 || (block_size & (block_size - 1)) != 0)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d must be a power of two in [16, 256]", fn, block_size);
  if ((int64_t)block_size * num_kv_heads * head_dim * (fp8 ? 1 : 2) >= ((int64_t)1 << 31))
    return fail(PKV_EUNSUPPORTED, "%s: a cache block must be under 2 GiB", fn);
  if ((int64_t)num_blocks * block_size > (int64_t)0xffffffff)
    return fail(PKV_EUNSUPPORTED, "%s: the pool must hold fewer than 2^32 token rows", fn);
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "%s: max_blocks_per_seq must be positive", fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_context_len outside [0, max_blocks_per_seq * block_size]", fn);
  if (max_q_len > max_context_len) return fail(PKV_EINVAL, "%s: max_q_len exceeds max_context_len", fn);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
  if (num_seqs > 65535 || num_kv_heads > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs and num_kv_heads are limited to 65535", fn);
  if (num_seqs == 0 || total_q == 0 || max_q_len == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !cu_seqlens_q || !context_lens)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (fp8 && (!k_scale || !v_scale)) return fail(PKV_EINVAL, "%s: null scale pointer", fn);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_seqlens_q, 4) ||
      (fp8 && (!aligned(k_scale, 4) || !aligned(v_scale, 4))))
    return fail(PKV_EINVAL, "%s: q, out and caches must be 16-byte aligned; index arrays and scales 4-byte", fn);
  pkv::PrefillParams p;
  p.out = out;
  p.q = q;
  p.k_cache = k_cache;
  p.v_cache = v_cache;
  p.block_tables = block_tables;
  p.cu_seqlens_q = cu_seqlens_q;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.total_q = total_q;
  p.max_q_len = max_q_len;
  p.max_blocks = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.block_size_log2 = __builtin_ctz((unsigned)block_size);
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.group = group;
  p.max_ctx = max_context_len;
  p.scale_log2 = scale * pkv::kLog2e;
  p.causal = causal != 0;
  p.table_row_is_first_q = 0;
  p.part_m = p.part_l = p.part_o = nullptr;
  p.seq_prefix = nullptr;
  p.k_scale = fp8 ? k_scale : nullptr;
  p.v_scale = fp8 ? v_scale : nullptr;
  const hipStream_t st = (hipStream_t)stream;
  return hip_status(fp8 ? pkv::launch_prefill_fp8(p, head_dim, st) : pkv::launch_prefill(p, head_dim, st), fn);
}

extern "C" int pkv_paged_attention_prefill_chunk(void* out, const void* q, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_tables,
                                                 const int32_t* cu_seqlens_q,
                                                 const int32_t* context_lens, int32_t num_seqs,
                                                 int32_t total_q, int32_t max_q_len,
                                                 int32_t max_blocks_per_seq, int32_t max_context_len,
                                                 int32_t num_blocks, int32_t block_size,
                                                 int32_t num_q_heads, int32_t num_kv_heads,
                                                 int32_t head_dim, float scale, int32_t causal,
                                                 pkv_dtype dtype, void* stream) {
  return prefill_impl("pkv_paged_attention_prefill_chunk", out, q, k_cache, v_cache, block_tables,
                      cu_seqlens_q, context_lens, num_seqs, total_q, max_q_len, max_blocks_per_seq,
                      max_context_len, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale,
                      causal, dtype, false, nullptr, nullptr, stream);
}

extern "C" int pkv_paged_attention_prefill_chunk_fp8(void* out, const void* q, const void* k_cache,
                                                     const void* v_cache, const float* k_scale,
                                                     const float* v_scale, const int32_t* block_tables,
                                                     const int32_t* cu_seqlens_q,
                                                     const int32_t* context_lens, int32_t num_seqs,
                                                     int32_t total_q, int32_t max_q_len,
                                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                                     int32_t num_blocks, int32_t block_size,
                                                     int32_t num_q_heads, int32_t num_kv_heads,
                                                     int32_t head_dim, float scale, int32_t causal,
                                                     void* stream) {
  return prefill_impl("pkv_paged_attention_prefill_chunk_fp8", out, q, k_cache, v_cache, block_tables,
                      cu_seqlens_q, context_lens, num_seqs, total_q, max_q_len, max_blocks_per_seq,
                      max_context_len, num_blocks, block_size, num_q_heads, num_kv_heads, head_dim, scale,
                      causal, PKV_BF16, true, k_scale, v_scale, stream);
}

extern "C" size_t pkv_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                                          int32_t head_dim) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  // partials m, l, o per (sequence, q-head), then the prefix length of each sequence
  return (size_t)num_seqs * num_q_heads * (head_dim + 2) * sizeof(float) + (size_t)num_seqs * sizeof(int32_t);
}

extern "C" int pkv_paged_attention_decode_shared_prefix(
    void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
    const int32_t* context_lens, const int32_t* group_starts, const int32_t* group_prefix_lens,
    int32_t num_groups, int32_t max_group_size, int32_t max_prefix_len, int32_t num_seqs,
    int32_t max_blocks_per_seq, int32_t max_context_len, int32_t num_blocks, int32_t block_size,
    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, float scale, void* workspace,
    size_t workspace_bytes, void* stream) {
  const char* fn = "pkv_paged_attention_decode_shared_prefix";
  if (num_seqs < 0 || num_groups < 0 || max_group_size < 0 || max_prefix_len < 0)
    return fail(PKV_EINVAL, "%s: negative size", fn);
  if (int rc = check_common(fn, num_blocks, block_size, num_kv_heads, head_dim, PKV_BF16)) return rc;
  if (num_q_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_EINVAL, "%s: num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)", fn,
                num_q_heads, num_kv_heads);
  const int group = num_q_heads / num_kv_heads;
  if (head_dim != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim 128 only", fn);
  if (group != 1 && group != 2 && group != 4 && group != 8 && group != 16)
    return fail(PKV_EUNSUPPORTED, "%s: GQA group %d not in {1, 2, 4, 8, 16}", fn, group);
  if (block_size < 16 || block_size > 256 || (block_size & (block_size - 1)) != 0)
    return fail(PKV_EUNSUPPORTED, "%s: block_size %d must be a power of two in [16, 256]", fn, block_size);
  if ((int64_t)block_size * num_kv_heads * head_dim * 2 >= ((int64_t)1 << 31))
    return fail(PKV_EUNSUPPORTED, "%s: a cache block must be under 2 GiB", fn);
  if ((int64_t)num_blocks * block_size > (int64_t)0xffffffff)
    return fail(PKV_EUNSUPPORTED, "%s: the pool must hold fewer than 2^32 token rows", fn);
  if (max_blocks_per_seq <= 0) return fail(PKV_EINVAL, "%s: max_blocks_per_seq must be positive", fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_context_len outside [0, max_blocks_per_seq * block_size]", fn);
  if (max_prefix_len > max_context_len)
    return fail(PKV_EINVAL, "%s: max_prefix_len exceeds max_context_len", fn);
  if (!std::isfinite(scale)) return fail(PKV_EINVAL, "%s: scale is not finite", fn);
  if (num_seqs > 65535 || num_kv_heads > 65535 || num_groups > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: num_seqs, num_groups and num_kv_heads are limited to 65535", fn);
  if (num_seqs == 0) return PKV_OK;
  if (num_groups == 0 || max_group_size == 0)
    return fail(PKV_EINVAL, "%s: the groups must cover the sequences", fn);
  if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !group_starts ||
      !group_prefix_lens)
    return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 4) ||
      !aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(group_starts, 4) ||
      !aligned(group_prefix_lens, 4))
    return fail(PKV_EINVAL, "%s: q and caches must be 16-byte aligned; out and index arrays 4-byte", fn);
  const size_t need = pkv_decode_shared_prefix_workspace_size(num_seqs, num_q_heads, head_dim);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EWORKSPACE, "%s: needs %zu workspace bytes, got %zu", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 16)) return fail(PKV_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  const int64_t cells = (int64_t)num_seqs * num_q_heads;
  float* ws = reinterpret_cast<float*>(workspace);
  float* part_m = ws;
  float* part_l = ws + cells;
  float* part_o = ws + 2 * cells;
  int32_t* seq_prefix = reinterpret_cast<int32_t*>(ws + 2 * cells + cells * head_dim);
  hipStream_t st = (hipStream_t)stream;

  // first pass: each group's query rows over its shared prefix, as one
  // non-causal chunk read through the first member's table
  pkv::PrefillParams a;
  a.out = nullptr;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.cu_seqlens_q = group_starts;
  a.context_lens = group_prefix_lens;
  a.num_seqs = num_groups;
  a.total_q = num_seqs;
  a.max_q_len = max_group_size;
  a.max_blocks = max_blocks_per_seq;
  a.num_blocks = num_blocks;
  a.block_size = block_size;
  a.block_size_log2 = __builtin_ctz((unsigned)block_size);
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = group;
  a.max_ctx = max_prefix_len;
  a.scale_log2 = scale * pkv::kLog2e;
  a.causal = 0;
  a.table_row_is_first_q = 1;
  a.part_m = part_m;
  a.part_l = part_l;
  a.part_o = part_o;
  a.seq_prefix = seq_prefix;
  a.k_scale = a.v_scale = nullptr;
  if (hipError_t e = pkv::launch_prefill(a, head_dim, st); e != hipSuccess) return hip_status(e, fn);

  // second pass: each sequence's own tokens, merged with its prefix partials
  pkv::DecodeParams b;
  b.out = out;
  b.q = q;
  b.k_cache = k_cache;
  b.v_cache = v_cache;
  b.block_tables = block_tables;
  b.context_lens = context_lens;
  b.num_seqs = num_seqs;
  b.max_blocks = max_blocks_per_seq;
  b.num_blocks = num_blocks;
  b.block_size = block_size;
  b.num_q_heads = num_q_heads;
  b.num_kv_heads = num_kv_heads;
  b.group = group;
  b.scale_log2 = scale * pkv::kLog2e;
  b.max_ctx = max_context_len;
  int32_t part;
  int64_t nparts;
  partitioning(max_context_len, 0, &part, &nparts);
  b.partition_size = part;
  b.num_partitions = 1;
  b.ws_m = b.ws_l = b.ws_o = nullptr;
  b.part_counters = nullptr;
  b.k_new = b.v_new = nullptr;
  b.new_slots = nullptr;
  b.seq_prefix = seq_prefix;
  b.pre_m = part_m;
  b.pre_l = part_l;
  b.pre_o = part_o;
  b.k_scale = b.v_scale = nullptr;
  b.bal_counters = nullptr;
  b.bal_pieces = nullptr;
  b.bal_piece_stride = 0;
  b.pair_span = 0;
  b.plan = nullptr;
  return hip_status(pkv::launch_decode_mfma(b, head_dim, st), fn);
}

extern "C" int pkv_check_paged_inputs(const int32_t* block_tables, const int32_t* context_lens,
                                      const int32_t* cu_seqlens_q, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int32_t max_context_len, int32_t total_q,
                                      int32_t max_q_len, int32_t num_blocks, int32_t block_size,
                                      int32_t* report, void* stream) {
  const char* fn = "pkv_check_paged_inputs";
  if (num_seqs < 0 || total_q < 0 || max_q_len < 0) return fail(PKV_EINVAL, "%s: negative size", fn);
  if (num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
    return fail(PKV_EINVAL, "%s: num_blocks, block_size and max_blocks_per_seq must be positive", fn);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return fail(PKV_EINVAL, "%s: max_context_len outside [0, max_blocks_per_seq * block_size]", fn);
  if (!report || !aligned(report, 4)) return fail(PKV_EINVAL, "%s: report must be a 4-byte aligned device array", fn);
  if (num_seqs > 0 && (!block_tables || !context_lens)) return fail(PKV_EINVAL, "%s: null pointer", fn);
  if (!aligned(block_tables, 4) || !aligned(context_lens, 4) || !aligned(cu_seqlens_q, 4))
    return fail(PKV_EINVAL, "%s: index arrays must be 4-byte aligned", fn);
  pkv::CheckParams p;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.cu_seqlens_q = cu_seqlens_q;
  p.num_seqs = num_seqs;
  p.max_blocks = max_blocks_per_seq;
  p.max_ctx = max_context_len;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.total_q = total_q;
  p.max_q_len = max_q_len;
  p.report = report;
  return hip_status(pkv::launch_check_tables(p, (hipStream_t)stream), fn);
}

extern "C" size_t pkv_check_slots_workspace_size(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return 0;
  const int64_t words = ((int64_t)num_blocks * block_size + 31) / 32;
  return (size_t)(2 * words * 4);
}

extern "C" int pkv_check_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                               int32_t block_size, void* workspace, size_t workspace_bytes, int32_t* report,
                               void* stream) {
  const char* fn = "pkv_check_slots";
  if (num_tokens < 0) return fail(PKV_EINVAL, "%s: num_tokens < 0", fn);
  if (num_blocks <= 0 || block_size <= 0)
    return fail(PKV_EINVAL, "%s: num_blocks and block_size must be positive", fn);
  if (!report || !aligned(report, 4)) return fail(PKV_EINVAL, "%s: report must be a 4-byte aligned device array", fn);
  if (num_tokens > 0 && !slot_mapping) return fail(PKV_EINVAL, "%s: null slot_mapping", fn);
  if (!aligned(slot_mapping, 4)) return fail(PKV_EINVAL, "%s: slot_mapping must be 4-byte aligned", fn);
  const size_t need = pkv_check_slots_workspace_size(num_blocks, block_size);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EWORKSPACE, "%s: needs %zu workspace bytes, got %zu", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned(workspace, 4)) return fail(PKV_EINVAL, "%s: workspace must be 4-byte aligned", fn);
  pkv::SlotCheckParams p;
  const int64_t words = ((int64_t)num_blocks * block_size + 31) / 32;
  p.slot_mapping = slot_mapping;
  p.num_tokens = num_tokens;
  p.num_slots = (int64_t)num_blocks * block_size;
  p.seen = reinterpret_cast<uint32_t*>(workspace);
  p.dup = p.seen + words;
  p.report = report;
  return hip_status(pkv::launch_check_slots(p, (hipStream_t)stream), fn);
}
