/*
 * pkv.h -- C ABI of the paged-KV attention library for MI355X (gfx950).
 *
 * Attention over a paged KV cache: the keys and values of every sequence live
 * in fixed-size token blocks of one shared pool ("Building a minimal vLLM
 * implementation", section config.py, kvcache_block_size), and each sequence
 * reaches its blocks through a block table that maps logical blocks to
 * physical ones (same page, section sequence.py, block_table). The pool's
 * blocks are numbered 0..num_blocks-1 ("Implementation Details", section
 * "PagedAttention -- BlockPool"). Decode runs one query row per sequence;
 * prefill runs chunks of query rows after the tokens already cached (section
 * sequence.py, num_cached_tokens). Both compute exactly what naive softmax
 * attention over the gathered K/V computes ("A vLLM engine small enough to
 * read in one sitting", sections "What it does" and "The interesting bit").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All tensor pointers are DEVICE pointers owned by the caller; the library
 *    keeps no pointer after a call returns and allocates nothing (the one
 *    piece of device memory it owns is the static decode scratch below).
 *  - Layouts are dense and row-major:
 *        q, out (decode)     [num_seqs, num_q_heads, head_dim]
 *        q, out (prefill)    [total_q,  num_q_heads, head_dim]   (packed chunks)
 *        k, v (new rows)     [num_tokens, num_kv_heads, head_dim]
 *        k_cache, v_cache    [num_blocks, block_size, num_kv_heads, head_dim]
 *        block_tables        int32 [num_seqs, max_blocks_per_seq]
 *        context_lens        int32 [num_seqs]
 *        slot_mapping        int32 [num_tokens]
 *        cu_seqlens_q        int32 [num_seqs + 1]
 *  - Position p of sequence s lives in physical block
 *    block_tables[s][p / block_size], row p % block_size. Table entries past
 *    ceil(context_lens[s] / block_size) may hold anything: their values never
 *    decide which cache memory is read (a kernel may load such an entry of
 *    the row, ahead of knowing the length, and then discard it), and nothing
 *    past the row's max_blocks_per_seq entries is ever loaded.
 *  - context_lens[s] counts every token of the sequence whose K/V is in the
 *    cache, including the rows stored in the same step; 0 yields zero output.
 *  - GQA: q-head h reads kv-head h / (num_q_heads / num_kv_heads).
 *  - Logits are scale * (q . k); softmax and accumulation run in fp32; the
 *    output has the dtype of q and is rounded to nearest-even once.
 *  - q, caches, new rows and out share one dtype (PKV_F32 or PKV_BF16).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream) and never synchronizes. The host never reads device memory:
 *    values held in device arrays (block ids, lengths, slots) are the
 *    caller's contract; kernels skip slots and block rows outside the pool
 *    rather than touching memory out of bounds.
 *  - Return value: PKV_OK, or a negative pkv_status with a message available
 *    from pkv_last_error() in the calling thread. Invalid arguments are
 *    reported before anything is launched. No exception crosses the ABI and
 *    nothing aborts.
 *  - out must not alias q or the caches. The store writes the caches in place.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = -1,        /* bad pointer, size, or inconsistent arguments */
  PKV_EUNSUPPORTED = -2,  /* valid request outside what the kernels implement */
  PKV_EWORKSPACE = -3,    /* split-K workspace missing or too small */
  PKV_EHIP = -4           /* the HIP runtime reported an error at launch */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

/* Decode kernel family. AUTO picks the matrix-core kernel for bf16 and the
 * vector kernel for fp32. */
typedef enum {
  PKV_DECODE_AUTO = 0,
  PKV_DECODE_VALU = 1,    /* vector FMA dot products, lane-shuffle reductions */
  PKV_DECODE_MFMA = 2     /* GQA group packed into matrix-core tiles (bf16 only) */
} pkv_decode_algo;

/* partition_size values selecting the work-balanced decode and the planned
 * decode (see pkv_paged_attention_decode and pkv_decode_plan). */
enum { PKV_PARTITION_BALANCED = -1, PKV_PARTITION_PLANNED = -2, PKV_PARTITION_AUTO = -3 };

/* Library version as major*10000 + minor*100 + patch. */
int pkv_version(void);

/* Message describing the last non-OK status returned in this thread. */
const char* pkv_last_error(void);

/*
 * kv_cache_store: writing the new tokens' K/V rows into the blocks that the
 * block table assigns them ("Building a minimal vLLM implementation", section
 * sequence.py: the block table maps a sequence's logical blocks to physical
 * ones, and the last block is filled token by token). A slot names one pool
 * row, slot = physical block * block_size + row. For every token t with
 * 0 <= slot_mapping[t] < num_blocks * block_size, copy k[t] into k_cache row
 * (slot / block_size, slot % block_size) and v[t] into the same row of v_cache. Negative slots are
 * padding and write nothing; slots past the pool are skipped. The copy is
 * bit-exact. Two tokens naming the same slot race (the result is one of
 * them); callers keep slots unique.
 *   num_tokens >= 0 (0 launches nothing); num_blocks, block_size,
 *   num_kv_heads, head_dim > 0; num_kv_heads * head_dim * dtype size must be
 *   a multiple of 16 bytes.
 */
int pkv_kv_cache_store(const void* k, const void* v, void* k_cache, void* v_cache,
                       const int32_t* slot_mapping, int32_t num_tokens,
                       int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                       int32_t head_dim, pkv_dtype dtype, void* stream);

/*
 * Bytes of workspace needed by pkv_paged_attention_decode for the same
 * num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len and
 * partition_size (0 for invalid sizes).
 *  Every mode that merges partial results keeps its arrival counters in one
 *  counter block, the first 256 KiB (65536 int32) of the workspace, and its
 *  partial results after it; every call leaves the whole block zero, so one
 *  workspace serves calls of any mode and size in turn.
 *  - partition_size > 0 (split-K): the counter block (counter
 *    s * num_kv_heads + g), then fp32 running max, sum and unnormalised
 *    output for every (sequence, q-head, partition); 0 when one partition
 *    covers max_context_len. Layout after the counters: m [num_seqs, num_q_heads, P],
 *    l [num_seqs, num_q_heads, P], o [num_seqs, num_q_heads, P, head_dim],
 *    P = ceil(max_context_len / partition_size). Split-K takes at most
 *    65536 (sequence, kv-head) pairs.
 *  - PKV_PARTITION_BALANCED: the counter block (its first 4096 counters, one
 *    per wave of the largest grid), then fp32 pieces of the partial results,
 *    two per wave of that grid (4096 waves).
 *  - PKV_PARTITION_PLANNED: pkv_decode_plan_size(num_seqs) (the plan).
 *  - PKV_PARTITION_AUTO: the larger of those of the choices it stands for
 *    (pkv_decode_auto_partition, and its split-K fallback).
 *  - 0 (single pass): 0.
 * The counter block must be zero before a workspace's first split-K or
 * work-balanced call: pkv_decode_workspace_init clears it.
 */
size_t pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_size);

/*
 * Zero the counter block at the start of a decode workspace (its first
 * min(workspace_bytes, 256 KiB) bytes, which hold the split-K and the
 * work-balanced counters), with a kernel on `stream`: no memset, so the call
 * may be captured in a graph. The rest of the workspace is scratch and needs
 * no initial contents. Call it once on a new workspace (e.g. from
 * torch.empty) or after a call that did not run to completion.
 *   workspace: 4-byte aligned device buffer (NULL allowed when
 *   workspace_bytes is 0).
 */
int pkv_decode_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * The partition_size that PKV_PARTITION_AUTO resolves to on the current
 * device, from host-side sizes only (C = the device's compute units, items =
 * num_seqs * num_kv_heads):
 *  - 0 (one pass) when items >= 2C or max_context_len <= 2048;
 *  - PKV_PARTITION_BALANCED when 2 * items >= C (and the work-balanced
 *    limits hold: at most 8192 sequences, fewer than 2^30 tiles). A call the
 *    work-balanced decode does not take (fp32 caches or the VALU kernel,
 *    E4M3 caches) splits instead, at the size of the next rule;
 *  - otherwise split-K at the power of two in [512, 2048] nearest above
 *    items * max_context_len / C tokens (about one partition per compute
 *    unit), or 0 when one partition holds max_context_len.
 * 0 for invalid sizes.
 */
int32_t pkv_decode_auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_context_len);

/*
 * Decode plan: the sequences of one decode step in order of their number of
 * 16-token tiles (ceil(min(context_lens[s], max_context_len) / 16), capped
 * at 2047), largest first, ties by sequence index, for a single-pass decode
 * whose workgroups then start their long items first and pair long with
 * short ones on each compute unit without ranking the batch themselves.
 * Every layer of a step shares one block table and one set of lengths, so
 * one plan serves all the layers' decode calls (pass partition_size =
 * PKV_PARTITION_PLANNED and the plan as `workspace`).
 *   plan: device buffer of pkv_decode_plan_size(num_seqs) bytes, 16-byte
 *     aligned, owned by the caller. Entry r (8 int32): the r-th sequence s,
 *     its context_lens value, the table entries block_tables[s][(16 w) /
 *     block_size] (w = 0..3, capped at the row's last entry), 0, 0.
 *   The other arguments are those of pkv_paged_attention_decode. One
 *   workgroup, asynchronous on `stream`. The plan describes context_lens and
 *   block_tables as they are when it runs: make a new plan whenever either
 *   changes. A decode whose plan does not match them (a sequence's length or
 *   first blocks differ) writes that sequence's rows as NaN; whether a fused
 *   store then wrote its new row is unspecified.
 * Supported: num_seqs <= 65535, block_size a multiple of 16 up to 256.
 */
size_t pkv_decode_plan_size(int32_t num_seqs);
int pkv_decode_plan(void* plan, size_t plan_bytes, const int32_t* block_tables,
                    const int32_t* context_lens, int32_t num_seqs, int32_t max_blocks_per_seq,
                    int32_t max_context_len, int32_t block_size, void* stream);

/*
 * paged_attention_decode: the decode step's attention, one query row per
 * sequence (in decode a sequence carries only its newest token: "Building a
 * minimal vLLM implementation", section sequence.py, the state sent to
 * workers), over K/V gathered through its block table (same section,
 * block_table); the same function naive attention computes ("A vLLM engine
 * small enough to read in one sitting", sections "What it does" and "The
 * interesting bit"): out[s, h] = softmax_j(scale * q[s, h] . K_s[j, g])
 * . V_s[j, g] over positions j < context_lens[s], g = h / (Hq / Hkv), with
 * K_s, V_s gathered through block_tables[s].
 *   max_context_len: a host-side bound >= every context_lens[s] and <=
 *     max_blocks_per_seq * block_size; it sizes the grid and the workspace.
 *     A device length above it breaks the contract and is truncated to it.
 *   partition_size: 0 runs one pass per (sequence, kv-head). Otherwise a
 *     positive multiple of 16: each (sequence, kv-head) is split into
 *     partitions of that many tokens whose partial results (running max,
 *     sum, unnormalised output) go to `workspace`; the partition that
 *     finishes last, found with the workspace's arrival counters, merges
 *     them (log-sum-exp) in the same launch. The counters must be zero
 *     before the first call (e.g. a zero-filled workspace); every call leaves
 *     them zero, so one workspace serves calls of any sizes, and of the
 *     work-balanced mode, in turn, but calls that run at the same time must
 *     not share it. Sequences that fit
 *     in one partition are written directly.
 *     PKV_PARTITION_BALANCED (MFMA kernel, bf16, at most 8192 sequences,
 *     fewer than 2^30 16-token tiles): one launch whose grid fills the GPU
 *     once; every wave takes an equal share of all (kv-head, sequence,
 *     16-token tile) work, so the time no longer follows the longest
 *     context. A (sequence, kv-head) split between waves is merged
 *     (log-sum-exp) in the same launch by the wave that finishes its part
 *     last, found with atomic counters in the first 16 KiB of `workspace`.
 *     Those must be zero before the first call (e.g. a zero-filled
 *     workspace); every call leaves them zero, so one workspace serves calls
 *     of any sizes, and of the split-K mode, in turn, but calls that run at
 *     the same time must not share it. out must be 16-byte aligned.
 *     PKV_PARTITION_PLANNED (MFMA kernel; bf16 or E4M3 caches): one pass per
 *     (sequence, kv-head), with the items handed out in the order of the
 *     plan that pkv_decode_plan wrote into `workspace` for the same
 *     num_seqs, context_lens and block_tables (workspace_bytes >=
 *     pkv_decode_plan_size(num_seqs)). The results are those of
 *     partition_size 0.
 *     PKV_PARTITION_AUTO: the choice pkv_decode_auto_partition returns for
 *     these sizes (one pass, work-balanced or split-K), with its workspace.
 *   workspace / workspace_bytes: device buffer of at least
 *     pkv_decode_workspace_size(...) bytes (may be NULL when that is 0),
 *     256-byte aligned for PKV_PARTITION_BALANCED.
 *   algo: pkv_decode_algo. The MFMA kernel needs bf16 and
 *     num_q_heads / num_kv_heads <= 16; the VALU kernel takes groups up to
 *     16 for fp32 and up to 8 for bf16 (PKV_DECODE_AUTO picks MFMA for bf16,
 *     VALU for fp32, so every group up to 16 runs in the default mode).
 * Supported: head_dim in {64, 128}; block_size a multiple of 16 up to 256;
 * num_q_heads / num_kv_heads <= 16.
 */
int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t max_blocks_per_seq, int32_t max_context_len,
                               int32_t num_blocks, int32_t block_size,
                               int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, float scale, int32_t partition_size,
                               void* workspace, size_t workspace_bytes,
                               pkv_dtype dtype, int32_t algo, void* stream);

/*
 * paged_attention_decode_store: kv_cache_store of one new row per sequence
 * followed by paged_attention_decode, in one launch. For each sequence s
 * with 0 <= slot_mapping[s] < num_blocks * block_size, k_new[s] and v_new[s]
 * ([num_seqs, num_kv_heads, head_dim], the dtype of q) are written to that
 * slot of k_cache / v_cache, and decode then sees them as the sequence's
 * newest token. Precondition (the usual decode step): slot_mapping[s] is the
 * slot of position context_lens[s] - 1 under block_tables[s]; the kernel
 * uses the new row for that position straight from k_new / v_new. A negative
 * slot stores nothing and leaves position ctx-1 as the cache holds it. The
 * other arguments, the results and the errors are those of
 * pkv_paged_attention_decode; k_new, v_new and slot_mapping must be non-null
 * (slot_mapping 4-byte, the rows 16-byte aligned).
 */
int pkv_paged_attention_decode_store(void* out, const void* q, void* k_cache, void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     const void* k_new, const void* v_new,
                                     const int32_t* slot_mapping, int32_t num_seqs,
                                     int32_t max_blocks_per_seq, int32_t max_context_len,
                                     int32_t num_blocks, int32_t block_size,
                                     int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, float scale, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes,
                                     pkv_dtype dtype, int32_t algo, void* stream);

/*
 * paged_attention_decode_static: pkv_paged_attention_decode for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc). It takes no workspace and calls no
 * allocating routine: the split-K and work-balanced modes keep their partial
 * results and arrival counters in a scratch array that the library holds on
 * each device it runs on (PKV_STATIC_SCRATCH_BYTES, created with the
 * library's device code on that device and held until the process ends).
 * Each call first clears the arrival counters it uses, with a kernel on
 * `stream`, then runs the decode; its results are those of
 * pkv_paged_attention_decode with the same arguments and a workspace.
 *   partition_size: 0, a positive multiple of 16, PKV_PARTITION_BALANCED or
 *   PKV_PARTITION_AUTO (PKV_PARTITION_PLANNED reads a caller's plan:
 *   PKV_EINVAL).
 * Errors: those of pkv_paged_attention_decode, and PKV_EWORKSPACE, before any
 * launch, when pkv_decode_workspace_size(...) for these arguments exceeds
 * PKV_STATIC_SCRATCH_BYTES.
 * Every call on a device shares that device's scratch, which keeps the last
 * call's contents: calls that overlap in time on one device (on different
 * streams, or from threads without ordering between them) race and give
 * unspecified results. Calls on one stream are ordered and safe.
 */
#define PKV_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
int pkv_paged_attention_decode_static(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                                      int32_t num_kv_heads, int32_t head_dim, float scale,
                                      int32_t partition_size, pkv_dtype dtype, int32_t algo,
                                      void* stream);

/*
 * E4M3 KV cache. The pages list support for quantized models among vLLM's
 * features ("Building a minimal vLLM implementation", the feature list that
 * opens the page) and fix nothing further; the format and scaling are this
 * library's reading. Cache elements are OCP FP8 E4M3 codes (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, no infinity, 0x7f/0xff NaN, largest finite
 * 448) in the same [num_blocks, block_size, num_kv_heads, head_dim] layout,
 * one byte each. k_scale and v_scale are device float32 arrays
 * [num_kv_heads]: a code c of kv-head g stands for value(c) * scale[g].
 *
 * kv_cache_store_fp8: like pkv_kv_cache_store, but each element x of k / v
 * (src_dtype bf16 or fp32, [num_tokens, num_kv_heads, head_dim], 16-byte
 * aligned) is stored as the code of t = x / scale[g] (one IEEE float32
 * division), rounded to nearest with ties to the even code, saturated to
 * +-448; a NaN is stored as 0x7f. The result is bit-exact. Slots as in
 * pkv_kv_cache_store (negative: no write; past the pool: skipped).
 * head_dim must be a multiple of 8; caches 8-byte aligned.
 */
int pkv_kv_cache_store_fp8(const void* k, const void* v, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, const float* k_scale, const float* v_scale,
                           int32_t num_tokens, int32_t num_blocks, int32_t block_size,
                           int32_t num_kv_heads, int32_t head_dim, pkv_dtype src_dtype,
                           void* stream);

/*
 * paged_attention_decode_fp8: pkv_paged_attention_decode over E4M3 caches
 * (values dequantised with k_scale / v_scale), q and out bf16, on the MFMA
 * kernel. partition_size 0 or a positive multiple of 16 (split-K, with the
 * same workspace); the work-balanced mode is not offered here. The other
 * arguments, results and errors are those of pkv_paged_attention_decode.
 */
int pkv_paged_attention_decode_fp8(void* out, const void* q, const void* k_cache,
                                   const void* v_cache, const float* k_scale, const float* v_scale,
                                   const int32_t* block_tables, const int32_t* context_lens,
                                   int32_t num_seqs, int32_t max_blocks_per_seq,
                                   int32_t max_context_len, int32_t num_blocks, int32_t block_size,
                                   int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   float scale, int32_t partition_size, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * paged_attention_decode_store_fp8: pkv_kv_cache_store_fp8 of one new row
 * per sequence (bf16 k_new / v_new [num_seqs, num_kv_heads, head_dim],
 * quantised exactly as that call does) followed by
 * pkv_paged_attention_decode_fp8, in one launch, under the precondition and
 * slot rules of pkv_paged_attention_decode_store. The codes of the new row
 * are used for position ctx-1 straight from the quantisation.
 */
int pkv_paged_attention_decode_store_fp8(void* out, const void* q, void* k_cache, void* v_cache,
                                         const float* k_scale, const float* v_scale,
                                         const int32_t* block_tables, const int32_t* context_lens,
                                         const void* k_new, const void* v_new,
                                         const int32_t* slot_mapping, int32_t num_seqs,
                                         int32_t max_blocks_per_seq, int32_t max_context_len,
                                         int32_t num_blocks, int32_t block_size,
                                         int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, float scale, int32_t partition_size,
                                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Shared-prefix decode. With prefix caching, sequences that start from the
 * same prompt share its blocks ("Implementation Details", section "Getting
 * Started": serving with prefix caching enabled; section "PagedAttention --
 * BlockPool": a hash table looks up cached blocks by content, and blocks
 * carry reference counts). This
 * decode reads each shared block once per group instead of once per
 * sequence; its result is that of pkv_paged_attention_decode.
 *
 * Sequences are split into num_groups groups of consecutive sequences:
 * group j is sequences group_starts[j] .. group_starts[j+1]-1 (device int32
 * [num_groups + 1], group_starts[0] = 0, group_starts[num_groups] =
 * num_seqs; every sequence in exactly one group, singletons allowed). Its
 * members share their first group_prefix_lens[j] tokens (device int32
 * [num_groups]): a multiple of block_size (and of 16), at most every
 * member's context length, with the same physical blocks in every member's
 * block table (the first member's entries are the ones read). An unshared
 * sequence is a group of one with prefix length 0.
 *   max_group_size >= every group's size; max_prefix_len >= every prefix
 *   length, <= max_context_len (host bounds for the grids).
 * Two launches on `stream`: the groups' query rows over their prefixes (the
 * prefill kernel, one non-causal chunk per group), writing fp32 partials to
 * `workspace`; then decode over each sequence's remaining tokens, merged
 * with its partials. A prefix length that is not a multiple of 16 or exceeds
 * the context gives NaN rows; other violations give unspecified values.
 *   workspace: pkv_decode_shared_prefix_workspace_size(...) bytes, 16-byte
 *   aligned: m, l [num_seqs, num_q_heads], o [num_seqs, num_q_heads,
 *   head_dim] fp32, then int32 [num_seqs]; scratch, no initial contents.
 * Supported: bf16, head_dim 128, GQA group in {1, 2, 4, 8, 16}, block_size a
 * power of two in [16, 256], num_blocks * block_size < 2^32.
 */
size_t pkv_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim);
int pkv_paged_attention_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_tables,
                                             const int32_t* context_lens,
                                             const int32_t* group_starts,
                                             const int32_t* group_prefix_lens, int32_t num_groups,
                                             int32_t max_group_size, int32_t max_prefix_len,
                                             int32_t num_seqs, int32_t max_blocks_per_seq,
                                             int32_t max_context_len, int32_t num_blocks,
                                             int32_t block_size, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, float scale,
                                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_prefill_chunk: attention of packed query chunks over their
 * paged contexts: the prefill of a sequence whose first tokens are already
 * cached ("Building a minimal vLLM implementation", section sequence.py,
 * num_cached_tokens and num_scheduled_tokens), computing what naive causal
 * attention computes, as the pages' flash-attention prefill does ("A vLLM
 * engine small enough to read in one sitting", section "What it does"). Chunk c owns q rows cu_seqlens_q[c] .. cu_seqlens_q[c+1]-1
 * (L_c rows); context_lens[c] >= L_c counts its cached tokens plus its own
 * L_c rows, whose K/V must already be stored. Row i of chunk c sits at
 * position P0 + i with P0 = context_lens[c] - L_c and, when causal != 0,
 * attends to positions 0 .. P0 + i; otherwise to all context_lens[c]
 * positions.
 *   total_q: rows of q and out; max_q_len >= every L_c (sizes the grid);
 *   max_context_len >= every context_lens[c], <= max_blocks_per_seq * block_size.
 * Supported: bf16, head_dim 128, block_size a power of two in [16, 256],
 * num_q_heads / num_kv_heads in {1, 2, 4, 8, 16}, num_blocks * block_size < 2^32
 * (PKV_EUNSUPPORTED otherwise).
 */
int pkv_paged_attention_prefill_chunk(void* out, const void* q, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables,
                                      const int32_t* cu_seqlens_q,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t total_q, int32_t max_q_len,
                                      int32_t max_blocks_per_seq, int32_t max_context_len,
                                      int32_t num_blocks, int32_t block_size,
                                      int32_t num_q_heads, int32_t num_kv_heads,
                                      int32_t head_dim, float scale, int32_t causal,
                                      pkv_dtype dtype, void* stream);

/*
 * paged_attention_prefill_chunk_fp8: paged_attention_prefill_chunk over E4M3
 * caches (the format, scales and dequantisation of paged_attention_decode_fp8;
 * cache rows as written by kv_cache_store_fp8). Quantized-model support is in
 * the feature list that opens "Building a minimal vLLM implementation"; the
 * attention is the chunked-prefill definition above applied to the
 * dequantised rows.
 *   q, out: bf16 [total_q, num_q_heads, head_dim]; k_cache, v_cache: uint8
 *   codes [num_blocks, block_size, num_kv_heads, head_dim]; k_scale, v_scale:
 *   float32 [num_kv_heads] on the device (a row's values are code * scale).
 * Supported and errors as paged_attention_prefill_chunk, plus PKV_EINVAL for a
 * null or misaligned scale pointer.
 */
int pkv_paged_attention_prefill_chunk_fp8(void* out, const void* q, const void* k_cache,
                                          const void* v_cache, const float* k_scale,
                                          const float* v_scale, const int32_t* block_tables,
                                          const int32_t* cu_seqlens_q, const int32_t* context_lens,
                                          int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                          int32_t max_blocks_per_seq, int32_t max_context_len,
                                          int32_t num_blocks, int32_t block_size, int32_t num_q_heads,
                                          int32_t num_kv_heads, int32_t head_dim, float scale,
                                          int32_t causal, void* stream);

/*
 * Checks of device-held inputs, for debugging. The attention and store entry
 * points never read block ids, lengths or slots on the host; kernels skip or
 * poison what is out of range (a block id outside the pool turns that row's
 * output into NaN, a slot outside the pool writes nothing, a length above
 * max_context_len is truncated) and two tokens storing to one slot race.
 * These calls count such violations into `report` (a device int32[4] owned
 * by the caller, overwritten) with kernels on `stream`, touching nothing out
 * of bounds; the caller copies the report back when it wants to look.
 *
 * check_paged_inputs, for a decode (cu_seqlens_q NULL) or a chunked prefill:
 *   report[0]: sequences with context_lens[s] outside [0, max_context_len];
 *   report[1]: entries among the first ceil(min(max(ctx, 0), max_context_len)
 *              / block_size) of each table row outside [0, num_blocks) (the
 *              pool's blocks, "Implementation Details", section
 *              "PagedAttention -- BlockPool");
 *   report[2]: chunks c whose row count L = cu_seqlens_q[c+1] - cu_seqlens_q[c]
 *              is negative, above max_q_len or above context_lens[c], plus
 *              cu_seqlens_q[0] != 0 and cu_seqlens_q[num_seqs] != total_q
 *              (counted on the first and last chunk);
 *   report[3]: the lowest sequence index with any of these, or num_seqs.
 *   Arguments as in the attention calls (total_q and max_q_len are read only
 *   with cu_seqlens_q).
 */
int pkv_check_paged_inputs(const int32_t* block_tables, const int32_t* context_lens,
                           const int32_t* cu_seqlens_q, int32_t num_seqs, int32_t max_blocks_per_seq,
                           int32_t max_context_len, int32_t total_q, int32_t max_q_len,
                           int32_t num_blocks, int32_t block_size, int32_t* report, void* stream);

/*
 * check_slots, for a kv_cache_store (or a fused store) call:
 *   report[0]: tokens whose slot is >= num_blocks * block_size;
 *   report[1]: repeated claims: a slot named by k tokens adds k - 1;
 *   report[2]: negative slots (padding: allowed, counted for information);
 *   report[3]: the lowest token index whose slot is past the pool or named
 *              more than once, or num_tokens.
 *   workspace: pkv_check_slots_workspace_size(num_blocks, block_size) bytes,
 *   4-byte aligned (two bitmaps of one bit per pool row; no initial contents).
 */
size_t pkv_check_slots_workspace_size(int32_t num_blocks, int32_t block_size);
int pkv_check_slots(const int32_t* slot_mapping, int32_t num_tokens, int32_t num_blocks,
                    int32_t block_size, void* workspace, size_t workspace_bytes, int32_t* report,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
