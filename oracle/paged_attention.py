"""CPU float64 oracle for attention over a paged KV cache.

TEST INFRASTRUCTURE. Only the test suite, the smoke check and the CPU-baseline
leg of the benchmark may import, call or execute anything in this package. The
product path (the HIP library and its Python binding) never does, and this
package imports nothing from it: the two share no kernels, headers, helpers,
tables or pre/post-processing.

What is computed, and where it comes from
-----------------------------------------
The pages describe "paged attention": a sequence's keys and values live in
fixed-size token blocks of a shared pool ("Building a minimal vLLM
implementation", section config.py, ``kvcache_block_size``), and each sequence
owns a block table that maps its logical blocks to physical blocks (same page,
section sequence.py, ``block_table``; the pool of physical blocks numbered
0..num_gpu_blocks-1 is "Implementation Details", section "PagedAttention --
BlockPool"). The optimised kernels the pages mention (flash attention for
prefill, paged attention for decode) are presented as faster, less
memory-hungry routes to the very function that naive O(N^2) attention computes
("A vLLM engine small enough to read in one sitting", sections "What it does",
"The interesting bit" and "Key highlights"). The oracle is therefore that plain
definition, written out directly:

  * store   -- copy each new K/V row into the cache row its slot names;
  * gather  -- logical position p of a sequence lives in physical block
               block_table[p // block_size], row p % block_size;
  * attend  -- softmax(scale * q . K^T) . V over the gathered rows, in float64,
               with GQA grouping (q-head h reads kv-head h // (Hq / Hkv)) and,
               for a prefill chunk, a causal mask aligned to the chunk's end.

No blocking, split-K, online softmax or reduced-precision step appears here:
those are re-associations the GPU path may use, and they may change the result
only by rounding.

Readings taken where the pages are silent (the pages fix none of these):
  * cache layout [num_blocks, block_size, kv_heads, head_dim], row-major;
  * slot s names physical row (s // block_size, s % block_size); s < 0 skips;
  * context_lens count the tokens stored in the same step (a decode token sits
    at position ctx-1, a prefill chunk of L rows at ctx-L .. ctx-1);
  * an empty context (ctx == 0) yields a zero output row;
  * the causal mask of a chunk is bottom-right aligned: row i of an L-row chunk
    sees keys 0 .. ctx-L+i; all earlier (cached) tokens are visible.

Data formats accepted: float64, float32, or bfloat16 given as its raw 16-bit
patterns in a uint16 array (upcast exactly: bf16 is the top half of an fp32).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "to_f64",
    "kv_cache_store",
    "gather_context",
    "attend_rows",
    "paged_attention_decode",
    "paged_attention_prefill_chunk",
]


def to_f64(x: np.ndarray) -> np.ndarray:
    """Exact upcast of stored values to float64.

    uint16 input is read as bfloat16 bit patterns: a bf16 value is the upper
    16 bits of the fp32 with the same sign, exponent and leading mantissa bits,
    so shifting left by 16 reproduces it exactly.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported storage dtype {x.dtype}")


def kv_cache_store(k, v, k_cache, v_cache, slot_mapping, block_size):
    """Write new K/V rows into their cache slots; returns updated copies.

    The caches are the block pool of "Implementation Details", section
    "PagedAttention -- BlockPool" (one entry per physical block), each block
    holding block_size token rows ("Building a minimal vLLM implementation",
    section config.py). Token t goes to physical block slot // block_size, row
    slot % block_size; a negative slot means "no write" (padding). The copy is
    of raw storage, so it is bit-exact for every dtype. Two tokens naming the
    same slot have no single correct result, so that is rejected.
    """
    k = np.asarray(k)
    v = np.asarray(v)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    num_blocks = kc.shape[0]
    assert kc.shape[1] == block_size and vc.shape == kc.shape
    assert k.shape[0] == v.shape[0] == len(slot_mapping)
    assert k.shape[1:] == kc.shape[2:] and v.shape[1:] == vc.shape[2:]
    seen = set()
    for t, slot in enumerate(np.asarray(slot_mapping).tolist()):
        if slot < 0:
            continue
        if slot >= num_blocks * block_size:
            raise IndexError(f"slot {slot} outside a pool of {num_blocks} blocks")
        if slot in seen:
            raise ValueError(f"slot {slot} written twice in one call")
        seen.add(slot)
        block, row = divmod(slot, block_size)
        kc[block, row] = k[t]
        vc[block, row] = v[t]
    return kc, vc


def gather_context(cache, block_table, context_len, block_size):
    """Rows of logical positions 0..context_len-1 of one sequence, in order.

    "Building a minimal vLLM implementation", section sequence.py: the block
    table maps logical blocks to physical locations, and a sequence tracks how
    many blocks it uses and how full the last one is. Position p is therefore
    in logical block p // block_size at offset p % block_size. Table entries
    past the last used logical block are never read. Returns float64
    [context_len, kv_heads, head_dim].
    """
    positions = np.arange(int(context_len))
    table = np.asarray(block_table)
    physical = table[positions // block_size]
    return to_f64(np.asarray(cache)[physical, positions % block_size])


def attend_rows(q_rows, keys, values, scale, visible):
    """Softmax attention of query rows over key/value rows, float64.

    q_rows [n, D], keys/values [L, D]; visible[i] is how many leading keys row
    i may see (0 gives a zero row). out_i = sum_j w_ij v_j / sum_j w_ij with
    w_ij = exp(scale * q_i . k_j - max_j'(scale * q_i . k_j')) over j < visible[i].
    Subtracting the row maximum leaves the ratio unchanged and keeps exp finite.
    """
    n, d = q_rows.shape
    out = np.zeros((n, values.shape[1]), dtype=np.float64)
    for i in range(n):
        m = int(visible[i])
        if m == 0:
            continue
        logits = scale * (keys[:m] @ q_rows[i])
        w = np.exp(logits - logits.max())
        out[i] = (w @ values[:m]) / w.sum()
    return out


def _check_heads(num_q_heads, num_kv_heads):
    if num_kv_heads <= 0 or num_q_heads % num_kv_heads != 0:
        raise ValueError("q heads must be a positive multiple of kv heads")
    return num_q_heads // num_kv_heads


def paged_attention_decode(q, k_cache, v_cache, block_tables, context_lens,
                           scale, block_size):
    """Decode attention: one query row per sequence over its paged context.

    In decode a sequence carries only its newest token ("Building a minimal
    vLLM implementation", section sequence.py, the state shipped to workers),
    so each sequence contributes one query row per q-head. q [S, Hq, D]; the
    caches [NB, block_size, Hkv, D]; block_tables [S, MB]; context_lens [S]
    (including the token stored this step). q-head h reads kv-head h // G,
    G = Hq / Hkv. Returns float64 [S, Hq, D].
    """
    qf = to_f64(q)
    num_seqs, num_q_heads, head_dim = qf.shape
    num_kv_heads = np.asarray(k_cache).shape[2]
    group = _check_heads(num_q_heads, num_kv_heads)
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        keys = gather_context(k_cache, block_tables[s], ctx, block_size)
        values = gather_context(v_cache, block_tables[s], ctx, block_size)
        for h in range(num_q_heads):
            g = h // group
            out[s, h] = attend_rows(qf[s, h][None, :], keys[:, g], values[:, g],
                                    scale, [ctx])[0]
    return out


def paged_attention_prefill_chunk(q, k_cache, v_cache, block_tables,
                                  cu_seqlens_q, context_lens, scale,
                                  block_size, causal=True):
    """Attention of a batch of prefill chunks over their paged contexts.

    Chunk c owns query rows cu_seqlens_q[c] .. cu_seqlens_q[c+1]-1 of the
    packed q [Tq, Hq, D]; its context_lens[c] counts the cached tokens
    ("Building a minimal vLLM implementation", section sequence.py,
    num_cached_tokens) plus the chunk's own L rows, whose K/V are already in
    the cache. Row i sits at absolute position P0 + i, P0 = ctx - L. With
    causal set it sees keys 0 .. P0 + i; otherwise all ctx keys. Returns
    float64 [Tq, Hq, D].
    """
    qf = to_f64(q)
    total_q, num_q_heads, head_dim = qf.shape
    num_kv_heads = np.asarray(k_cache).shape[2]
    group = _check_heads(num_q_heads, num_kv_heads)
    cu = np.asarray(cu_seqlens_q).tolist()
    assert cu[0] == 0 and cu[-1] == total_q
    out = np.zeros((total_q, num_q_heads, head_dim), dtype=np.float64)
    for c in range(len(cu) - 1):
        start, end = cu[c], cu[c + 1]
        rows = end - start
        ctx = int(context_lens[c])
        prior = ctx - rows
        if prior < 0:
            raise ValueError(f"chunk {c}: {rows} rows but context {ctx}")
        if rows == 0:
            continue
        keys = gather_context(k_cache, block_tables[c], ctx, block_size)
        values = gather_context(v_cache, block_tables[c], ctx, block_size)
        if causal:
            visible = [prior + i + 1 for i in range(rows)]
        else:
            visible = [ctx] * rows
        for h in range(num_q_heads):
            g = h // group
            out[start:end, h] = attend_rows(qf[start:end, h], keys[:, g],
                                            values[:, g], scale, visible)
    return out
