"""Seeded synthetic inputs for paged-KV attention.

This module only draws inputs: sequence lengths, block tables drawn as seeded
permutations of a block pool, slot mappings, and N(0,1) values for q, the K/V
caches and the new K/V rows. It performs none of the attention arithmetic and
is shared by the tests, the benchmark and the oracle-side checks, so that both
sides of a parity test see the very same bits.

Shapes follow serving batches of the kind the pages describe (a small Qwen3
decoding 60 batched prompts, Llama-class serving with prefix caching, chunked
prefill mixed with decode); the sizes are this library's six standard
workloads:

  tiny          4 seqs, ctx {1,17,100,256}, 8 q / 4 kv heads, D 64, fp32,
                pool of 64 blocks, one new token stored per sequence
  qwen3_decode  60 seqs, ctx U{64..1024}, 16 q / 8 kv heads, D 128, bf16,
                28 layers with distinct caches and queries, one shared table
  llama_prefix  256 seqs, ctx U{512..4096}, 32 q / 8 kv heads, D 128, bf16;
                each group of 8 seqs shares its first 32 physical blocks
  long_splitk   32 seqs, ctx log-uniform 1K..32K, 32 q / 8 kv heads, D 128,
                bf16, decoded with 512-token partitions and a reduce pass
  mixed         8 prefill chunks of 512 rows after U{0..8192} cached tokens,
                plus 128 decode seqs with ctx U{256..4096}; 32 q / 8 kv heads,
                D 128, bf16; all 4224 new tokens stored first
  spec_verify   128 seqs, each 4 causal query rows (one accepted and three
                drafted tokens) after U{256..4096} cached tokens; 32 q / 8 kv
                heads, D 128, bf16; the 512 new rows stored first

E4M3 variants (qwen3_decode_fp8, random_decode_batch_fp8) keep the shapes and
draw the caches as codes: N(0,1) values divided by per-kv-head scales drawn
U(0.008, 0.016), kept inside +-448 and cast by torch's float8_e4m3fn; dead
rows hold the NaN code 0x7f. q and the new rows stay bf16.

Recipe: the metadata comes from numpy PCG64 streams spawned from
SeedSequence(seed); values come from a torch generator (on the target device)
seeded from the same SeedSequence, drawn in fp32 and rounded to nearest-even
when the dtype is bf16. Pools hold ceil(1.25 x blocks in use) blocks unless
fixed. Every cache row that no live token owns (unused blocks, rows past the
end of a sequence's last block, and the slots the store is about to fill) is
set to NaN, and block-table padding points at an unused, NaN-filled block, so
any stray read reaches the output as NaN.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

BLOCK_SIZE = 16


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a tensor as host numpy: float32 and integer types as they
    are (uint8 for E4M3 codes), bf16 as uint16 bits."""
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.float64, torch.int32, torch.int64, torch.uint8):
        return t.numpy()
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class Pool:
    """Block tables of a batch and the pool they index."""

    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, MB]
    num_blocks: int
    used: np.ndarray                  # bool [NB], block holds a live token
    pad_block: int                    # unused block that padding points at


@dataclass
class PagedBatch:
    """One attention call's inputs over one paged pool (one layer)."""

    pool: Pool
    q: torch.Tensor                   # [S, Hq, D] (decode) or [Tq, Hq, D]
    k_cache: torch.Tensor             # [NB, bs, Hkv, D]
    v_cache: torch.Tensor
    scale: float
    block_size: int = BLOCK_SIZE
    # optional store performed before attention
    k_new: Optional[torch.Tensor] = None     # [T, Hkv, D]
    v_new: Optional[torch.Tensor] = None
    slot_mapping: Optional[torch.Tensor] = None   # int32 [T]
    # prefill chunks only
    cu_seqlens_q: Optional[np.ndarray] = None      # int32 [S+1]
    # E4M3 caches only: the caches hold uint8 codes; one scale per kv-head
    k_scale: Optional[torch.Tensor] = None          # float32 [Hkv]
    v_scale: Optional[torch.Tensor] = None

    @property
    def num_seqs(self) -> int:
        return int(self.pool.context_lens.shape[0])

    @property
    def num_q_heads(self) -> int:
        return int(self.q.shape[1])

    @property
    def num_kv_heads(self) -> int:
        return int(self.k_cache.shape[2])

    @property
    def head_dim(self) -> int:
        return int(self.k_cache.shape[3])

    @property
    def max_blocks(self) -> int:
        return int(self.pool.block_tables.shape[1])

    @property
    def max_ctx(self) -> int:
        return int(self.pool.context_lens.max()) if self.num_seqs else 0


@dataclass
class Workload:
    name: str
    batches: List[PagedBatch] = field(default_factory=list)   # decode layers
    prefill: Optional[PagedBatch] = None
    partition_size: int = 0
    notes: str = ""


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(n)]


def _torch_seed(seed: int, salt: int) -> int:
    return int(np.random.SeedSequence([seed, salt]).generate_state(1)[0])


def make_pool(rng, context_lens, block_size=BLOCK_SIZE, pool_factor=1.25,
              num_blocks=None, share_group=0, shared_blocks=0,
              max_blocks=None, reserve=0) -> Pool:
    """Assign physical blocks to sequences from a seeded permutation.

    share_group > 0: consecutive groups of that many sequences share their
    first shared_blocks logical blocks (same physical ids, read-only).
    reserve extra blocks are kept unused beyond the 1.25x rule.
    """
    ctx = np.asarray(context_lens, dtype=np.int64)
    needed = -(-ctx // block_size)
    num_seqs = len(ctx)
    if share_group:
        assert num_seqs % share_group == 0
        assert (needed >= shared_blocks).all()
        unique = (num_seqs // share_group) * shared_blocks + int((needed - shared_blocks).sum())
    else:
        unique = int(needed.sum())
    if num_blocks is None:
        num_blocks = int(math.ceil(pool_factor * unique)) + reserve
    if num_blocks <= unique:
        raise ValueError("pool leaves no unused block for padding")
    perm = rng.permutation(num_blocks).astype(np.int32)
    mb = int(needed.max()) if max_blocks is None else int(max_blocks)
    mb = max(mb, 1)
    pad_block = int(perm[-1])
    tables = np.full((num_seqs, mb), pad_block, dtype=np.int32)
    cursor = 0
    shared_ids = None
    for s in range(num_seqs):
        first = 0
        if share_group:
            if s % share_group == 0:
                shared_ids = perm[cursor:cursor + shared_blocks]
                cursor += shared_blocks
            tables[s, :shared_blocks] = shared_ids
            first = shared_blocks
        count = int(needed[s]) - first
        tables[s, first:first + count] = perm[cursor:cursor + count]
        cursor += count
    assert cursor == unique
    used = np.zeros(num_blocks, dtype=bool)
    used[perm[:unique]] = True
    return Pool(context_lens=ctx.astype(np.int32), block_tables=tables,
                num_blocks=num_blocks, used=used, pad_block=pad_block)


def _slots_of(pool: Pool, seq: int, positions, block_size) -> np.ndarray:
    positions = np.asarray(positions, dtype=np.int64)
    blocks = pool.block_tables[seq][positions // block_size].astype(np.int64)
    return (blocks * block_size + positions % block_size).astype(np.int32)


def _dead_rows(pool: Pool, block_size: int, extra_slots=()) -> np.ndarray:
    """Flat row indices (block * bs + row) that no live token owns."""
    rows = [np.flatnonzero(~pool.used)[:, None] * block_size
            + np.arange(block_size)[None, :]]
    for s, c in enumerate(pool.context_lens.tolist()):
        if c % block_size:
            last = int(pool.block_tables[s][(c - 1) // block_size])
            rows.append(last * block_size + np.arange(c % block_size, block_size))
    rows.append(np.asarray(extra_slots, dtype=np.int64).reshape(-1))
    return np.unique(np.concatenate([r.reshape(-1) for r in rows]).astype(np.int64))


def _normal(shape, dtype, gen, device):
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    return x.to(dtype)


def _poisoned_cache(num_blocks, block_size, num_kv_heads, head_dim, dtype, gen,
                    device, dead_rows):
    cache = _normal((num_blocks, block_size, num_kv_heads, head_dim), dtype, gen, device)
    if len(dead_rows):
        flat = cache.view(num_blocks * block_size, num_kv_heads * head_dim)
        idx = torch.as_tensor(dead_rows, dtype=torch.long, device=device)
        flat.index_fill_(0, idx, float("nan"))
    return cache


E4M3_NAN = 0x7F


def _e4m3_cache(num_blocks, block_size, num_kv_heads, head_dim, scale, gen, device, dead_rows):
    """Cache of E4M3 codes standing for N(0,1) values at the given per-head
    scales: the draws divided by the scale, kept inside the format's +-448 and
    cast by torch's float8_e4m3fn; dead rows hold the NaN code."""
    x = torch.randn((num_blocks, block_size, num_kv_heads, head_dim), generator=gen, device=device,
                    dtype=torch.float32)
    x = (x / scale.view(1, 1, -1, 1)).clamp_(-448.0, 448.0)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    if len(dead_rows):
        flat = codes.view(num_blocks * block_size, num_kv_heads * head_dim)
        flat[torch.as_tensor(dead_rows, dtype=torch.long, device=device)] = E4M3_NAN
    return codes


def build_batch_fp8(pool: Pool, num_q_heads, num_kv_heads, head_dim, seed, salt, device,
                    num_queries=None, store_slots=None, block_size=BLOCK_SIZE,
                    scale=None) -> PagedBatch:
    """Like build_batch with E4M3 caches: q and the new rows are bf16, the
    caches uint8 codes, k_scale / v_scale drawn U(0.008, 0.016) per kv-head
    (about max|x| / 448 for N(0,1) rows)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(seed, salt))
    n_q = pool.context_lens.shape[0] if num_queries is None else num_queries
    store_slots = None if store_slots is None else np.asarray(store_slots, np.int32)
    live_store = () if store_slots is None else store_slots[store_slots >= 0]
    dead = _dead_rows(pool, block_size, live_store)
    q = _normal((n_q, num_q_heads, head_dim), torch.bfloat16, gen, device)
    k_scale = torch.empty(num_kv_heads, device=device).uniform_(0.008, 0.016, generator=gen)
    v_scale = torch.empty(num_kv_heads, device=device).uniform_(0.008, 0.016, generator=gen)
    kc = _e4m3_cache(pool.num_blocks, block_size, num_kv_heads, head_dim, k_scale, gen, device, dead)
    vc = _e4m3_cache(pool.num_blocks, block_size, num_kv_heads, head_dim, v_scale, gen, device, dead)
    batch = PagedBatch(pool=pool, q=q, k_cache=kc, v_cache=vc,
                       scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                       block_size=block_size, k_scale=k_scale, v_scale=v_scale)
    if store_slots is not None:
        t = len(store_slots)
        batch.k_new = _normal((t, num_kv_heads, head_dim), torch.bfloat16, gen, device)
        batch.v_new = _normal((t, num_kv_heads, head_dim), torch.bfloat16, gen, device)
        batch.slot_mapping = torch.as_tensor(store_slots, dtype=torch.int32, device=device)
    return batch


def build_batch(pool: Pool, num_q_heads, num_kv_heads, head_dim, dtype, seed,
                salt, device, num_queries=None, store_slots=None,
                block_size=BLOCK_SIZE, scale=None) -> PagedBatch:
    """Draw q, caches and (optionally) new K/V rows for one call."""
    gen = torch.Generator(device=device)
    gen.manual_seed(_torch_seed(seed, salt))
    n_q = pool.context_lens.shape[0] if num_queries is None else num_queries
    store_slots = None if store_slots is None else np.asarray(store_slots, np.int32)
    live_store = () if store_slots is None else store_slots[store_slots >= 0]
    dead = _dead_rows(pool, block_size, live_store)
    q = _normal((n_q, num_q_heads, head_dim), dtype, gen, device)
    kc = _poisoned_cache(pool.num_blocks, block_size, num_kv_heads, head_dim,
                         dtype, gen, device, dead)
    vc = _poisoned_cache(pool.num_blocks, block_size, num_kv_heads, head_dim,
                         dtype, gen, device, dead)
    batch = PagedBatch(pool=pool, q=q, k_cache=kc, v_cache=vc,
                       scale=(1.0 / math.sqrt(head_dim)) if scale is None else scale,
                       block_size=block_size)
    if store_slots is not None:
        t = len(store_slots)
        batch.k_new = _normal((t, num_kv_heads, head_dim), dtype, gen, device)
        batch.v_new = _normal((t, num_kv_heads, head_dim), dtype, gen, device)
        batch.slot_mapping = torch.as_tensor(store_slots, dtype=torch.int32, device=device)
    return batch


def decode_store_slots(pool: Pool, block_size=BLOCK_SIZE) -> np.ndarray:
    """Slot of each sequence's newest token (position ctx-1); -1 if ctx == 0."""
    out = np.full(pool.context_lens.shape[0], -1, dtype=np.int32)
    for s, c in enumerate(pool.context_lens.tolist()):
        if c > 0:
            out[s] = _slots_of(pool, s, [c - 1], block_size)[0]
    return out


# --------------------------------------------------------------------------
# The six standard workloads.
# --------------------------------------------------------------------------

def tiny(seed: int = 0, device="cpu") -> Workload:
    (rng,) = _streams(seed, 1)
    ctx = np.array([1, 17, 100, 256], dtype=np.int32)
    pool = make_pool(rng, ctx, num_blocks=64)
    slots = decode_store_slots(pool)
    batch = build_batch(pool, 8, 4, 64, torch.float32, seed, 0, device,
                        store_slots=slots, scale=1.0 / 8.0)
    return Workload("tiny", [batch], notes="fp32 GQA-2 decode + store, 64-block pool")


def qwen3_decode(seed: int = 1, device="cpu", layers: int = 28) -> Workload:
    (rng,) = _streams(seed, 1)
    ctx = rng.integers(64, 1024, size=60, endpoint=True).astype(np.int32)
    pool = make_pool(rng, ctx)
    slots = decode_store_slots(pool)
    batches = [build_batch(pool, 16, 8, 128, torch.bfloat16, seed, 1 + layer, device,
                           store_slots=slots)
               for layer in range(layers)]
    return Workload("qwen3_decode", batches,
                    notes=f"{layers} layers, distinct caches, one block table")


def llama_prefix(seed: int = 2, device="cpu") -> Workload:
    (rng,) = _streams(seed, 1)
    ctx = rng.integers(512, 4096, size=256, endpoint=True).astype(np.int32)
    pool = make_pool(rng, ctx, share_group=8, shared_blocks=32)
    batch = build_batch(pool, 32, 8, 128, torch.bfloat16, seed, 0, device)
    return Workload("llama_prefix", [batch],
                    notes="groups of 8 seqs share their first 32 physical blocks")


def long_splitk(seed: int = 3, device="cpu") -> Workload:
    (rng,) = _streams(seed, 1)
    u = rng.uniform(math.log(1024), math.log(32768), size=32)
    ctx = np.floor(np.exp(u)).astype(np.int32)
    pool = make_pool(rng, ctx)
    batch = build_batch(pool, 32, 8, 128, torch.bfloat16, seed, 0, device)
    return Workload("long_splitk", [batch], partition_size=512,
                    notes="log-uniform 1K..32K, 512-token partitions")


def mixed(seed: int = 4, device="cpu") -> Workload:
    """Chunked prefill (8 x 512 rows) plus 128 decode seqs on one pool.

    Sequences 0..7 are the prefill chunks (context = prior + 512), 8..135 the
    decode sequences. The store writes the 4096 chunk tokens then the 128
    decode tokens, in that order.
    """
    (rng,) = _streams(seed, 1)
    chunk = 512
    prior = rng.integers(0, 8192, size=8, endpoint=True).astype(np.int32)
    dctx = rng.integers(256, 4096, size=128, endpoint=True).astype(np.int32)
    ctx = np.concatenate([prior + chunk, dctx]).astype(np.int32)
    pool = make_pool(rng, ctx)
    slots = []
    for c in range(8):
        slots.append(_slots_of(pool, c, np.arange(prior[c], prior[c] + chunk), BLOCK_SIZE))
    slots.append(decode_store_slots(
        Pool(pool.context_lens[8:], pool.block_tables[8:], pool.num_blocks,
             pool.used, pool.pad_block)))
    slots = np.concatenate(slots).astype(np.int32)
    # one draw for the whole pool; q rows: 4096 prefill rows then 128 decode rows
    base = build_batch(pool, 32, 8, 128, torch.bfloat16, seed, 0, device,
                       num_queries=8 * chunk + 128, store_slots=slots)
    mb_prefill = int(-(-int(ctx[:8].max()) // BLOCK_SIZE))
    mb_decode = int(-(-int(dctx.max()) // BLOCK_SIZE))
    pre_pool = Pool(pool.context_lens[:8].copy(),
                    np.ascontiguousarray(pool.block_tables[:8, :mb_prefill]),
                    pool.num_blocks, pool.used, pool.pad_block)
    dec_pool = Pool(pool.context_lens[8:].copy(),
                    np.ascontiguousarray(pool.block_tables[8:, :mb_decode]),
                    pool.num_blocks, pool.used, pool.pad_block)
    prefill = PagedBatch(pool=pre_pool, q=base.q[:8 * chunk], k_cache=base.k_cache,
                         v_cache=base.v_cache, scale=base.scale,
                         k_new=base.k_new, v_new=base.v_new,
                         slot_mapping=base.slot_mapping,
                         cu_seqlens_q=np.arange(0, 8 * chunk + 1, chunk, dtype=np.int32))
    decode = PagedBatch(pool=dec_pool, q=base.q[8 * chunk:], k_cache=base.k_cache,
                        v_cache=base.v_cache, scale=base.scale)
    return Workload("mixed", [decode], prefill=prefill,
                    notes="store 4224 tokens, prefill 8x512 causal, decode 128 seqs")


def spec_verify(seed: int = 5, device="cpu", rows: int = 4) -> Workload:
    """Verification of drafted tokens: 128 seqs x `rows` causal query rows.

    Each sequence has U{256..4096} cached tokens before the rows (the last
    accepted token plus rows-1 drafted ones); the rows' own K/V are stored
    first, so context = prior + rows. Shapes as the decode half of `mixed`.
    """
    (rng,) = _streams(seed, 1)
    prior = rng.integers(256, 4096, size=128, endpoint=True).astype(np.int32)
    ctx = (prior + rows).astype(np.int32)
    pool = make_pool(rng, ctx)
    slots = np.concatenate([_slots_of(pool, c, np.arange(prior[c], ctx[c]), BLOCK_SIZE)
                            for c in range(len(ctx))]).astype(np.int32)
    batch = build_batch(pool, 32, 8, 128, torch.bfloat16, seed, 0, device,
                        num_queries=rows * len(ctx), store_slots=slots)
    batch.cu_seqlens_q = np.arange(0, rows * len(ctx) + 1, rows, dtype=np.int32)
    return Workload("spec_verify", [], prefill=batch,
                    notes=f"128 seqs x {rows} causal query rows after U{{256..4096}} cached")


WORKLOADS = {
    "tiny": tiny,
    "qwen3_decode": qwen3_decode,
    "llama_prefix": llama_prefix,
    "long_splitk": long_splitk,
    "mixed": mixed,
    "spec_verify": spec_verify,
}


def random_decode_batch(seed, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        dtype, max_ctx, min_ctx=0, block_size=BLOCK_SIZE,
                        device="cpu", store=True, scale=None,
                        share_group=0, shared_blocks=0) -> PagedBatch:
    """A small random decode batch for parity sweeps (lengths U{min..max})."""
    (rng,) = _streams(seed, 1)
    ctx = rng.integers(min_ctx, max_ctx, size=num_seqs, endpoint=True).astype(np.int32)
    if share_group:
        ctx = np.maximum(ctx, shared_blocks * block_size + 1).astype(np.int32)
    pool = make_pool(rng, ctx, block_size=block_size, share_group=share_group,
                     shared_blocks=shared_blocks,
                     max_blocks=max(1, -(-int(max(max_ctx, ctx.max())) // block_size)),
                     reserve=2)
    slots = decode_store_slots(pool, block_size) if store else None
    return build_batch(pool, num_q_heads, num_kv_heads, head_dim, dtype, seed, 7,
                       device, store_slots=slots, block_size=block_size, scale=scale)


def random_decode_batch_fp8(seed, num_seqs, num_q_heads, num_kv_heads, head_dim, max_ctx,
                            min_ctx=0, block_size=BLOCK_SIZE, device="cpu", store=True,
                            scale=None) -> PagedBatch:
    """random_decode_batch with E4M3 caches (bf16 q and new rows)."""
    (rng,) = _streams(seed, 1)
    ctx = rng.integers(min_ctx, max_ctx, size=num_seqs, endpoint=True).astype(np.int32)
    pool = make_pool(rng, ctx, block_size=block_size,
                     max_blocks=max(1, -(-int(max(max_ctx, ctx.max())) // block_size)), reserve=2)
    slots = decode_store_slots(pool, block_size) if store else None
    return build_batch_fp8(pool, num_q_heads, num_kv_heads, head_dim, seed, 8, device,
                           store_slots=slots, block_size=block_size, scale=scale)


def qwen3_decode_fp8(seed: int = 1, device="cpu", layers: int = 28) -> Workload:
    """The Qwen3-shaped decode step over E4M3 caches: the same lengths,
    tables and new-row slots as qwen3_decode (same seed), bf16 q."""
    (rng,) = _streams(seed, 1)
    ctx = rng.integers(64, 1024, size=60, endpoint=True).astype(np.int32)
    pool = make_pool(rng, ctx)
    slots = decode_store_slots(pool)
    batches = [build_batch_fp8(pool, 16, 8, 128, seed, 101 + layer, device, store_slots=slots)
               for layer in range(layers)]
    return Workload("qwen3_decode_fp8", batches,
                    notes=f"{layers} layers, E4M3 caches with per-kv-head scales")


def random_prefill_batch_fp8(seed, num_chunks, num_q_heads, num_kv_heads, head_dim, max_rows,
                             max_prior, min_rows=1, block_size=BLOCK_SIZE, device="cpu",
                             scale=None) -> PagedBatch:
    """random_prefill_batch with E4M3 caches (bf16 q and new rows)."""
    (rng,) = _streams(seed, 1)
    rows = rng.integers(min_rows, max_rows, size=num_chunks, endpoint=True).astype(np.int32)
    prior = rng.integers(0, max_prior, size=num_chunks, endpoint=True).astype(np.int32)
    ctx = (rows + prior).astype(np.int32)
    pool = make_pool(rng, ctx, block_size=block_size, reserve=2)
    slots = np.concatenate(
        [_slots_of(pool, c, np.arange(prior[c], ctx[c]), block_size) for c in range(num_chunks)]
        + [np.zeros(0, np.int32)]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    batch = build_batch_fp8(pool, num_q_heads, num_kv_heads, head_dim, seed, 10, device,
                            num_queries=int(cu[-1]), store_slots=slots, block_size=block_size,
                            scale=scale)
    batch.cu_seqlens_q = cu
    return batch


def mixed_prefill_fp8(seed: int = 4, device="cpu") -> PagedBatch:
    """The mixed workload's prefill part (8 chunks x 512 rows after U{0..8192}
    cached tokens, 32 q / 8 kv heads) over E4M3 caches: the same lengths and
    tables as mixed(seed), its own draws of q, caches and new rows."""
    (rng,) = _streams(seed, 1)
    chunk = 512
    prior = rng.integers(0, 8192, size=8, endpoint=True).astype(np.int32)
    dctx = rng.integers(256, 4096, size=128, endpoint=True).astype(np.int32)
    ctx = np.concatenate([prior + chunk, dctx]).astype(np.int32)
    pool = make_pool(rng, ctx)
    slots = np.concatenate([_slots_of(pool, c, np.arange(prior[c], prior[c] + chunk), BLOCK_SIZE)
                            for c in range(8)]).astype(np.int32)
    mb = int(-(-int(ctx[:8].max()) // BLOCK_SIZE))
    pre_pool = Pool(pool.context_lens[:8].copy(), np.ascontiguousarray(pool.block_tables[:8, :mb]),
                    pool.num_blocks, pool.used, pool.pad_block)
    batch = build_batch_fp8(pre_pool, 32, 8, 128, seed, 11, device, num_queries=8 * chunk,
                            store_slots=slots)
    batch.cu_seqlens_q = np.arange(0, 8 * chunk + 1, chunk, dtype=np.int32)
    return batch


def random_prefill_batch(seed, num_chunks, num_q_heads, num_kv_heads, head_dim,
                         dtype, max_rows, max_prior, min_rows=1,
                         block_size=BLOCK_SIZE, device="cpu", scale=None, priors=None) -> PagedBatch:
    """Small random prefill chunks (rows U{min..max}, prior U{0..max_prior},
    or the given prior lengths)."""
    (rng,) = _streams(seed, 1)
    rows = rng.integers(min_rows, max_rows, size=num_chunks, endpoint=True).astype(np.int32)
    prior = rng.integers(0, max_prior, size=num_chunks, endpoint=True).astype(np.int32)
    if priors is not None:
        prior = np.asarray(priors, np.int32)
        assert prior.shape == (num_chunks,)
    ctx = (rows + prior).astype(np.int32)
    pool = make_pool(rng, ctx, block_size=block_size, reserve=2)
    slots = np.concatenate(
        [_slots_of(pool, c, np.arange(prior[c], ctx[c]), block_size) for c in range(num_chunks)]
        + [np.zeros(0, np.int32)]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    batch = build_batch(pool, num_q_heads, num_kv_heads, head_dim, dtype, seed, 9,
                        device, num_queries=int(cu[-1]), store_slots=slots,
                        block_size=block_size, scale=scale)
    batch.cu_seqlens_q = cu
    return batch


def decode_batch_of_lengths(seed, context_lens, num_q_heads, num_kv_heads, head_dim, dtype,
                            block_size=BLOCK_SIZE, device="cpu", store=True) -> PagedBatch:
    """A decode batch with the given context lengths; dtype "e4m3" draws
    E4M3 caches (bf16 q and new rows), any torch dtype plain caches."""
    (rng,) = _streams(seed, 1)
    ctx = np.asarray(context_lens, np.int32)
    pool = make_pool(rng, ctx, block_size=block_size, reserve=2)
    slots = decode_store_slots(pool, block_size) if store else None
    if dtype == "e4m3":
        return build_batch_fp8(pool, num_q_heads, num_kv_heads, head_dim, seed, 11, device,
                               store_slots=slots, block_size=block_size)
    return build_batch(pool, num_q_heads, num_kv_heads, head_dim, dtype, seed, 11, device,
                       store_slots=slots, block_size=block_size)


def prefill_batch_of_lengths(seed, rows, priors, num_q_heads, num_kv_heads, head_dim, dtype,
                             block_size=BLOCK_SIZE, device="cpu") -> PagedBatch:
    """Prefill chunks with the given query rows and cached tokens before them
    (context = prior + rows); the chunks' own rows are the new rows to store.
    dtype "e4m3" draws E4M3 caches (bf16 q and new rows)."""
    (rng,) = _streams(seed, 1)
    rows = np.asarray(rows, np.int32)
    prior = np.asarray(priors, np.int32)
    ctx = (rows + prior).astype(np.int32)
    pool = make_pool(rng, ctx, block_size=block_size, reserve=2)
    slots = np.concatenate(
        [_slots_of(pool, c, np.arange(prior[c], ctx[c]), block_size) for c in range(len(ctx))]
        + [np.zeros(0, np.int32)]).astype(np.int32)
    cu = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    if dtype == "e4m3":
        batch = build_batch_fp8(pool, num_q_heads, num_kv_heads, head_dim, seed, 12, device,
                                num_queries=int(cu[-1]), store_slots=slots, block_size=block_size)
    else:
        batch = build_batch(pool, num_q_heads, num_kv_heads, head_dim, dtype, seed, 12, device,
                            num_queries=int(cu[-1]), store_slots=slots, block_size=block_size)
    batch.cu_seqlens_q = cu
    return batch
