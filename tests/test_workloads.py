"""CPU checks of the seeded input generators (no attention arithmetic here)."""

import numpy as np
import torch

import oracle
from paged_attention_kv_store_amd import workloads as W


def test_pool_is_a_permutation_with_unused_padding():
    rng = np.random.default_rng(0)
    ctx = np.array([1, 16, 17, 40, 0])
    pool = W.make_pool(rng, ctx, block_size=16)
    need = -(-ctx // 16)
    ids = np.concatenate([pool.block_tables[s, :need[s]] for s in range(len(ctx))])
    assert len(np.unique(ids)) == len(ids) == need.sum()
    assert pool.used.sum() == need.sum()
    assert pool.num_blocks == int(np.ceil(1.25 * need.sum()))
    assert not pool.used[pool.pad_block]
    for s in range(len(ctx)):
        assert (pool.block_tables[s, need[s]:] == pool.pad_block).all()


def test_shared_prefix_groups():
    rng = np.random.default_rng(1)
    ctx = rng.integers(513, 900, size=16)
    pool = W.make_pool(rng, ctx, share_group=8, shared_blocks=32)
    for g in range(2):
        grp = pool.block_tables[8 * g:8 * g + 8, :32]
        assert (grp == grp[0]).all()
    assert not np.intersect1d(pool.block_tables[0, :32], pool.block_tables[8, :32]).size
    private = np.concatenate([pool.block_tables[s, 32:-(-ctx[s] // 16)] for s in range(16)])
    assert len(np.unique(private)) == len(private)


def test_tiny_store_fills_the_poisoned_newest_rows():
    wl = W.tiny()
    b = wl.batches[0]
    assert b.k_cache.shape == (64, 16, 4, 64) and b.q.shape == (4, 8, 64)
    assert b.k_cache.dtype == torch.float32
    bits = lambda t: W.host_bits(t)
    bt, ctx = b.pool.block_tables, b.pool.context_lens
    before = oracle.paged_attention_decode(bits(b.q), bits(b.k_cache), bits(b.v_cache),
                                           bt, ctx, b.scale, 16)
    assert np.isnan(before).all(axis=(1, 2)).all()      # newest row is still poison
    kc, vc = oracle.kv_cache_store(bits(b.k_new), bits(b.v_new), bits(b.k_cache),
                                   bits(b.v_cache), bits(b.slot_mapping), 16)
    after = oracle.paged_attention_decode(bits(b.q), kc, vc, bt, ctx, b.scale, 16)
    assert np.isfinite(after).all()
    # context 1: the output is the stored V row of kv-head h // 2
    np.testing.assert_array_equal(after[0], W.host_bits(b.v_new)[0][np.arange(8) // 2])


def test_standard_workload_shapes():
    wl = W.qwen3_decode(layers=1)
    b = wl.batches[0]
    ctx = b.pool.context_lens
    assert ctx.shape == (60,) and ctx.min() >= 64 and ctx.max() <= 1024
    assert b.q.shape == (60, 16, 128) and b.k_cache.dtype == torch.bfloat16
    assert b.block_size == 16 and b.k_cache.shape[2:] == (8, 128)


def test_random_prefill_batch_slots_cover_the_chunks():
    b = W.random_prefill_batch(3, 3, 4, 2, 64, torch.float32, max_rows=20, max_prior=40)
    cu = b.cu_seqlens_q
    assert len(b.slot_mapping) == cu[-1] == b.q.shape[0]
    bits = W.host_bits
    kc, vc = oracle.kv_cache_store(bits(b.k_new), bits(b.v_new), bits(b.k_cache),
                                   bits(b.v_cache), bits(b.slot_mapping), 16)
    out = oracle.paged_attention_prefill_chunk(bits(b.q), kc, vc, b.pool.block_tables, cu,
                                               b.pool.context_lens, b.scale, 16)
    assert np.isfinite(out).all()


def test_spec_verify_rows_follow_their_prefix():
    wl = W.spec_verify()
    b = wl.prefill
    ctx, cu = b.pool.context_lens, b.cu_seqlens_q
    assert ctx.shape == (128,) and (ctx >= 260).all() and (ctx <= 4100).all()
    assert (np.diff(cu) == 4).all() and b.q.shape == (512, 32, 128)
    # the store fills exactly positions ctx-4 .. ctx-1 of each sequence
    slots = b.slot_mapping.numpy().reshape(128, 4)
    for s in range(0, 128, 17):
        pos = np.arange(ctx[s] - 4, ctx[s])
        want = b.pool.block_tables[s][pos // 16].astype(np.int64) * 16 + pos % 16
        np.testing.assert_array_equal(slots[s], want)
    assert len(np.unique(slots)) == slots.size
