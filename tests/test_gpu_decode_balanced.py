"""GPU parity of the work-balanced decode (partition_size "balanced") against
the float64 oracle, through the C ABI: batches whose items fall inside one
wave's share, items cut into many pieces merged in-kernel, share boundaries
that cross sequences and kv-heads, empty and one-token contexts, out-of-pool
block ids, the fused store, repeated calls on one workspace and HIP-graph
replays."""

import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, gpu_decode, oracle_caches, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu

BAL = "balanced"

SWEEP = [
    # (seed, seqs, hq, hkv, d, min_ctx, max_ctx, block_size)
    (1, 9, 16, 8, 128, 0, 300, 16),       # fewer tiles than waves x 4: most waves idle
    (2, 40, 32, 8, 128, 0, 2000, 16),     # shares cross sequences and kv-heads
    (3, 3, 32, 8, 128, 3000, 6000, 16),   # each item cut into hundreds of pieces
    (4, 64, 8, 8, 128, 1, 64, 16),        # G = 1, many short items per share
    (5, 17, 32, 2, 128, 0, 900, 16),      # G = 16
    (6, 12, 12, 4, 64, 0, 700, 16),       # head_dim 64, G = 3
    (7, 20, 64, 4, 64, 10, 1500, 32),     # head_dim 64, G = 16, block 32
    (8, 11, 16, 4, 128, 0, 1000, 48),     # block size not a power of two
    (9, 7, 32, 8, 128, 100, 2500, 256),   # largest block size
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"s{c[0]}-{c[1]}x{c[2]}x{c[3]}-d{c[4]}-bs{c[7]}")
def test_random_sweep(case):
    seed, seqs, hq, hkv, d, lo, hi, bs = case
    b = W.random_decode_batch(1000 + seed, seqs, hq, hkv, d, torch.bfloat16, max_ctx=hi, min_ctx=lo,
                              block_size=bs)
    say(f"balanced {case} ctx={b.pool.context_lens.tolist()}")
    got = gpu_decode(b, algo="mfma", partition_size=BAL)
    assert_close(got, oracle_decode(b), torch.bfloat16, f"balanced {case[0]}")


def test_shares_longer_than_one_descriptor_chunk():
    """More than 64 tiles per wave: the tile descriptors are refilled mid-walk."""
    b = W.random_decode_batch(1100, 32, 32, 8, 128, torch.bfloat16, max_ctx=10000, min_ctx=9000,
                              store=False)
    total = 8 * int(sum(-(-c // 16) for c in b.pool.context_lens.tolist()))
    say(f"balanced long shares: {total} tiles")
    assert total > 2048 * 64
    dev = to_device(b)
    got = gpu_decode(b, dev=dev, algo="mfma", partition_size=BAL, store=False)
    seqs = [0, 5, 13, 31]
    want = oracle_decode(b, seqs=seqs, store=False)
    assert_close(got[seqs], want, torch.bfloat16, "long shares")


def test_context_one_returns_the_v_row_exactly():
    b = W.random_decode_batch(1200, 7, 32, 8, 128, torch.bfloat16, max_ctx=1, min_ctx=1, store=False)
    v = W.host_bits(b.v_cache)
    want = np.repeat(np.stack([v[b.pool.block_tables[s, 0], 0] for s in range(7)]), 4, axis=1)
    got = gpu_decode(b, algo="mfma", partition_size=BAL, store=False)
    np.testing.assert_array_equal(got, oracle.to_f64(want))


def test_identical_keys_give_mean_of_v():
    b = W.random_decode_batch(1300, 5, 16, 8, 128, torch.bfloat16, max_ctx=3000, min_ctx=1,
                              store=False)
    b.k_cache.fill_(0.5)
    got = gpu_decode(b, algo="mfma", partition_size=BAL, store=False)
    v = oracle_caches(b, store=False)[1]
    want = np.zeros_like(got)
    for s, c in enumerate(b.pool.context_lens.tolist()):
        want[s] = np.repeat(oracle.gather_context(v, b.pool.block_tables[s], c, 16).mean(axis=0), 2, axis=0)
    assert_close(got, want, torch.bfloat16, "mean of V")


def test_empty_contexts():
    b = W.random_decode_batch(1400, 30, 16, 8, 128, torch.bfloat16, max_ctx=400, min_ctx=0,
                              store=False)
    b.pool.context_lens[::3] = 0              # every third sequence empty
    got = gpu_decode(b, algo="mfma", partition_size=BAL, store=False)
    assert (got[::3] == 0).all()
    live = [s for s in range(30) if s % 3]
    assert_close(got[live], oracle_decode(b, seqs=live, store=False), torch.bfloat16, "beside empty")
    b.pool.context_lens[:] = 0
    got = gpu_decode(b, algo="mfma", partition_size=BAL, store=False)
    assert (got == 0).all()


def test_out_of_pool_block_ids_poison_the_row():
    b = W.random_decode_batch(1500, 6, 16, 8, 128, torch.bfloat16, max_ctx=4000, min_ctx=2500,
                              store=False)
    b.pool.block_tables[2, 100] = b.pool.num_blocks + 5    # inside a sequence cut into pieces
    b.pool.block_tables[4, 0] = -3
    got = gpu_decode(b, algo="mfma", partition_size=BAL, store=False)
    assert np.isnan(got[2]).all() and np.isnan(got[4]).all()
    want = oracle_decode(b, seqs=[0, 1, 3, 5], store=False)
    assert_close(got[[0, 1, 3, 5]], want, torch.bfloat16, "rows beside the bad ones")


def test_repeated_calls_on_one_workspace():
    """Counters come back to zero after every call: the same workspace serves
    calls of different shapes, and repeats are bit-identical."""
    b1 = W.random_decode_batch(1600, 24, 32, 8, 128, torch.bfloat16, max_ctx=3000, min_ctx=0,
                               store=False)
    b2 = W.random_decode_batch(1601, 50, 32, 8, 128, torch.bfloat16, max_ctx=800, min_ctx=0,
                               store=False)
    need = max(pkv.decode_workspace_size(b.num_seqs, 32, 8, 128, b.max_ctx, BAL) for b in (b1, b2))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    d1, d2 = to_device(b1), to_device(b2)

    def run(b, dev):
        out = torch.empty_like(dev["q"])
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=BAL,
                                   workspace=ws, algo="mfma")
        torch.cuda.synchronize()
        return out.float().cpu().double().numpy()

    first = run(b1, d1)
    assert_close(first, oracle_decode(b1, store=False), torch.bfloat16, "first call")
    assert_close(run(b2, d2), oracle_decode(b2, store=False), torch.bfloat16, "second shape")
    for _ in range(3):
        np.testing.assert_array_equal(run(b1, d1), first)
    counters = ws[:65536 * 4].view(torch.int32)   # the whole counter block
    assert int(counters.abs().sum()) == 0


def test_graph_replays_match_eager():
    b = W.random_decode_batch(1700, 40, 16, 8, 128, torch.bfloat16, max_ctx=1024, min_ctx=64,
                              store=False)
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    call = pkv.DecodeLaunch(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                            dev["context_lens"], b.scale, b.max_ctx, partition_size=BAL, algo="mfma")
    call()
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(4):
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    assert_close(want.float().cpu().double().numpy(), oracle_decode(b, store=False), torch.bfloat16,
                 "graph")


FUSED = [
    # (seed, seqs, hq, hkv, d, max_ctx)
    (1, 11, 16, 8, 128, 400),
    (2, 30, 32, 8, 128, 2500),
    (3, 9, 12, 4, 64, 700),
    (4, 600, 16, 8, 128, 40),         # 4800 new rows: more than one pass of 2048 waves
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"s{c[0]}-{c[1]}x{c[2]}x{c[3]}-d{c[4]}")
def test_decode_store_fused(case):
    seed, seqs, hq, hkv, d, max_ctx = case
    b = W.random_decode_batch(1800 + seed, seqs, hq, hkv, d, torch.bfloat16, max_ctx=max_ctx, min_ctx=0)
    say(f"balanced fused {case}")
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["context_lens"], dev["k_new"], dev["v_new"], dev["slot_mapping"],
                                     b.scale, b.max_ctx, partition_size=BAL, algo="mfma")
    torch.cuda.synchronize()
    kc, vc = oracle_caches(b)
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert W.host_bits(dev["v_cache"]).tobytes() == vc.tobytes()
    assert_close(out.float().cpu().double().numpy(), oracle_decode(b, caches=(kc, vc)), torch.bfloat16,
                 f"fused {case[0]}")


def test_decode_store_fused_skips_negative_slots():
    b = W.random_decode_batch(1900, 12, 16, 8, 128, torch.bfloat16, max_ctx=600, min_ctx=1)
    b.slot_mapping[::4] = -1              # padding: stores nothing, the cache row is used as is
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["context_lens"], dev["k_new"], dev["v_new"], dev["slot_mapping"],
                                     b.scale, b.max_ctx, partition_size=BAL, algo="mfma")
    torch.cuda.synchronize()
    kc, vc = oracle_caches(b)
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    got = out.float().cpu().double().numpy()
    live = [s for s in range(12) if s % 4]
    assert_close(got[live], oracle_decode(b, caches=(kc, vc), seqs=live), torch.bfloat16, "stored rows")
    # the padded sequences read their (poisoned) newest row from the cache
    assert np.isnan(got[::4]).all()
