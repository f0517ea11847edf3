"""GPU parity of paged_attention_decode (single pass, split-K + reduce, VALU
and MFMA kernels) against the float64 oracle, through the C ABI."""

import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import (assert_close, gpu_decode, oracle_caches, oracle_decode, say,
                               to_device)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("partition", [0, 16, 32, 64, 256])
def test_tiny_fp32(partition):
    b = W.tiny().batches[0]
    say(f"tiny fp32 partition={partition}")
    got = gpu_decode(b, algo="valu", partition_size=partition)
    assert_close(got, oracle_decode(b), torch.float32, f"tiny p={partition}")


SWEEP = [
    # (dtype, hq, hkv, d, max_ctx, algo)
    (torch.float32, 8, 4, 64, 300, "valu"),
    (torch.float32, 8, 8, 128, 170, "valu"),
    (torch.float32, 24, 3, 64, 120, "valu"),
    (torch.bfloat16, 16, 8, 128, 300, "valu"),
    (torch.bfloat16, 32, 8, 128, 300, "valu"),
    (torch.bfloat16, 12, 2, 64, 250, "valu"),
    (torch.bfloat16, 16, 8, 128, 300, "mfma"),
    (torch.bfloat16, 32, 8, 128, 300, "mfma"),
    (torch.bfloat16, 8, 8, 128, 200, "mfma"),
    (torch.bfloat16, 32, 2, 128, 200, "mfma"),
    (torch.bfloat16, 12, 4, 64, 250, "mfma"),
    (torch.bfloat16, 64, 4, 64, 150, "mfma"),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{str(c[0])[6:]}-{c[1]}x{c[2]}-d{c[3]}-{c[5]}")
@pytest.mark.parametrize("partition", [0, 32, 128])
def test_random_sweep(case, partition):
    dtype, hq, hkv, d, max_ctx, algo = case
    b = W.random_decode_batch(hq * 131 + d + max_ctx, 9, hq, hkv, d, dtype, max_ctx=max_ctx,
                              min_ctx=0)
    say(f"sweep {case} p={partition} ctx={b.pool.context_lens.tolist()}")
    got = gpu_decode(b, algo=algo, partition_size=partition)
    assert_close(got, oracle_decode(b), dtype, f"{algo} p={partition}")


@pytest.mark.parametrize("num_seqs", [40, 70, 150])
def test_items_handed_out_by_size(num_seqs):
    """The single-pass kernel hands (sequence, kv-head) items to workgroups by
    size, ties by index: between one and two items per compute unit (40 x 8),
    more than two (70 x 8, 150 x 8), with short contexts so that most sizes
    tie and some are empty. Every row must be written, and right."""
    b = W.random_decode_batch(500 + num_seqs, num_seqs, 16, 8, 128, torch.bfloat16, max_ctx=70,
                              min_ctx=0)
    say(f"by size: S={num_seqs} ctx={b.pool.context_lens.tolist()}")
    got = gpu_decode(b, algo="mfma", partition_size=0)
    assert_close(got, oracle_decode(b), torch.bfloat16, f"S={num_seqs}")
    assert (got[b.pool.context_lens == 0] == 0).all()


@pytest.mark.parametrize("bs", [32, 64])
@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_larger_blocks(bs, algo):
    b = W.random_decode_batch(3 + bs, 6, 16, 4, 128, torch.bfloat16, max_ctx=400, min_ctx=1,
                              block_size=bs)
    say(f"block_size {bs} {algo}")
    got = gpu_decode(b, algo=algo, partition_size=64)
    assert_close(got, oracle_decode(b), torch.bfloat16, f"bs={bs} {algo}")


@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_context_one_returns_the_v_row_exactly(algo):
    b = W.random_decode_batch(21, 7, 32, 8, 128, torch.bfloat16, max_ctx=1, min_ctx=1,
                              store=False)
    say(f"ctx=1 {algo}")
    v = W.host_bits(b.v_cache)
    want = np.stack([v[b.pool.block_tables[s, 0], 0] for s in range(7)])
    want = np.repeat(want, 4, axis=1)          # q-head h reads kv-head h // 4
    for partition in (0, 16):
        got = gpu_decode(b, algo=algo, partition_size=partition, store=False)
        np.testing.assert_array_equal(got, oracle.to_f64(want))


@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_identical_keys_give_mean_of_v(algo):
    b = W.random_decode_batch(23, 5, 16, 8, 128, torch.bfloat16, max_ctx=200, min_ctx=1,
                              store=False)
    b.k_cache.fill_(0.5)                        # every key equal
    say(f"identical keys {algo}")
    got = gpu_decode(b, algo=algo, store=False)
    v = oracle_caches(b, store=False)[1]
    want = np.zeros_like(got)
    for s, c in enumerate(b.pool.context_lens.tolist()):
        rows = oracle.gather_context(v, b.pool.block_tables[s], c, b.block_size).mean(axis=0)
        want[s] = np.repeat(rows, 2, axis=0)
    assert_close(got, want, torch.bfloat16, "mean of V")


@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_block_permutation_invariance_is_bit_exact(algo):
    b = W.random_decode_batch(29, 8, 32, 8, 128, torch.bfloat16, max_ctx=500, min_ctx=100,
                              store=False)
    dev = to_device(b)
    out1 = gpu_decode(b, dev=dev, algo=algo, partition_size=64, store=False)
    pi = torch.as_tensor(np.random.default_rng(1).permutation(b.pool.num_blocks), device="cuda")
    kc2 = torch.empty_like(dev["k_cache"])
    vc2 = torch.empty_like(dev["v_cache"])
    kc2[pi.long()] = dev["k_cache"]
    vc2[pi.long()] = dev["v_cache"]
    dev2 = dict(dev, k_cache=kc2, v_cache=vc2,
                block_tables=pi.to(torch.int32)[dev["block_tables"].long()].contiguous())
    out2 = gpu_decode(b, dev=dev2, algo=algo, partition_size=64, store=False)
    np.testing.assert_array_equal(out1, out2)


@pytest.mark.parametrize("algo", ["valu", "mfma"])
def test_deterministic(algo):
    b = W.random_decode_batch(31, 16, 32, 8, 128, torch.bfloat16, max_ctx=900, min_ctx=1)
    dev = to_device(b)
    a = gpu_decode(b, dev=dev, algo=algo, partition_size=128)
    c = gpu_decode(b, dev=dev, algo=algo, partition_size=128, store=False)
    np.testing.assert_array_equal(a, c)


def test_empty_contexts_give_zero_rows():
    b = W.random_decode_batch(37, 6, 16, 8, 128, torch.bfloat16, max_ctx=50, min_ctx=0)
    b.pool.context_lens[:] = 0
    for algo in ("valu", "mfma"):
        for partition in (0, 16):
            got = gpu_decode(b, algo=algo, partition_size=partition, store=False)
            assert (got == 0).all()


def test_out_of_pool_block_ids_poison_the_row():
    b = W.random_decode_batch(41, 4, 16, 8, 128, torch.bfloat16, max_ctx=64, min_ctx=40,
                              store=False)
    b.pool.block_tables[2, 0] = b.pool.num_blocks + 5    # rejected in-kernel, not dereferenced
    for algo in ("valu", "mfma"):
        got = gpu_decode(b, algo=algo, store=False)
        assert np.isnan(got[2]).all()
        want = oracle_decode(b, seqs=[0, 1, 3], store=False)
        assert_close(got[[0, 1, 3]], want, torch.bfloat16, f"rows beside the bad one {algo}")


# --------------------------------------------------------------------------
# two streams
# --------------------------------------------------------------------------

@pytest.mark.slow
def test_mixed_prefill_and_decode_on_two_streams_match_serial():
    """The mixed batch with its prefill chunks and decode sequences on two
    streams (after the store) gives the bits of the serial run."""
    wl = W.mixed(device="cuda")
    pre, dec = wl.prefill, wl.batches[0]
    store = pkv.StoreLaunch(pre.k_new, pre.v_new, pre.k_cache, pre.v_cache, pre.slot_mapping)
    outs = {}
    for mode in ("serial", "two"):
        po = torch.full_like(pre.q, float("nan"))
        do = torch.full_like(dec.q, float("nan"))
        prefill = pkv.PrefillLaunch(po, pre.q, pre.k_cache, pre.v_cache,
                                    torch.as_tensor(pre.pool.block_tables, device="cuda"),
                                    torch.as_tensor(pre.cu_seqlens_q, device="cuda"),
                                    torch.as_tensor(pre.pool.context_lens, device="cuda"), pre.scale,
                                    int(np.diff(pre.cu_seqlens_q).max()), pre.max_ctx, causal=True)
        decode = pkv.DecodeLaunch(do, dec.q, dec.k_cache, dec.v_cache,
                                  torch.as_tensor(dec.pool.block_tables, device="cuda"),
                                  torch.as_tensor(dec.pool.context_lens, device="cuda"), dec.scale, dec.max_ctx)
        torch.cuda.synchronize()
        store()
        if mode == "serial":
            prefill()
            decode()
        else:
            cur = torch.cuda.current_stream()
            sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
            sa.wait_stream(cur)
            sb.wait_stream(cur)
            with torch.cuda.stream(sa):
                prefill()
            with torch.cuda.stream(sb):
                decode()
            cur.wait_stream(sa)
            cur.wait_stream(sb)
        torch.cuda.synchronize()
        outs[mode] = (po, do)
    assert torch.isfinite(outs["serial"][0].float()).all() and torch.isfinite(outs["serial"][1].float()).all()
    for a, b in zip(outs["serial"], outs["two"]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# --------------------------------------------------------------------------
# store fused into decode
# --------------------------------------------------------------------------

FUSED = [
    # (dtype, hq, hkv, d, max_ctx, algo, partition)
    (torch.float32, 8, 4, 64, 300, "valu", 0),
    (torch.float32, 8, 4, 64, 300, "valu", 32),
    (torch.bfloat16, 16, 8, 128, 400, "valu", 64),
    (torch.bfloat16, 16, 8, 128, 400, "mfma", 0),
    (torch.bfloat16, 32, 8, 128, 700, "mfma", 128),
    (torch.bfloat16, 32, 8, 128, 700, "mfma", 32),
    (torch.bfloat16, 12, 4, 64, 250, "mfma", 0),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"{str(c[0])[6:]}-{c[1]}x{c[2]}-d{c[3]}-{c[5]}-p{c[6]}")
def test_decode_store_fused(case):
    dtype, hq, hkv, d, max_ctx, algo, partition = case
    b = W.random_decode_batch(hq * 17 + d + partition, 11, hq, hkv, d, dtype, max_ctx=max_ctx,
                              min_ctx=0)
    say(f"fused {case} ctx={b.pool.context_lens.tolist()}")
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"],
                                     dev["block_tables"], dev["context_lens"], dev["k_new"],
                                     dev["v_new"], dev["slot_mapping"], b.scale, b.max_ctx,
                                     partition_size=partition, algo=algo)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(b)                      # the oracle's store, then its decode
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert W.host_bits(dev["v_cache"]).tobytes() == vc.tobytes()
    want = oracle_decode(b, caches=(kc, vc))
    assert_close(out.float().cpu().double().numpy(), want, dtype, f"fused {algo} p={partition}")


def test_decode_store_fused_tiny_and_qwen3_layer():
    for b in (W.tiny().batches[0], W.qwen3_decode(layers=1).batches[0]):
        dev = to_device(b)
        out = torch.empty_like(dev["q"])
        pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"],
                                         dev["block_tables"], dev["context_lens"], dev["k_new"],
                                         dev["v_new"], dev["slot_mapping"], b.scale, b.max_ctx)
        torch.cuda.synchronize()
        kc, vc = oracle_caches(b)
        assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
        assert_close(out.float().cpu().double().numpy(), oracle_decode(b, caches=(kc, vc)),
                     b.q.dtype, "fused workload")


def test_split_k_counters_reset_across_calls_and_shapes():
    """The partitions' arrival counters come back to zero: one workspace
    serves repeated split-K calls of different shapes bit-identically."""
    b1 = W.random_decode_batch(91, 20, 32, 8, 128, torch.bfloat16, max_ctx=2000, min_ctx=0, store=False)
    b2 = W.random_decode_batch(92, 33, 32, 8, 128, torch.bfloat16, max_ctx=700, min_ctx=0, store=False)
    need = max(pkv.decode_workspace_size(b.num_seqs, 32, 8, 128, 2000, 64) for b in (b1, b2))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    d1, d2 = to_device(b1), to_device(b2)

    def run(b, dev, part):
        out = torch.empty_like(dev["q"])
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                   workspace=ws)
        torch.cuda.synchronize()
        return out.float().cpu().double().numpy()

    first = run(b1, d1, 64)
    assert_close(first, oracle_decode(b1, store=False), torch.bfloat16, "first")
    assert_close(run(b2, d2, 128), oracle_decode(b2, store=False), torch.bfloat16, "second shape")
    for _ in range(3):
        np.testing.assert_array_equal(run(b1, d1, 64), first)
    assert int(ws[:65536 * 4].view(torch.int32).abs().sum()) == 0


def test_split_k_graph_replays_match_eager():
    b = W.random_decode_batch(93, 40, 16, 8, 128, torch.bfloat16, max_ctx=1024, min_ctx=64, store=False)
    dev = to_device(b)
    out = torch.empty_like(dev["q"])
    call = pkv.DecodeLaunch(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                            dev["context_lens"], b.scale, b.max_ctx, partition_size=256)
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
    assert_close(want.float().cpu().double().numpy(), oracle_decode(b, store=False), torch.bfloat16, "graph")
