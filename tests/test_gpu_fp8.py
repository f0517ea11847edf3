"""GPU parity of the E4M3 KV cache against the float64 oracle, through the C
ABI: the quantising store bit for bit, and decode over E4M3 caches within the
bf16 tolerance."""

import numpy as np
import pytest
import torch

from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, say

pytestmark = pytest.mark.gpu


def _dev(b):
    d = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale")}
    d["block_tables"] = torch.as_tensor(b.pool.block_tables, device="cuda")
    d["context_lens"] = torch.as_tensor(b.pool.context_lens, device="cuda")
    if b.k_new is not None:
        for k in ("k_new", "v_new", "slot_mapping"):
            d[k] = getattr(b, k).to("cuda")
    return d


def _oracle_caches(b, store=True):
    kc, vc = W.host_bits(b.k_cache), W.host_bits(b.v_cache)
    if store and b.k_new is not None:
        kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), kc, vc,
                                        W.host_bits(b.slot_mapping), W.host_bits(b.k_scale),
                                        W.host_bits(b.v_scale), b.block_size)
    return kc, vc


def _oracle_decode(b, caches, seqs=None):
    kc, vc = caches
    q, bt, ctx = W.host_bits(b.q), b.pool.block_tables, b.pool.context_lens
    if seqs is not None:
        q, bt, ctx = q[seqs], bt[seqs], ctx[seqs]
    return FP8.paged_attention_decode_fp8(q, kc, vc, W.host_bits(b.k_scale), W.host_bits(b.v_scale),
                                          bt, ctx, b.scale, b.block_size)


def _gpu_decode(b, d, partition=0):
    out = torch.empty_like(d["q"])
    pkv.paged_attention_decode_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                   d["block_tables"], d["context_lens"], b.scale, b.max_ctx,
                                   partition_size=partition)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


EDGE = np.array([0.0, -0.0, 1.0, -1.0, 447.9, 448.0, 449.0, 464.0, 1e4, -1e4, np.inf, -np.inf, np.nan,
                 2.0 ** -10, -2.0 ** -10, 1.5 * 2.0 ** -9, 2.0 ** -12, -2.0 ** -12, 1.0625, 1.1875,
                 -3.3, 0.07, 250.0, 1e-30], np.float32)


@pytest.mark.parametrize("src", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("hkv,d", [(8, 128), (2, 64), (3, 40)])
def test_store_is_bit_exact(src, hkv, d):
    rng = np.random.default_rng(hkv * 100 + d)
    nb, bs, t = 40, 16, 300
    x = rng.normal(0, 4, (2, t, hkv, d)).astype(np.float32)
    x[0, :2].reshape(-1)[:len(EDGE)] = EDGE                      # special values, divided by scale 1
    k = torch.from_numpy(x[0]).to(src)
    v = torch.from_numpy(x[1]).to(src)
    ks = torch.from_numpy(rng.uniform(0.005, 0.05, hkv).astype(np.float32))
    vs = torch.from_numpy(rng.uniform(0.005, 0.05, hkv).astype(np.float32))
    ks[0] = 1.0
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[5::37] = -1
    kc = torch.from_numpy(rng.integers(0, 256, (nb, bs, hkv, d)).astype(np.uint8))
    vc = torch.from_numpy(rng.integers(0, 256, (nb, bs, hkv, d)).astype(np.uint8))
    want_k, want_v = FP8.kv_cache_store_fp8(W.host_bits(k), W.host_bits(v), kc.numpy(), vc.numpy(), slots,
                                            ks.numpy(), vs.numpy(), bs)
    dk, dv = kc.cuda(), vc.cuda()
    say(f"fp8 store src={src} hkv={hkv} d={d}")
    pkv.kv_cache_store_fp8(k.cuda(), v.cuda(), dk, dv, torch.from_numpy(slots).cuda(), ks.cuda(), vs.cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dk.cpu().numpy(), want_k)
    np.testing.assert_array_equal(dv.cpu().numpy(), want_v)


SWEEP = [
    # (hq, hkv, d, max_ctx, block_size)
    (16, 8, 128, 600, 16),
    (32, 8, 128, 1500, 16),
    (8, 8, 128, 300, 32),
    (32, 2, 128, 700, 16),
    (12, 4, 64, 500, 16),
    (64, 4, 64, 400, 48),
]


@pytest.mark.parametrize("case", SWEEP, ids=lambda c: f"{c[0]}x{c[1]}-d{c[2]}-bs{c[4]}")
@pytest.mark.parametrize("partition", [0, 64, 256])
def test_store_then_decode(case, partition):
    hq, hkv, d, max_ctx, bs = case
    b = W.random_decode_batch_fp8(hq * 7 + d + max_ctx, 10, hq, hkv, d, max_ctx=max_ctx, min_ctx=0,
                                  block_size=bs)
    say(f"fp8 decode {case} p={partition} ctx={b.pool.context_lens.tolist()}")
    dv = _dev(b)
    pkv.kv_cache_store_fp8(dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], dv["slot_mapping"],
                           dv["k_scale"], dv["v_scale"])
    caches = _oracle_caches(b)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(dv["k_cache"].cpu().numpy(), caches[0])
    got = _gpu_decode(b, dv, partition)
    assert_close(got, _oracle_decode(b, caches), torch.bfloat16, f"fp8 p={partition}")


def test_empty_and_one_token_contexts():
    b = W.random_decode_batch_fp8(501, 9, 32, 8, 128, max_ctx=3, min_ctx=0, store=False)
    b.pool.context_lens[:3] = 0
    b.pool.context_lens[3:6] = 1
    dv = _dev(b)
    got = _gpu_decode(b, dv)
    assert (got[:3] == 0).all()
    assert_close(got, _oracle_decode(b, _oracle_caches(b, store=False)), torch.bfloat16, "short")


def test_out_of_pool_block_poisons_the_row():
    b = W.random_decode_batch_fp8(503, 5, 16, 8, 128, max_ctx=300, min_ctx=100, store=False)
    b.pool.block_tables[1, 2] = b.pool.num_blocks + 1
    got = _gpu_decode(b, _dev(b))
    assert np.isnan(got[1]).all()
    want = _oracle_decode(b, _oracle_caches(b, store=False), seqs=[0, 2, 3, 4])
    assert_close(got[[0, 2, 3, 4]], want, torch.bfloat16, "beside the bad row")


def test_deterministic():
    b = W.random_decode_batch_fp8(505, 12, 32, 8, 128, max_ctx=900, min_ctx=1, store=False)
    dv = _dev(b)
    np.testing.assert_array_equal(_gpu_decode(b, dv, 128), _gpu_decode(b, dv, 128))


@pytest.mark.slow
def test_qwen3_fp8_layer():
    b = W.qwen3_decode_fp8(layers=1).batches[0]
    dv = _dev(b)
    pkv.kv_cache_store_fp8(dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], dv["slot_mapping"],
                           dv["k_scale"], dv["v_scale"])
    caches = _oracle_caches(b)
    got = _gpu_decode(b, dv)
    assert_close(got, _oracle_decode(b, caches), torch.bfloat16, "qwen3 fp8 layer")


FUSED = [
    # (hq, hkv, d, max_ctx, partition)
    (16, 8, 128, 700, 0),
    (32, 8, 128, 1500, 256),
    (12, 4, 64, 400, 0),
    (32, 2, 128, 500, 64),
]


@pytest.mark.parametrize("case", FUSED, ids=lambda c: f"{c[0]}x{c[1]}-d{c[2]}-p{c[4]}")
def test_decode_store_fused(case):
    hq, hkv, d, max_ctx, partition = case
    b = W.random_decode_batch_fp8(hq * 11 + d + partition, 13, hq, hkv, d, max_ctx=max_ctx, min_ctx=0)
    b.slot_mapping[3] = -1                       # padding: nothing stored, the cache row is read
    say(f"fp8 fused {case}")
    dv = _dev(b)
    out = torch.empty_like(dv["q"])
    pkv.paged_attention_decode_store_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["k_scale"],
                                         dv["v_scale"], dv["block_tables"], dv["context_lens"], dv["k_new"],
                                         dv["v_new"], dv["slot_mapping"], b.scale, b.max_ctx,
                                         partition_size=partition)
    torch.cuda.synchronize()
    caches = _oracle_caches(b)
    np.testing.assert_array_equal(dv["k_cache"].cpu().numpy(), caches[0])
    np.testing.assert_array_equal(dv["v_cache"].cpu().numpy(), caches[1])
    got = out.float().cpu().double().numpy()
    live = [s for s in range(13) if s != 3]
    assert_close(got[live], _oracle_decode(b, caches, seqs=live), torch.bfloat16, "fp8 fused")
    if b.pool.context_lens[3] > 0:
        assert np.isnan(got[3]).all()            # its newest row is a poisoned cache row


# ---- chunked prefill over E4M3 caches ------------------------------------------

def _gpu_prefill(b, d, causal=True):
    pkv.kv_cache_store_fp8(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"],
                           d["k_scale"], d["v_scale"])
    out = torch.full_like(d["q"], float("nan"))   # a row no workgroup writes stays NaN
    cu = torch.as_tensor(b.cu_seqlens_q, device="cuda")
    pkv.paged_attention_prefill_chunk_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"],
                                          d["v_scale"], d["block_tables"], cu, d["context_lens"],
                                          b.scale, int(np.diff(b.cu_seqlens_q).max()), b.max_ctx,
                                          causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def _oracle_prefill(b, caches, causal=True):
    kc, vc = caches
    return FP8.paged_attention_prefill_chunk_fp8(W.host_bits(b.q), kc, vc, W.host_bits(b.k_scale),
                                                 W.host_bits(b.v_scale), b.pool.block_tables,
                                                 b.cu_seqlens_q, b.pool.context_lens, b.scale,
                                                 b.block_size, causal=causal)


PREFILL = [
    # (hq, hkv, chunks, max_rows, max_prior, block_size)
    (32, 8, 3, 150, 300, 16),
    (16, 8, 4, 70, 90, 16),
    (8, 8, 2, 200, 20, 32),
    (32, 4, 3, 40, 200, 64),
    (8, 1, 2, 33, 64, 16),
    (32, 8, 9, 4, 1500, 16),     # verification-sized chunks
]


@pytest.mark.parametrize("case", PREFILL, ids=lambda c: f"{c[0]}x{c[1]}-r{c[3]}-p{c[4]}-bs{c[5]}")
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_fp8_matches_oracle(case, causal):
    hq, hkv, chunks, max_rows, max_prior, bs = case
    b = W.random_prefill_batch_fp8(hq * 11 + max_rows + bs, chunks, hq, hkv, 128, max_rows=max_rows,
                                   max_prior=max_prior, block_size=bs)
    say(f"prefill fp8 {case} causal={causal} rows={np.diff(b.cu_seqlens_q).tolist()} "
        f"ctx={b.pool.context_lens.tolist()}")
    d = _dev(b)
    got = _gpu_prefill(b, d, causal=causal)
    assert_close(got, _oracle_prefill(b, _oracle_caches(b), causal=causal), torch.bfloat16,
                 f"prefill fp8 causal={causal}")


def test_prefill_fp8_rows_match_fp8_decode():
    """Row i of a chunk after P0 cached tokens is single-query decode over the
    first P0 + i + 1 keys: both the chunked prefill and the E4M3 decode kernel
    (one context length per row) match the oracle's E4M3 decode run row by
    row with those lengths."""
    b = W.random_prefill_batch_fp8(77, 5, 32, 8, 128, max_rows=6, min_rows=6, max_prior=700)
    d = _dev(b)
    got = _gpu_prefill(b, d)
    cu, ctx = b.cu_seqlens_q, b.pool.context_lens
    seq = np.repeat(np.arange(len(ctx)), 6)
    row_ctx = np.concatenate([ctx[c] - 6 + 1 + np.arange(6) for c in range(len(ctx))]).astype(np.int32)
    bt = np.ascontiguousarray(b.pool.block_tables[seq])
    out = torch.full_like(d["q"], float("nan"))
    pkv.paged_attention_decode_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                   torch.as_tensor(bt, device="cuda"), torch.as_tensor(row_ctx, device="cuda"),
                                   b.scale, int(row_ctx.max()))
    torch.cuda.synchronize()
    dec = out.float().cpu().double().numpy()
    assert cu[-1] == len(row_ctx)
    kc, vc = _oracle_caches(b)
    want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), kc, vc, W.host_bits(b.k_scale),
                                          W.host_bits(b.v_scale), bt, row_ctx, b.scale, b.block_size)
    assert_close(got, want, torch.bfloat16, "prefill rows vs the oracle's per-row decode")
    assert_close(dec, want, torch.bfloat16, "decode per row vs the oracle")


def test_prefill_fp8_out_of_pool_block_poisons_its_chunk():
    b = W.random_prefill_batch_fp8(79, 3, 32, 8, 128, max_rows=60, max_prior=80)
    d = _dev(b)
    bt = b.pool.block_tables.copy()
    bt[1, 0] = b.pool.num_blocks + 3
    d["block_tables"] = torch.as_tensor(bt, device="cuda")
    got = _gpu_prefill(b, d)
    cu = b.cu_seqlens_q
    assert np.isnan(got[cu[1]:cu[2]]).all()
    want = _oracle_prefill(b, _oracle_caches(b))
    for c in (0, 2):
        assert_close(got[cu[c]:cu[c + 1]], want[cu[c]:cu[c + 1]], torch.bfloat16, f"chunk {c}")



def test_store_and_prefill_fp8_graph_replays_match_eager():
    """The quantising store and the E4M3 prefill captured in one HIP graph:
    four replays (output reset to NaN, eager work in between) give the eager
    call's bits, which match the oracle."""
    b = W.random_prefill_batch_fp8(613, 4, 32, 8, 128, max_rows=150, max_prior=400)
    say(f"graph prefill fp8 rows={np.diff(b.cu_seqlens_q).tolist()} ctx={b.pool.context_lens.tolist()}")
    d = _dev(b)
    out = torch.full_like(d["q"], float("nan"))
    cu = torch.as_tensor(b.cu_seqlens_q, device="cuda")
    store = pkv.StoreFp8Launch(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"],
                               d["k_scale"], d["v_scale"])
    pre = pkv.PrefillFp8Launch(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                               d["block_tables"], cu, d["context_lens"], b.scale,
                               int(np.diff(b.cu_seqlens_q).max()), b.max_ctx, causal=True)

    def step():
        store()
        pre()

    step()
    torch.cuda.synchronize()
    want = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.zeros(1 << 20, device="cuda")
    for i in range(4):
        out.fill_(float("nan"))
        scratch.add_(1.0)   # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {i}"
    assert_close(want.float().cpu().double().numpy(), _oracle_prefill(b, _oracle_caches(b)), torch.bfloat16,
                 "graph prefill fp8")
