"""GPU parity of paged_attention_prefill_chunk against the float64 oracle,
through the C ABI (bf16, head_dim 128, causal and non-causal)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_caches, say, to_device

pytestmark = pytest.mark.gpu


def gpu_prefill(b, dev=None, causal=True, store=True):
    dev = dev or to_device(b)
    if store and b.k_new is not None:
        pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                           dev["slot_mapping"])
    out = torch.full_like(dev["q"], float("nan"))   # a row no workgroup writes stays NaN
    cu = b.cu_seqlens_q
    pkv.paged_attention_prefill_chunk(out, dev["q"], dev["k_cache"], dev["v_cache"],
                                      dev["block_tables"], dev["cu_seqlens_q"],
                                      dev["context_lens"], b.scale, int(np.diff(cu).max()),
                                      b.max_ctx, causal=causal)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def oracle_prefill(b, caches=None, causal=True, rows=None):
    kc, vc = caches if caches is not None else oracle_caches(b)
    q = W.host_bits(b.q)
    return oracle.paged_attention_prefill_chunk(q, kc, vc, b.pool.block_tables, b.cu_seqlens_q,
                                                b.pool.context_lens, b.scale, b.block_size,
                                                causal=causal)


CASES = [
    # (hq, hkv, chunks, max_rows, max_prior)
    (128, 8, 3, 70, 300),      # G = 16: 8 query rows per workgroup
    (32, 8, 3, 150, 300),
    (16, 8, 4, 70, 90),
    (8, 8, 2, 200, 20),
    (32, 4, 3, 40, 200),
    (8, 1, 2, 33, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}-r{c[3]}-p{c[4]}")
@pytest.mark.parametrize("causal", [True, False])
def test_random_chunks(case, causal):
    hq, hkv, chunks, max_rows, max_prior = case
    b = W.random_prefill_batch(hq * 7 + max_rows, chunks, hq, hkv, 128, torch.bfloat16,
                               max_rows=max_rows, max_prior=max_prior)
    say(f"prefill {case} causal={causal} rows={np.diff(b.cu_seqlens_q).tolist()} "
        f"ctx={b.pool.context_lens.tolist()}")
    got = gpu_prefill(b, causal=causal)
    assert_close(got, oracle_prefill(b, causal=causal), torch.bfloat16, f"prefill causal={causal}")


@pytest.mark.parametrize("bs", [32, 64, 128, 256])
def test_larger_blocks(bs):
    # contexts span several 64-key tiles per block (whole-tile gather at each
    # 64-key offset inside a block) and end in a ragged tile
    b = W.random_prefill_batch(50 + bs, 3, 32, 8, 128, torch.bfloat16, max_rows=100,
                               max_prior=150 if bs <= 64 else 700, block_size=bs)
    assert_close(gpu_prefill(b), oracle_prefill(b), torch.bfloat16, f"bs={bs}")


def test_single_row_chunk_matches_decode():
    b = W.random_prefill_batch(61, 4, 32, 8, 128, torch.bfloat16, max_rows=1, max_prior=700)
    dev = to_device(b)
    got = gpu_prefill(b, dev=dev)
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                               dev["context_lens"], b.scale, b.max_ctx)
    torch.cuda.synchronize()
    dec = out.float().cpu().double().numpy()
    # both within tolerance of the oracle, and of each other
    want = oracle_prefill(b)
    assert_close(got, want, torch.bfloat16, "prefill L=1")
    assert_close(dec, want, torch.bfloat16, "decode")


def test_first_row_without_prior_returns_v_row():
    b = W.random_prefill_batch(67, 2, 16, 8, 128, torch.bfloat16, max_rows=40, max_prior=0)
    got = gpu_prefill(b)
    kc, vc = oracle_caches(b)
    for c in range(2):
        row0 = b.cu_seqlens_q[c]
        v0 = oracle.gather_context(vc, b.pool.block_tables[c], 1, b.block_size)[0]
        np.testing.assert_array_equal(got[row0], np.repeat(v0, 2, axis=0))


def test_deterministic():
    b = W.random_prefill_batch(71, 3, 32, 8, 128, torch.bfloat16, max_rows=130, max_prior=500)
    dev = to_device(b)
    a = gpu_prefill(b, dev=dev)
    c = gpu_prefill(b, dev=dev, store=False)
    np.testing.assert_array_equal(a, c)


def test_out_of_pool_block_poisons_its_chunk():
    b = W.random_prefill_batch(73, 3, 32, 8, 128, torch.bfloat16, max_rows=60, max_prior=80)
    dev = to_device(b)
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                       dev["slot_mapping"])
    bt = b.pool.block_tables.copy()
    bt[1, 0] = b.pool.num_blocks + 3
    dev["block_tables"] = torch.as_tensor(bt, device="cuda")
    got = gpu_prefill(b, dev=dev, store=False)
    cu = b.cu_seqlens_q
    assert np.isnan(got[cu[1]:cu[2]]).all()
    want = oracle_prefill(b)
    for c in (0, 2):
        assert_close(got[cu[c]:cu[c + 1]], want[cu[c]:cu[c + 1]], torch.bfloat16, f"chunk {c}")


# prior lengths putting each chunk's last rows at every offset just past a
# 16-key tile boundary (and past a 64-key round of the four waves): an early
# row's causal limit then falls before the whole last tile
TILE_EDGE_PRIORS = [0, 1, 13, 14, 15, 30, 31, 45, 46, 47, 61, 62, 63, 126, 127, 240]


@pytest.mark.parametrize("case", [(16, 8, 3), (32, 8, 4), (64, 8, 2), (8, 8, 16), (8, 8, 5), (32, 8, 1)],
                         ids=lambda c: f"{c[0]}x{c[1]}-L{c[2]}")
def test_short_chunks_at_tile_edges(case):
    """Rows of a short chunk whose causal limits end before the last key
    tile (the chunk's rows times the group fill at most one matrix tile)."""
    hq, hkv, rows = case
    b = W.random_prefill_batch(700 + hq + rows, len(TILE_EDGE_PRIORS), hq, hkv, 128, torch.bfloat16,
                               max_rows=rows, min_rows=rows, max_prior=0, priors=TILE_EDGE_PRIORS)
    say(f"tile-edge short chunks {case} ctx={b.pool.context_lens.tolist()}")
    assert_close(gpu_prefill(b), oracle_prefill(b), torch.bfloat16, f"L={rows}")


SHORT = [
    # (hq, hkv, rows): verification of rows-1 drafted tokens, every GQA group
    (32, 8, 2), (32, 8, 4), (32, 8, 8), (16, 8, 3), (8, 8, 5), (32, 4, 7), (8, 1, 6),
]


@pytest.mark.parametrize("case", SHORT, ids=lambda c: f"{c[0]}x{c[1]}-L{c[2]}")
def test_short_chunks_match_decode_over_each_prefix(case):
    """Multi-query decode: row i of an L-row chunk after P0 cached tokens is
    single-query decode over the first P0 + i + 1 keys."""
    hq, hkv, rows = case
    b = W.random_prefill_batch(hq + 13 * rows, 9, hq, hkv, 128, torch.bfloat16,
                               max_rows=rows, min_rows=rows, max_prior=1500)
    say(f"short chunks {case} ctx={b.pool.context_lens.tolist()}")
    dev = to_device(b)
    got = gpu_prefill(b, dev=dev)
    kc, vc = oracle_caches(b)
    assert_close(got, oracle_prefill(b, caches=(kc, vc)), torch.bfloat16, f"L={rows}")
    # the same rows through the decode kernel, one context length per row
    cu, ctx = b.cu_seqlens_q, b.pool.context_lens
    seq = np.repeat(np.arange(len(ctx)), rows)
    row_ctx = np.concatenate([ctx[c] - rows + 1 + np.arange(rows) for c in range(len(ctx))])
    bt = np.ascontiguousarray(b.pool.block_tables[seq])
    out = torch.empty_like(dev["q"])
    pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"],
                               torch.as_tensor(bt, device="cuda"),
                               torch.as_tensor(row_ctx.astype(np.int32), device="cuda"),
                               b.scale, int(row_ctx.max()))
    torch.cuda.synchronize()
    dec = out.float().cpu().double().numpy()
    want = oracle.paged_attention_decode(W.host_bits(b.q), kc, vc, bt, row_ctx, b.scale, 16)
    assert_close(dec, want, torch.bfloat16, "decode per row")
    assert_close(got, want, torch.bfloat16, "chunk vs per-row decode oracle")
    assert cu[-1] == len(row_ctx)



def _replays_match(step, out, label):
    """Runs `step` eagerly, warms it on a side stream, captures it in a HIP
    graph and replays it four times (output reset to NaN and other eager
    work on the stream in between): every replay must give the eager bits."""
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
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"{label}: replay {i}"
    return want


def test_store_and_prefill_graph_replays_match_eager():
    """The store of the chunks' rows and the prefill over them in one graph."""
    b = W.random_prefill_batch(611, 4, 32, 8, 128, torch.bfloat16, max_rows=150, max_prior=400)
    say(f"graph prefill rows={np.diff(b.cu_seqlens_q).tolist()} ctx={b.pool.context_lens.tolist()}")
    dev = to_device(b)
    out = torch.full_like(dev["q"], float("nan"))
    store = pkv.StoreLaunch(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
    pre = pkv.PrefillLaunch(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                            dev["cu_seqlens_q"], dev["context_lens"], b.scale,
                            int(np.diff(b.cu_seqlens_q).max()), b.max_ctx, causal=True)

    def step():
        store()
        pre()

    want = _replays_match(step, out, "bf16 prefill")
    assert_close(want.float().cpu().double().numpy(), oracle_prefill(b), torch.bfloat16, "graph prefill")


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, "e4m3"], ids=["bf16", "e4m3"])
def test_empty_chunks_between_others(causal, dtype):
    """Chunks with no query rows (equal consecutive cu_seqlens_q entries,
    with or without cached context) produce nothing and shift nothing: the
    other chunks' rows match the oracle. An all-empty batch is a no-op."""
    rows, priors = [5, 0, 33, 0, 1, 0], [10, 7, 0, 0, 200, 64]
    b = W.prefill_batch_of_lengths(9200, rows, priors, 32, 8, 128, dtype)
    say(f"empty chunks: rows {rows}, cached {priors}, causal={causal}, {dtype}")
    mq = max(rows)
    if dtype == "e4m3":
        d = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "k_new",
                                                    "v_new", "slot_mapping")}
        bt = torch.as_tensor(b.pool.block_tables, device="cuda")
        cu = torch.as_tensor(b.cu_seqlens_q, device="cuda")
        cl = torch.as_tensor(b.pool.context_lens, device="cuda")
        pkv.kv_cache_store_fp8(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"], d["k_scale"],
                               d["v_scale"])
        ks, vs = W.host_bits(b.k_scale), W.host_bits(b.v_scale)
        kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                        W.host_bits(b.v_cache), W.host_bits(b.slot_mapping), ks, vs, b.block_size)
        want = FP8.paged_attention_prefill_chunk_fp8(W.host_bits(b.q), kc, vc, ks, vs, b.pool.block_tables,
                                                     b.cu_seqlens_q, b.pool.context_lens, b.scale, b.block_size,
                                                     causal=causal)
        out = torch.full_like(d["q"], float("nan"))
        pkv.paged_attention_prefill_chunk_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                              bt, cu, cl, b.scale, mq, b.max_ctx, causal=causal)
    else:
        d = to_device(b)
        pkv.kv_cache_store(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
        want = oracle_prefill(b, causal=causal)
        out = torch.full_like(d["q"], float("nan"))
        pkv.paged_attention_prefill_chunk(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                          d["cu_seqlens_q"], d["context_lens"], b.scale, mq, b.max_ctx,
                                          causal=causal)
        bt, cu, cl = d["block_tables"], d["cu_seqlens_q"], d["context_lens"]
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "rows of the non-empty chunks")

    # every chunk empty: nothing to write, nothing launched that could read
    none = torch.zeros(len(rows) + 1, dtype=torch.int32, device="cuda")
    empty = torch.empty((0,) + tuple(out.shape[1:]), dtype=out.dtype, device="cuda")
    if dtype == "e4m3":
        pkv.paged_attention_prefill_chunk_fp8(empty, empty, d["k_cache"], d["v_cache"], d["k_scale"],
                                              d["v_scale"], bt, none, cl, b.scale, 0, b.max_ctx, causal=causal)
    else:
        pkv.paged_attention_prefill_chunk(empty, empty, d["k_cache"], d["v_cache"], bt, none, cl, b.scale, 0,
                                          b.max_ctx, causal=causal)
    torch.cuda.synchronize()
