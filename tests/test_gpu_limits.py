"""Sizes at the edges of what the library accepts, against the float64 oracle
on every output row (outputs start as NaN, so a row that no workgroup writes
fails):

* very long contexts (262,144 tokens, a ragged 131,071, 40,000 and the
  degenerate 0, 1 and 17) in every decode launch mode, over bf16 and E4M3
  caches, split-K down to 16-token partitions (16,384 partials merged per
  row);
* prefill chunks after up to 200,000 cached tokens, bf16 and E4M3;
* more prefill (chunk, q-tile) items than the kernel ranks in LDS (8192),
  which hands the items out in the unranked order;
* the largest batch the host accepts, 65,535 sequences, in the single-pass,
  planned and split-K decodes; the work-balanced decode refuses it.

Every case first stores its new rows on the GPU and checks the caches bit
for bit against the oracle's store.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests import full_size
from tests.gpu_helpers import assert_close, oracle_caches, say, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_CACHE = {}


def _one(name, make):
    """One case at a time: its host batch, device tensors and oracle result."""
    if name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[name] = make()
    return _CACHE[name]


def _stored(b):
    """Device tensors of batch b with its new rows stored on the GPU, and the
    oracle's caches (plus scales for E4M3), checked equal bit for bit."""
    fp8 = b.k_scale is not None
    if fp8:
        d = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "k_new",
                                                    "v_new", "slot_mapping")}
        d["block_tables"] = torch.as_tensor(b.pool.block_tables, device="cuda")
        d["context_lens"] = torch.as_tensor(b.pool.context_lens, device="cuda")
        if b.cu_seqlens_q is not None:
            d["cu_seqlens_q"] = torch.as_tensor(b.cu_seqlens_q, device="cuda")
        pkv.kv_cache_store_fp8(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"],
                               d["k_scale"], d["v_scale"])
        ks, vs = W.host_bits(b.k_scale), W.host_bits(b.v_scale)
        kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                        W.host_bits(b.v_cache), W.host_bits(b.slot_mapping), ks, vs,
                                        b.block_size)
        scales = dict(k_scale=ks, v_scale=vs)
    else:
        d = to_device(b)
        pkv.kv_cache_store(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"])
        kc, vc = oracle_caches(b)
        scales = {}
    torch.cuda.synchronize()
    assert np.array_equal(W.host_bits(d["k_cache"]), kc), "K cache after the store"
    assert np.array_equal(W.host_bits(d["v_cache"]), vc), "V cache after the store"
    return d, kc, vc, scales


def _decode_entry(b):
    d, kc, vc, scales = _stored(b)
    say(f"  oracle over {b.num_seqs} sequences on {full_size.workers()} host workers")
    want = full_size.decode(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.pool.context_lens, b.scale,
                            b.block_size, **scales)
    return b, d, want


def _prefill_entry(b, workers=True):
    """workers=False runs the oracle in this process: one call over all
    chunks, which for many tiny chunks beats a task per (chunk, kv-head)."""
    d, kc, vc, scales = _stored(b)
    args = (W.host_bits(b.q), kc, vc, b.pool.block_tables, b.cu_seqlens_q, b.pool.context_lens, b.scale,
            b.block_size)
    if workers:
        say(f"  oracle over {len(b.cu_seqlens_q) - 1} chunks on {full_size.workers()} host workers")
        want = full_size.prefill(*args, causal=True, **scales)
    elif scales:
        want = FP8.paged_attention_prefill_chunk_fp8(args[0], kc, vc, scales["k_scale"], scales["v_scale"],
                                                     *args[3:], causal=True)
    else:
        want = oracle.paged_attention_prefill_chunk(*args, causal=True)
    return b, d, want


def _run_decode(b, d, algo, part):
    out = torch.full_like(d["q"], float("nan"))
    ws = None
    if part == "planned":
        ws = pkv.new_decode_plan(b.num_seqs, "cuda")
        pkv.decode_plan(ws, d["block_tables"], d["context_lens"], b.max_ctx, b.block_size)
    if b.k_scale is not None:
        pkv.paged_attention_decode_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                       d["block_tables"], d["context_lens"], b.scale, b.max_ctx,
                                       partition_size=part, workspace=ws)
    else:
        pkv.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], b.scale, b.max_ctx, partition_size=part, workspace=ws,
                                   algo=algo)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def _run_prefill(b, d):
    out = torch.full_like(d["q"], float("nan"))
    mq = int(np.diff(b.cu_seqlens_q).max())
    if b.k_scale is not None:
        pkv.paged_attention_prefill_chunk_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"],
                                              d["v_scale"], d["block_tables"], d["cu_seqlens_q"],
                                              d["context_lens"], b.scale, mq, b.max_ctx, causal=True)
    else:
        pkv.paged_attention_prefill_chunk(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                          d["cu_seqlens_q"], d["context_lens"], b.scale, mq, b.max_ctx,
                                          causal=True)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


# ---- very long contexts: 8 q / 2 kv heads, D 128 --------------------------------------------

LONG_CTX = [262144, 131071, 1, 0, 40000, 17]
LONG_MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", 16), ("mfma", 512), ("mfma", 4096), ("mfma", "balanced"),
              ("mfma", "auto"), ("valu", 0), ("valu", 16), ("valu", 512)]


@pytest.mark.parametrize("mode", LONG_MODES, ids=lambda m: f"{m[0]}-{m[1]}")
def test_very_long_contexts_bf16(mode):
    b, d, want = _one("long_bf16", lambda: _decode_entry(
        W.decode_batch_of_lengths(7100, LONG_CTX, 8, 2, 128, torch.bfloat16)))
    say(f"long contexts {LONG_CTX} bf16 {mode}")
    got = _run_decode(b, d, *mode)
    assert_close(got, want, torch.bfloat16, f"long bf16 {mode}")
    assert (got[np.asarray(LONG_CTX) == 0] == 0).all()


@pytest.mark.parametrize("part", [0, "planned", 2048, "auto"])
def test_very_long_contexts_e4m3(part):
    b, d, want = _one("long_e4m3", lambda: _decode_entry(
        W.decode_batch_of_lengths(7200, LONG_CTX, 8, 2, 128, "e4m3")))
    say(f"long contexts {LONG_CTX} E4M3 p={part}")
    got = _run_decode(b, d, "mfma", part)
    assert_close(got, want, torch.bfloat16, f"long E4M3 p={part}")
    assert (got[np.asarray(LONG_CTX) == 0] == 0).all()


# ---- prefill after long cached contexts -----------------------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, "e4m3"], ids=["bf16", "e4m3"])
def test_prefill_after_200k_cached_tokens(dtype):
    rows, priors = [100, 5, 64], [200000, 0, 70000]
    b, d, want = _one(f"prefill_long_{dtype}", lambda: _prefill_entry(
        W.prefill_batch_of_lengths(7300, rows, priors, 8, 2, 128, dtype)))
    say(f"prefill rows {rows} after {priors} cached tokens, {dtype}")
    assert_close(_run_prefill(b, d), want, torch.bfloat16, f"long prefill {dtype}")


# ---- more (chunk, q-tile) items than the kernel ranks ----------------------------------------

@pytest.mark.parametrize("dtype", [torch.bfloat16, "e4m3"], ids=["bf16", "e4m3"])
def test_prefill_past_the_ranking_limit(dtype):
    """8300 chunks of 1-3 rows at 8 q / 2 kv heads: one 32-row q-tile per
    chunk, so 8300 items, past the 8192 the kernel ranks in LDS."""
    def make():
        rng = np.random.default_rng(7400)
        rows = rng.integers(1, 3, size=8300, endpoint=True)
        priors = rng.integers(0, 100, size=8300, endpoint=True)
        return _prefill_entry(W.prefill_batch_of_lengths(7400, rows, priors, 8, 2, 128, dtype), workers=False)
    b, d, want = _one(f"prefill_many_{dtype}", make)
    num_q_tiles = -(-int(np.diff(b.cu_seqlens_q).max()) // 32)
    assert num_q_tiles * (len(b.cu_seqlens_q) - 1) > 8192
    say(f"prefill of 8300 short chunks, {dtype}")
    assert_close(_run_prefill(b, d), want, torch.bfloat16, f"8300 chunks {dtype}")


# ---- the largest batch: 65,535 sequences, ctx U{0..40}, 4 q / 1 kv head, D 64 ---------------

MANY_MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", 16), ("mfma", "auto"), ("valu", 0), ("valu", 16)]


@pytest.mark.parametrize("mode", MANY_MODES, ids=lambda m: f"{m[0]}-{m[1]}")
def test_largest_batch(mode):
    b, d, want = _one("many", lambda: _decode_entry(
        W.random_decode_batch(7500, 65535, 4, 1, 64, torch.bfloat16, max_ctx=40, min_ctx=0)))
    say(f"65535 sequences {mode}")
    got = _run_decode(b, d, *mode)
    assert_close(got, want, torch.bfloat16, f"65535 seqs {mode}")
    assert (got[b.pool.context_lens == 0] == 0).all()


def test_largest_batch_is_refused_by_the_work_balanced_decode():
    b, d, _ = _one("many", lambda: _decode_entry(
        W.random_decode_batch(7500, 65535, 4, 1, 64, torch.bfloat16, max_ctx=40, min_ctx=0)))
    out = torch.full_like(d["q"], float("nan"))
    with pytest.raises(pkv.PkvError, match="8192"):
        pkv.paged_attention_decode(out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"],
                                   d["context_lens"], b.scale, b.max_ctx, partition_size="balanced",
                                   algo="mfma")
    torch.cuda.synchronize()
    assert torch.isnan(out).all()   # refused on the host: nothing ran
