"""Non-finite values inside live cache rows, against the float64 oracle.

By the definition, a NaN in a visible key makes every weight of its rows
NaN, so those rows are NaN in every column; an infinite value element of a
visible row makes that column non-finite (an infinity, or NaN where it
meets a zero weight or an infinity of the other sign). The kernels must
give the same pattern: each output element is non-finite exactly where the
oracle's is, and the finite elements agree within the bf16 bound. Whether a
non-finite element is an infinity or a NaN is not compared: a weight that
the oracle keeps as a tiny positive number may round to zero in bf16, which
turns inf into NaN.

Planted (all in live rows, the new rows stored first): a NaN in one K
element, +inf and -inf in V elements of the same column of one sequence,
and +inf in a V element of another; E4M3 caches have no infinity, so there
only NaN codes are planted, in K and in V.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import TOL, oracle_caches, say, to_device

# the oracle's sums meet the planted NaN and infinities on purpose
pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore:invalid value encountered:RuntimeWarning")]


def _slot(b, s, pos):
    blk = int(b.pool.block_tables[s][pos // b.block_size])
    return blk, pos % b.block_size


def _plant(b, rng, specs):
    """specs: (cache 'k' or 'v', value) per planted element, each in a random
    live row of a random sequence with context; returns what was planted."""
    live = [s for s in range(len(b.pool.context_lens)) if b.pool.context_lens[s] > 1]
    hkv, d = b.k_cache.shape[2], b.k_cache.shape[3]
    done = []
    for which, value in specs:
        s = int(rng.choice(live))
        pos = int(rng.integers(0, int(b.pool.context_lens[s]) - 1))   # not the new row (position ctx-1)
        g, col = int(rng.integers(0, hkv)), int(rng.integers(0, d))
        blk, row = _slot(b, s, pos)
        cache = b.k_cache if which == "k" else b.v_cache
        if cache.dtype == torch.uint8:
            cache[blk, row, g, col] = value
        else:
            cache[blk, row, g, col] = float(value)
        done.append((which, s, pos, g, col, value))
    return done


def _compare(got, want, what):
    bad_got, bad_want = ~np.isfinite(got), ~np.isfinite(want)
    say(f"  {what}: {int(bad_want.sum())} non-finite elements in the oracle, {int(bad_got.sum())} in the kernel")
    assert bad_want.any(), "the planted values must reach the output"
    np.testing.assert_array_equal(bad_got, bad_want, err_msg=f"{what}: non-finite pattern")
    err = np.abs(got[~bad_want] - want[~bad_want]).max()
    assert err <= TOL[torch.bfloat16], f"{what}: max abs error {err}"


def _same_column_pair(b, rng):
    """+inf and -inf in V at the same (kv-head, column) of one sequence: that
    column of its heads is NaN by the definition."""
    s = int(np.argmax(b.pool.context_lens))
    g, col = int(rng.integers(0, b.v_cache.shape[2])), int(rng.integers(0, b.v_cache.shape[3]))
    for pos, value in ((0, float("inf")), (1, float("-inf"))):
        blk, row = _slot(b, s, pos)
        b.v_cache[blk, row, g, col] = value


MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", 256), ("mfma", "balanced"), ("valu", 0), ("valu", 256)]


def test_decode_bf16_every_mode():
    b = W.random_decode_batch(8500, 16, 32, 8, 128, torch.bfloat16, max_ctx=800, min_ctx=2, store=True)
    rng = np.random.default_rng(8501)
    planted = _plant(b, rng, [("k", float("nan")), ("v", float("inf")), ("v", float("-inf"))])
    _same_column_pair(b, rng)
    say(f"planted {planted}")
    dev = to_device(b)
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
    kc, vc = oracle_caches(b)
    want = oracle.paged_attention_decode(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.pool.context_lens,
                                         b.scale, b.block_size)
    for algo, part in MODES:
        ws = None
        if part == "planned":
            ws = pkv.new_decode_plan(b.num_seqs, "cuda")
            pkv.decode_plan(ws, dev["block_tables"], dev["context_lens"], b.max_ctx, b.block_size)
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part, workspace=ws,
                                   algo=algo)
        torch.cuda.synchronize()
        _compare(out.float().cpu().double().numpy(), want, f"{algo} {part}")


def test_decode_e4m3_every_mode():
    b = W.random_decode_batch_fp8(8600, 16, 32, 8, 128, max_ctx=800, min_ctx=2, store=False)
    rng = np.random.default_rng(8601)
    planted = _plant(b, rng, [("k", W.E4M3_NAN), ("v", W.E4M3_NAN), ("v", 0xFF)])   # 0xff: NaN, sign set
    say(f"planted {planted}")
    want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), W.host_bits(b.k_cache), W.host_bits(b.v_cache),
                                          W.host_bits(b.k_scale), W.host_bits(b.v_scale), b.pool.block_tables,
                                          b.pool.context_lens, b.scale, b.block_size)
    dv = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale")}
    bt = torch.as_tensor(b.pool.block_tables, device="cuda")
    cl = torch.as_tensor(b.pool.context_lens, device="cuda")
    for part in (0, "planned", 256):
        ws = None
        if part == "planned":
            ws = pkv.new_decode_plan(b.num_seqs, "cuda")
            pkv.decode_plan(ws, bt, cl, b.max_ctx, b.block_size)
        out = torch.full_like(dv["q"], float("nan"))
        pkv.paged_attention_decode_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["k_scale"], dv["v_scale"],
                                       bt, cl, b.scale, b.max_ctx, partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        _compare(out.float().cpu().double().numpy(), want, f"E4M3 p={part}")


def test_prefill_bf16():
    b = W.random_prefill_batch(8700, 4, 32, 8, 128, torch.bfloat16, max_rows=100, max_prior=300, min_rows=2)
    rng = np.random.default_rng(8701)
    # cached positions only (the chunks' own rows are stored over any plant)
    prior = b.pool.context_lens - np.diff(b.cu_seqlens_q)
    hkv, d = b.k_cache.shape[2], b.k_cache.shape[3]
    planted = []
    for which, value in (("k", float("nan")), ("v", float("inf")), ("v", float("-inf"))):
        c = int(rng.choice([c for c in range(len(prior)) if prior[c] > 0]))
        pos = int(rng.integers(0, int(prior[c])))
        g, col = int(rng.integers(0, hkv)), int(rng.integers(0, d))
        blk, row = _slot(b, c, pos)
        (b.k_cache if which == "k" else b.v_cache)[blk, row, g, col] = value
        planted.append((which, c, pos, g, col, value))
    say(f"planted {planted}")
    dv = to_device(b)
    pkv.kv_cache_store(dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], dv["slot_mapping"])
    kc, vc = oracle_caches(b)
    mq = int(np.diff(b.cu_seqlens_q).max())
    for causal in (True, False):
        want = oracle.paged_attention_prefill_chunk(W.host_bits(b.q), kc, vc, b.pool.block_tables,
                                                    b.cu_seqlens_q, b.pool.context_lens, b.scale, b.block_size,
                                                    causal=causal)
        out = torch.full_like(dv["q"], float("nan"))
        pkv.paged_attention_prefill_chunk(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                          dv["cu_seqlens_q"], dv["context_lens"], b.scale, mq, b.max_ctx,
                                          causal=causal)
        torch.cuda.synchronize()
        _compare(out.float().cpu().double().numpy(), want, f"prefill causal={causal}")
