"""Every output row of the standard workloads at full size, in every launch
configuration the library offers for them, against the float64 oracle
(through the C ABI). Outputs start as NaN, so a row that no workgroup
writes fails the comparison.

The oracle runs over all rows, spread over host worker processes
(tests/full_size.py); its result for a workload is computed once and
shared by that workload's launch configurations.
"""

import pytest
import torch

from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests import full_size
from tests.gpu_helpers import assert_close, oracle_caches, say, to_device

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

_CACHE = {}


def _one(name, make):
    """One workload at a time: its host batch, device tensors and oracle result."""
    if name not in _CACHE:
        _CACHE.clear()
        torch.cuda.empty_cache()
        _CACHE[name] = make()
    return _CACHE[name]


def _decode_entry(b, store):
    """Host batch -> (device tensors with the store applied, oracle output)."""
    dev = to_device(b)
    if store and b.k_new is not None:
        pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
    kc, vc = oracle_caches(b, store=store)
    say(f"  oracle over {b.num_seqs} sequences on {full_size.workers()} host workers")
    want = full_size.decode(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.pool.context_lens, b.scale,
                            b.block_size)
    torch.cuda.synchronize()
    return b, dev, want


def _run_decode(b, dev, mode):
    """The decode in one launch configuration; mode = (algo, partition)."""
    algo, part = mode
    out = torch.full_like(dev["q"], float("nan"))
    ws = None
    if part == "planned":
        ws = pkv.new_decode_plan(b.num_seqs, "cuda")
        pkv.decode_plan(ws, dev["block_tables"], dev["context_lens"], b.max_ctx, b.block_size)
    pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                               dev["context_lens"], b.scale, b.max_ctx, partition_size=part, workspace=ws,
                               algo=algo)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def _ids(m):
    return f"{m[0]}-{m[1]}"


# ---- decode: the Qwen3-shaped layer (60 seqs, ctx U{64..1024}, 16 q / 8 kv) ------------

QWEN3_MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", 256), ("mfma", "balanced"), ("mfma", "auto"),
               ("valu", 0), ("valu", 256)]


@pytest.mark.parametrize("mode", QWEN3_MODES, ids=_ids)
def test_qwen3_layer_every_row(mode):
    b, dev, want = _one("qwen3", lambda: _decode_entry(W.qwen3_decode(layers=1).batches[0], store=True))
    say(f"qwen3 layer {mode}")
    assert_close(_run_decode(b, dev, mode), want, torch.bfloat16, f"qwen3 {mode}")


# ---- decode: the prefix-shared batch (256 seqs, ctx U{512..4096}, 32 q / 8 kv) ------------

LLAMA_MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", 512), ("mfma", "balanced"), ("mfma", "auto"),
               ("valu", 0)]


@pytest.mark.parametrize("mode", LLAMA_MODES + [("shared_prefix", 0)], ids=_ids)
def test_llama_prefix_every_row(mode):
    b, dev, want = _one("llama", lambda: _decode_entry(W.llama_prefix().batches[0], store=False))
    say(f"llama prefix {mode}")
    if mode[0] == "shared_prefix":
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode_shared_prefix(
            out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
            torch.arange(0, b.num_seqs + 1, 8, dtype=torch.int32, device="cuda"),
            torch.full((b.num_seqs // 8,), 32 * b.block_size, dtype=torch.int32, device="cuda"),
            b.scale, b.max_ctx, 8, 32 * b.block_size)
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
    else:
        got = _run_decode(b, dev, mode)
    assert_close(got, want, torch.bfloat16, f"llama {mode}")


# ---- decode: long contexts (32 seqs, ctx log-uniform 1K..32K, 32 q / 8 kv) ----------------

LONG_MODES = [("mfma", 512), ("mfma", 1024), ("mfma", 0), ("mfma", "planned"), ("mfma", "balanced"),
              ("mfma", "auto"), ("valu", 512), ("valu", "auto")]


@pytest.mark.parametrize("mode", LONG_MODES, ids=_ids)
def test_long_splitk_every_row(mode):
    b, dev, want = _one("long", lambda: _decode_entry(W.long_splitk().batches[0], store=False))
    say(f"long contexts {mode}")
    assert_close(_run_decode(b, dev, mode), want, torch.bfloat16, f"long {mode}")


# ---- the mixed batch: store of 4224 rows, decode of 128 seqs, 8 prefill chunks ------------

def _mixed_entry():
    wl = W.mixed()
    pre, dec = wl.prefill, wl.batches[0]
    dev = to_device(pre)
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
    ddev = to_device(dec)
    ddev["k_cache"], ddev["v_cache"] = dev["k_cache"], dev["v_cache"]
    kc, vc = oracle_caches(pre)
    torch.cuda.synchronize()
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert W.host_bits(dev["v_cache"]).tobytes() == vc.tobytes()
    say(f"  oracle: decode of 128 seqs and 8 x 512 prefill rows on {full_size.workers()} host workers")
    want_dec = full_size.decode(W.host_bits(dec.q), kc, vc, dec.pool.block_tables, dec.pool.context_lens,
                                dec.scale, dec.block_size)
    want_pre = full_size.prefill(W.host_bits(pre.q), kc, vc, pre.pool.block_tables, pre.cu_seqlens_q,
                                 pre.pool.context_lens, pre.scale, pre.block_size, causal=True)
    return pre, dec, dev, ddev, want_pre, want_dec


MIXED_DECODE_MODES = [("mfma", 0), ("mfma", "planned"), ("mfma", "balanced"), ("mfma", 512), ("mfma", "auto"),
                      ("valu", 0)]


@pytest.mark.parametrize("mode", MIXED_DECODE_MODES, ids=_ids)
def test_mixed_decode_every_row(mode):
    pre, dec, dev, ddev, want_pre, want_dec = _one("mixed", _mixed_entry)
    say(f"mixed decode {mode}")
    assert_close(_run_decode(dec, ddev, mode), want_dec, torch.bfloat16, f"mixed decode {mode}")


def test_mixed_prefill_every_row():
    pre, dec, dev, ddev, want_pre, want_dec = _one("mixed", _mixed_entry)
    say("mixed prefill: 8 chunks x 512 causal rows")
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_prefill_chunk(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                      dev["cu_seqlens_q"], dev["context_lens"], pre.scale, 512, pre.max_ctx,
                                      causal=True)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want_pre, torch.bfloat16, "mixed prefill")


# ---- chunked prefill over E4M3 caches (the mixed chunks' shapes) --------------------------

def _mixed_fp8_entry():
    b = W.mixed_prefill_fp8()
    d = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "k_new",
                                                "v_new", "slot_mapping")}
    d["block_tables"] = torch.as_tensor(b.pool.block_tables, device="cuda")
    d["context_lens"] = torch.as_tensor(b.pool.context_lens, device="cuda")
    d["cu_seqlens_q"] = torch.as_tensor(b.cu_seqlens_q, device="cuda")
    pkv.kv_cache_store_fp8(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"], d["k_scale"],
                           d["v_scale"])
    ks, vs = W.host_bits(b.k_scale), W.host_bits(b.v_scale)
    kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                    W.host_bits(b.v_cache), W.host_bits(b.slot_mapping), ks, vs, b.block_size)
    torch.cuda.synchronize()
    assert d["k_cache"].cpu().numpy().tobytes() == kc.tobytes()
    assert d["v_cache"].cpu().numpy().tobytes() == vc.tobytes()
    say(f"  oracle: 8 x 512 prefill rows over E4M3 caches on {full_size.workers()} host workers")
    want = full_size.prefill(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.cu_seqlens_q,
                             b.pool.context_lens, b.scale, b.block_size, causal=True, k_scale=ks, v_scale=vs)
    return b, d, want


def test_mixed_prefill_fp8_every_row():
    b, d, want = _one("mixed_fp8", _mixed_fp8_entry)
    out = torch.full_like(d["q"], float("nan"))
    pkv.paged_attention_prefill_chunk_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                          d["block_tables"], d["cu_seqlens_q"], d["context_lens"], b.scale, 512,
                                          b.max_ctx, causal=True)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "mixed prefill E4M3")


# ---- verification of drafted tokens: 128 seqs x 4 causal rows ------------------------------

def test_spec_verify_every_row():
    b = W.spec_verify().prefill
    dev = to_device(b)
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_prefill_chunk(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                      dev["cu_seqlens_q"], dev["context_lens"], b.scale, 4, b.max_ctx,
                                      causal=True)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(b)
    say(f"spec_verify: oracle over {b.num_seqs} x 4 rows on {full_size.workers()} host workers")
    want = full_size.prefill(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.cu_seqlens_q,
                             b.pool.context_lens, b.scale, b.block_size, causal=True)
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "spec_verify")


# ---- the Qwen3-shaped layer over E4M3 caches ------------------------------------------------

@pytest.mark.parametrize("part", [0, "planned", 256, "auto"])
def test_qwen3_fp8_layer_every_row(part):
    def make():
        b = W.qwen3_decode_fp8(layers=1).batches[0]
        d = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "k_new",
                                                    "v_new", "slot_mapping")}
        d["block_tables"] = torch.as_tensor(b.pool.block_tables, device="cuda")
        d["context_lens"] = torch.as_tensor(b.pool.context_lens, device="cuda")
        pkv.kv_cache_store_fp8(d["k_new"], d["v_new"], d["k_cache"], d["v_cache"], d["slot_mapping"],
                               d["k_scale"], d["v_scale"])
        ks, vs = W.host_bits(b.k_scale), W.host_bits(b.v_scale)
        kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                        W.host_bits(b.v_cache), W.host_bits(b.slot_mapping), ks, vs,
                                        b.block_size)
        want = full_size.decode(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.pool.context_lens, b.scale,
                                b.block_size, k_scale=ks, v_scale=vs)
        torch.cuda.synchronize()
        return b, d, want
    b, d, want = _one("qwen3_fp8", make)
    ws = None
    if part == "planned":
        ws = pkv.new_decode_plan(b.num_seqs, "cuda")
        pkv.decode_plan(ws, d["block_tables"], d["context_lens"], b.max_ctx, b.block_size)
    out = torch.full_like(d["q"], float("nan"))
    pkv.paged_attention_decode_fp8(out, d["q"], d["k_cache"], d["v_cache"], d["k_scale"], d["v_scale"],
                                   d["block_tables"], d["context_lens"], b.scale, b.max_ctx,
                                   partition_size=part, workspace=ws)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"qwen3 E4M3 p={part}")


def teardown_module(module):
    _CACHE.clear()
    full_size.shutdown()
