"""Seeded random shapes through every launch mode of the C ABI, against the
float64 oracle: decode over bf16 / fp32 / E4M3 caches and chunked prefill.

The shapes are drawn once, at import, from a fixed seed: GQA groups 1..16
(including groups that are not powers of two), head_dim 64 and 128, block
sizes 16..256, batches of one to a hundred sequences, and contexts from empty
to a few thousand tokens, including lengths on and next to tile and block
boundaries. Every mode the library offers for a shape is run (one pass per
item, split-K at a drawn partition size, the automatic choice, the
work-balanced kernel, a plan, the allocation-free entry point); a mode the
library reports as unsupported for that shape is skipped, and every shape
must run in at least its default mode. Outputs start as NaN, so a row that no
workgroup writes fails.
"""

import os

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from paged_attention_kv_store_amd.binding import PKV_EUNSUPPORTED, PKV_EWORKSPACE, PkvError
from tests.gpu_helpers import assert_close, oracle_caches, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu

# The draws are fixed; PKV_FUZZ_SEED and PKV_FUZZ_MULT (default 1) draw
# another set, PKV_FUZZ_MULT times as many cases of every kind, for longer runs.
_rng = np.random.default_rng(int(os.environ.get("PKV_FUZZ_SEED", "20261203")))
_MULT = max(1, int(os.environ.get("PKV_FUZZ_MULT", "1")))
_EDGE_CTX = [1, 15, 16, 17, 63, 64, 65, 255, 256, 257, 700, 1300, 2100]


def _draw_decode(i):
    dtype = torch.float32 if _rng.random() < 0.25 else torch.bfloat16
    hkv = int(_rng.choice([1, 2, 3, 4, 8]))
    g = int(_rng.choice([1, 2, 3, 4, 5, 8, 16]))
    d = 64 if _rng.random() < 0.3 else 128
    bs = int(_rng.choice([16, 32, 64, 128, 256]))
    s = int(_rng.integers(1, 101))
    max_ctx = int(_rng.choice(_EDGE_CTX))
    min_ctx = max_ctx if _rng.random() < 0.2 else 0   # sometimes every length equal
    split = 16 * int(_rng.choice([1, 2, 5, 16, 64]))
    return (i, dtype, s, g * hkv, hkv, d, bs, max_ctx, min_ctx, split)


DECODE = [_draw_decode(i) for i in range(24 * _MULT)]


def _draw_fp8(i):
    hkv = int(_rng.choice([1, 2, 4, 8]))
    g = int(_rng.choice([1, 2, 4, 8]))
    d = 64 if _rng.random() < 0.3 else 128
    bs = int(_rng.choice([16, 32, 64]))
    s = int(_rng.integers(1, 81))
    max_ctx = int(_rng.choice(_EDGE_CTX))
    split = 16 * int(_rng.choice([1, 4, 16, 32]))
    return (i, s, g * hkv, hkv, d, bs, max_ctx, split)


FP8_DECODE = [_draw_fp8(i) for i in range(10 * _MULT)]


def _draw_prefill(i):
    hkv = int(_rng.choice([1, 2, 4, 8]))
    g = int(_rng.choice([1, 2, 4, 8, 16]))
    bs = int(_rng.choice([16, 32, 64, 128, 256]))
    chunks = int(_rng.integers(1, 9))
    max_rows = int(_rng.choice([1, 2, 4, 7, 33, 130, 300]))
    max_prior = int(_rng.choice([0, 1, 15, 64, 200, 900]))
    causal = bool(_rng.random() < 0.75)
    return (i, g * hkv, hkv, bs, chunks, max_rows, max_prior, causal)


PREFILL = [_draw_prefill(i) for i in range(16 * _MULT)]


def oracle_prefill(b, causal):
    kc, vc = oracle_caches(b)
    return oracle.paged_attention_prefill_chunk(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.cu_seqlens_q,
                                                b.pool.context_lens, b.scale, b.block_size, causal=causal)


def _ids(c):
    return "-".join(str(x)[6:] if isinstance(x, torch.dtype) else str(x) for x in c)


def _run(what, fn):
    """fn's float64 output, or None when the library reports the shape
    unsupported in this mode (or, for the allocation-free entry point, a
    call beyond its fixed scratch)."""
    try:
        return fn()
    except PkvError as e:
        if e.status == PKV_EUNSUPPORTED or (what.startswith("static") and e.status == PKV_EWORKSPACE):
            say(f"  {what}: not for this shape ({e})")
            return None
        raise


@pytest.mark.parametrize("case", DECODE, ids=_ids)
def test_decode_every_mode(case):
    i, dtype, s, hq, hkv, d, bs, max_ctx, min_ctx, split = case
    b = W.random_decode_batch(9000 + i, s, hq, hkv, d, dtype, max_ctx=max_ctx, min_ctx=min_ctx, block_size=bs,
                              store=False)
    say(f"fuzz decode {case} ctx={b.pool.context_lens.tolist()[:12]}...")
    want = oracle_decode(b, store=False)
    dv = to_device(b)

    def decode(**kw):
        def run():
            out = torch.full_like(dv["q"], float("nan"))
            pkv.paged_attention_decode(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                       dv["context_lens"], b.scale, b.max_ctx, **kw)
            torch.cuda.synchronize()
            return out.float().cpu().double().numpy()
        return run

    def planned():
        plan = pkv.new_decode_plan(s, "cuda")
        pkv.decode_plan(plan, dv["block_tables"], dv["context_lens"], b.max_ctx, bs)
        return decode(partition_size="planned", workspace=plan)()

    def static():
        out = torch.full_like(dv["q"], float("nan"))
        pkv.paged_attention_decode_static(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                          dv["context_lens"], b.scale, b.max_ctx, partition_size=split)
        torch.cuda.synchronize()
        return out.float().cpu().double().numpy()

    modes = [("default", decode()), ("valu", decode(algo="valu")), ("mfma", decode(algo="mfma")),
             ("auto", decode(partition_size="auto")), (f"split {split}", decode(partition_size=split)),
             ("balanced", decode(partition_size="balanced")), ("planned", planned),
             (f"static {split}", static)]
    ran = []
    for name, fn in modes:
        got = _run(name, fn)
        if got is None:
            assert name != "default", "the default mode must support every shape drawn here"
            continue
        assert_close(got, want, dtype, name)
        ran.append(name)
    say(f"  modes run: {ran}")


@pytest.mark.parametrize("case", FP8_DECODE, ids=_ids)
def test_fp8_decode_every_mode(case):
    i, s, hq, hkv, d, bs, max_ctx, split = case
    b = W.random_decode_batch_fp8(9500 + i, s, hq, hkv, d, max_ctx=max_ctx, min_ctx=0, block_size=bs,
                                  store=False)
    say(f"fuzz fp8 decode {case} ctx={b.pool.context_lens.tolist()[:12]}...")
    kc, vc = W.host_bits(b.k_cache), W.host_bits(b.v_cache)
    want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), kc, vc, W.host_bits(b.k_scale),
                                          W.host_bits(b.v_scale), b.pool.block_tables, b.pool.context_lens,
                                          b.scale, b.block_size)
    dv = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale")}
    bt = torch.as_tensor(b.pool.block_tables, device="cuda")
    cl = torch.as_tensor(b.pool.context_lens, device="cuda")

    def decode(**kw):
        def run():
            out = torch.full_like(dv["q"], float("nan"))
            pkv.paged_attention_decode_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["k_scale"],
                                           dv["v_scale"], bt, cl, b.scale, b.max_ctx, **kw)
            torch.cuda.synchronize()
            return out.float().cpu().double().numpy()
        return run

    def planned():
        plan = pkv.new_decode_plan(s, "cuda")
        pkv.decode_plan(plan, bt, cl, b.max_ctx, bs)
        return decode(partition_size="planned", workspace=plan)()

    ran = []
    for name, fn in [("default", decode()), ("auto", decode(partition_size="auto")),
                     (f"split {split}", decode(partition_size=split)), ("planned", planned)]:
        got = _run(name, fn)
        if got is None:
            assert name != "default", "the default mode must support every shape drawn here"
            continue
        assert_close(got, want, torch.bfloat16, name)
        ran.append(name)
    say(f"  modes run: {ran}")


@pytest.mark.parametrize("case", PREFILL, ids=_ids)
def test_prefill_bf16_and_fp8(case):
    i, hq, hkv, bs, chunks, max_rows, max_prior, causal = case
    b = W.random_prefill_batch(9800 + i, chunks, hq, hkv, 128, torch.bfloat16, max_rows=max_rows,
                               max_prior=max_prior, block_size=bs)
    say(f"fuzz prefill {case} rows={np.diff(b.cu_seqlens_q).tolist()} ctx={b.pool.context_lens.tolist()}")
    dv = to_device(b)
    pkv.kv_cache_store(dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], dv["slot_mapping"])
    mq = int(np.diff(b.cu_seqlens_q).max())
    out = torch.full_like(dv["q"], float("nan"))
    pkv.paged_attention_prefill_chunk(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                      dv["cu_seqlens_q"], dv["context_lens"], b.scale, mq, b.max_ctx,
                                      causal=causal)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), oracle_prefill(b, causal=causal), torch.bfloat16,
                 f"bf16 causal={causal}")

    b8 = W.random_prefill_batch_fp8(9900 + i, chunks, hq, hkv, 128, max_rows=max_rows, max_prior=max_prior,
                                    block_size=bs)
    d8 = {k: getattr(b8, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale", "k_new",
                                                 "v_new", "slot_mapping")}
    bt8 = torch.as_tensor(b8.pool.block_tables, device="cuda")
    cu8 = torch.as_tensor(b8.cu_seqlens_q, device="cuda")
    cl8 = torch.as_tensor(b8.pool.context_lens, device="cuda")
    pkv.kv_cache_store_fp8(d8["k_new"], d8["v_new"], d8["k_cache"], d8["v_cache"], d8["slot_mapping"],
                           d8["k_scale"], d8["v_scale"])
    kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b8.k_new), W.host_bits(b8.v_new), W.host_bits(b8.k_cache),
                                    W.host_bits(b8.v_cache), W.host_bits(b8.slot_mapping),
                                    W.host_bits(b8.k_scale), W.host_bits(b8.v_scale), b8.block_size)
    want8 = FP8.paged_attention_prefill_chunk_fp8(W.host_bits(b8.q), kc, vc, W.host_bits(b8.k_scale),
                                                  W.host_bits(b8.v_scale), b8.pool.block_tables,
                                                  b8.cu_seqlens_q, b8.pool.context_lens, b8.scale,
                                                  b8.block_size, causal=causal)
    out8 = torch.full_like(d8["q"], float("nan"))
    mq8 = int(np.diff(b8.cu_seqlens_q).max())
    pkv.paged_attention_prefill_chunk_fp8(out8, d8["q"], d8["k_cache"], d8["v_cache"], d8["k_scale"],
                                          d8["v_scale"], bt8, cu8, cl8, b8.scale, mq8, b8.max_ctx, causal=causal)
    torch.cuda.synchronize()
    assert_close(out8.float().cpu().double().numpy(), want8, torch.bfloat16, f"fp8 causal={causal}")


def _draw_fused(i):
    dtype = [torch.float32, torch.bfloat16, "e4m3"][int(_rng.integers(0, 3))]
    hkv = int(_rng.choice([1, 2, 4, 8]))
    g = int(_rng.choice([1, 2, 3, 4, 8, 16]))
    if dtype == "e4m3":
        g = int(_rng.choice([1, 2, 4, 8]))
    d = 64 if _rng.random() < 0.3 else 128
    bs = int(_rng.choice([16, 32, 64, 128]))
    s = int(_rng.integers(1, 90))
    max_ctx = int(_rng.choice(_EDGE_CTX))
    split = 16 * int(_rng.choice([1, 3, 8, 32]))
    return (i, dtype, s, g * hkv, hkv, d, bs, max_ctx, split)


FUSED = [_draw_fused(i) for i in range(14 * _MULT)]


@pytest.mark.parametrize("case", FUSED, ids=_ids)
def test_fused_store_and_decode_every_mode(case):
    """One new row per sequence stored at position ctx-1 and used from
    registers in the same launch: caches bit-exact, outputs within tolerance."""
    i, dtype, s, hq, hkv, d, bs, max_ctx, split = case
    e4m3 = dtype == "e4m3"
    if e4m3:
        b = W.random_decode_batch_fp8(9600 + i, s, hq, hkv, d, max_ctx=max_ctx, min_ctx=1, block_size=bs)
        kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                        W.host_bits(b.v_cache), W.host_bits(b.slot_mapping),
                                        W.host_bits(b.k_scale), W.host_bits(b.v_scale), bs)
        want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), kc, vc, W.host_bits(b.k_scale),
                                              W.host_bits(b.v_scale), b.pool.block_tables, b.pool.context_lens,
                                              b.scale, bs)
        tol_dtype = torch.bfloat16
    else:
        b = W.random_decode_batch(9700 + i, s, hq, hkv, d, dtype, max_ctx=max_ctx, min_ctx=1, block_size=bs)
        kc, vc = oracle_caches(b)
        want = oracle_decode(b, caches=(kc, vc))
        tol_dtype = dtype
    say(f"fuzz fused {case} ctx={b.pool.context_lens.tolist()[:12]}...")

    def fused(partition):
        def run():
            dv = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_new", "v_new",
                                                        "slot_mapping")}
            bt = torch.as_tensor(b.pool.block_tables, device="cuda")
            cl = torch.as_tensor(b.pool.context_lens, device="cuda")
            ws = None
            if partition == "planned":
                ws = pkv.new_decode_plan(s, "cuda")
                pkv.decode_plan(ws, bt, cl, b.max_ctx, bs)
            out = torch.full_like(dv["q"], float("nan"))
            if e4m3:
                pkv.paged_attention_decode_store_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"],
                                                     b.k_scale.to("cuda"), b.v_scale.to("cuda"), bt, cl,
                                                     dv["k_new"], dv["v_new"], dv["slot_mapping"], b.scale,
                                                     b.max_ctx, partition_size=partition, workspace=ws)
            else:
                pkv.paged_attention_decode_store(out, dv["q"], dv["k_cache"], dv["v_cache"], bt, cl, dv["k_new"],
                                                 dv["v_new"], dv["slot_mapping"], b.scale, b.max_ctx,
                                                 partition_size=partition, workspace=ws)
            torch.cuda.synchronize()
            assert W.host_bits(dv["k_cache"]).tobytes() == kc.tobytes(), "K cache differs from the oracle's store"
            assert W.host_bits(dv["v_cache"]).tobytes() == vc.tobytes(), "V cache differs from the oracle's store"
            return out.float().cpu().double().numpy()
        return run

    ran = []
    for name, part in [("default", 0), (f"split {split}", split), ("planned", "planned"),
                       ("balanced", "balanced")]:
        got = _run(name, fused(part))
        if got is None:
            assert name != "default", "the default mode must support every shape drawn here"
            continue
        assert_close(got, want, tol_dtype, name)
        ran.append(name)
    say(f"  modes run: {ran}")


def _draw_store(i):
    dtype = [torch.float32, torch.bfloat16, "e4m3"][int(_rng.integers(0, 3))]
    hkv = int(_rng.choice([1, 2, 3, 8]))
    d = int(_rng.choice([32, 40, 64, 128, 256]))
    bs = int(_rng.choice([1, 8, 16, 32, 256]))
    nb = int(_rng.integers(1, 200))
    t = int(_rng.integers(0, min(nb * bs, 3000) + 1))
    pad = float(_rng.choice([0.0, 0.1, 0.5]))
    return (i, dtype, hkv, d, bs, nb, t, pad)


STORE = [_draw_store(i) for i in range(16 * _MULT)]


@pytest.mark.parametrize("case", STORE, ids=_ids)
def test_store_random_slots(case):
    """Distinct random slots (a share of them -1, skipped) across the pool:
    the caches match the oracle's store bit for bit, padding included."""
    i, dtype, hkv, d, bs, nb, t, pad = case
    rng = np.random.default_rng(9400 + i)
    slots = rng.permutation(nb * bs)[:t].astype(np.int32)
    slots[rng.random(t) < pad] = -1
    gen = torch.Generator().manual_seed(9400 + i)
    src = torch.float32 if dtype == torch.float32 else torch.bfloat16
    k = torch.randn(t, hkv, d, generator=gen).to(src)
    v = torch.randn(t, hkv, d, generator=gen).to(src)
    say(f"fuzz store {case}")
    if dtype == "e4m3":
        kc0 = torch.randint(0, 256, (nb, bs, hkv, d), generator=gen, dtype=torch.uint8)
        vc0 = torch.randint(0, 256, (nb, bs, hkv, d), generator=gen, dtype=torch.uint8)
        ks = (torch.rand(hkv, generator=gen) * 0.1 + 0.01).float()
        vs = (torch.rand(hkv, generator=gen) * 0.1 + 0.01).float()
        kc, vc = kc0.cuda(), vc0.cuda()
        pkv.kv_cache_store_fp8(k.cuda(), v.cuda(), kc, vc, torch.as_tensor(slots).cuda(), ks.cuda(), vs.cuda())
        wk, wv = FP8.kv_cache_store_fp8(W.host_bits(k), W.host_bits(v), kc0.numpy(), vc0.numpy(), slots,
                                        ks.numpy(), vs.numpy(), bs)
    else:
        kc0 = torch.randn(nb, bs, hkv, d, generator=gen).to(dtype)
        vc0 = torch.randn(nb, bs, hkv, d, generator=gen).to(dtype)
        kc, vc = kc0.cuda(), vc0.cuda()
        pkv.kv_cache_store(k.cuda(), v.cuda(), kc, vc, torch.as_tensor(slots).cuda())
        wk, wv = oracle.kv_cache_store(W.host_bits(k), W.host_bits(v), W.host_bits(kc0), W.host_bits(vc0), slots, bs)
    torch.cuda.synchronize()
    assert W.host_bits(kc.cpu()).tobytes() == np.asarray(wk).tobytes()
    assert W.host_bits(vc.cpu()).tobytes() == np.asarray(wv).tobytes()


def _draw_shared(i):
    hkv = int(_rng.choice([1, 2, 4, 8]))
    g = int(_rng.choice([1, 2, 4, 8, 16]))
    bs = int(_rng.choice([16, 32, 64]))
    groups = int(_rng.integers(1, 9))
    size = int(_rng.integers(1, 20))
    shared = int(_rng.integers(0, 12))
    max_ctx = shared * bs + int(_rng.choice([0, 1, 17, 300, 900]))
    return (i, g * hkv, hkv, bs, groups, size, shared, max_ctx)


SHARED = [_draw_shared(i) for i in range(10 * _MULT)]


@pytest.mark.parametrize("case", SHARED, ids=_ids)
def test_shared_prefix_random_groups(case):
    """Groups of consecutive sequences sharing their first blocks; each group's
    declared prefix is a random whole number of those blocks (possibly 0)."""
    i, hq, hkv, bs, groups, size, shared, max_ctx = case
    n = groups * size
    b = W.random_decode_batch(9200 + i, n, hq, hkv, 128, torch.bfloat16, max_ctx=max(max_ctx, 1), min_ctx=0,
                              block_size=bs, store=False, share_group=size, shared_blocks=shared)
    rng = np.random.default_rng(9200 + i)
    starts = np.arange(0, n + 1, size).astype(np.int32)
    ctx = b.pool.context_lens
    prefixes = []
    for j in range(groups):
        most = min(shared * bs, int(ctx[starts[j]:starts[j + 1]].min()))
        prefixes.append(bs * int(rng.integers(0, most // bs + 1)))
    say(f"fuzz shared {case} prefixes={prefixes} ctx={ctx.tolist()[:12]}...")
    dv = to_device(b)
    out = torch.full_like(dv["q"], float("nan"))
    pkv.paged_attention_decode_shared_prefix(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                             dv["context_lens"], torch.as_tensor(starts, device="cuda"),
                                             torch.as_tensor(np.asarray(prefixes, np.int32), device="cuda"),
                                             b.scale, b.max_ctx, size, max(prefixes))
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), oracle_decode(b, store=False), torch.bfloat16, "shared")


# Scales far from 1/sqrt(D) and block-table padding values, drawn from a
# stream of their own so that the draws above stay as they are. bf16 only:
# its 2e-2 bound holds at any scale (the fp32 bound assumes logits of order one).
_rng_sp = np.random.default_rng(int(os.environ.get("PKV_FUZZ_SEED", "20261203")) + 1)


def _draw_scale_pad(i):
    hkv = int(_rng_sp.choice([1, 2, 4, 8]))
    g = int(_rng_sp.choice([1, 2, 4, 8]))
    d = 64 if _rng_sp.random() < 0.3 else 128
    bs = int(_rng_sp.choice([16, 32, 64, 256]))
    s = int(_rng_sp.integers(1, 70))
    max_ctx = int(_rng_sp.choice(_EDGE_CTX))
    kind = int(_rng_sp.integers(0, 4))
    scale = [float(_rng_sp.uniform(-3.0, 3.0)), float(_rng_sp.choice([0.0, 20.0, -20.0, 100.0])),
             float(_rng_sp.uniform(0.02, 0.2)), float(-_rng_sp.uniform(0.02, 0.2))][kind]
    pad = int(_rng_sp.choice([-1, 2 ** 31 - 1, -(2 ** 31), 0]))
    split = 16 * int(_rng_sp.choice([1, 4, 16, 32]))
    return (i, s, g * hkv, hkv, d, bs, max_ctx, round(scale, 4), pad, split)


SCALE_PAD = [_draw_scale_pad(i) for i in range(10 * _MULT)]


@pytest.mark.parametrize("case", SCALE_PAD, ids=_ids)
def test_decode_scales_and_table_padding(case):
    i, s, hq, hkv, d, bs, max_ctx, scale, pad, split = case
    b = W.random_decode_batch(9700 + i, s, hq, hkv, d, torch.bfloat16, max_ctx=max_ctx, min_ctx=0, block_size=bs,
                              store=False, scale=scale)
    bt = b.pool.block_tables
    for q, c in enumerate(b.pool.context_lens.tolist()):
        bt[q, -(-c // bs):] = pad
    say(f"fuzz scale/padding {case}")
    want = oracle_decode(b, store=False)
    dv = to_device(b)

    def decode(**kw):
        def run():
            out = torch.full_like(dv["q"], float("nan"))
            pkv.paged_attention_decode(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                       dv["context_lens"], b.scale, b.max_ctx, **kw)
            torch.cuda.synchronize()
            return out.float().cpu().double().numpy()
        return run

    def planned():
        plan = pkv.new_decode_plan(s, "cuda")
        pkv.decode_plan(plan, dv["block_tables"], dv["context_lens"], b.max_ctx, bs)
        return decode(partition_size="planned", workspace=plan)()

    ran = []
    for name, fn in [("default", decode()), ("valu", decode(algo="valu")), ("auto", decode(partition_size="auto")),
                     (f"split {split}", decode(partition_size=split)),
                     ("balanced", decode(partition_size="balanced")), ("planned", planned)]:
        got = _run(name, fn)
        if got is None:
            assert name != "default", "the default mode must support every shape drawn here"
            continue
        assert_close(got, want, torch.bfloat16, name)
        ran.append(name)
    say(f"  modes run: {ran}")
