"""GPU tests of the planned decode: the plan's contents (an integer result,
compared exactly with the order the host computes), and the decode that
takes its items in the plan's order, against the float64 oracle and, bit for
bit, against the single-pass decode in the kernel's own order (the same
per-item arithmetic, only the work order differs), through the C ABI."""

import numpy as np
import pytest
import torch

from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_caches, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu

TILE = 16
BUCKETS = 2048


def expected_plan(block_tables, context_lens, max_ctx, block_size):
    """Sequences by 16-token tiles (lengths clamped to [0, max_ctx], tiles
    capped at BUCKETS - 1), most first, ties by index; each entry holds the
    sequence, its raw length, the table entries of 16-token tiles 0..3 (the
    row's last entry past its end) and two zeros."""
    ctx = np.asarray(context_lens, np.int64)
    tiles = np.minimum((np.clip(ctx, 0, max_ctx) + TILE - 1) // TILE, BUCKETS - 1)
    order = np.argsort(-tiles, kind="stable")
    mb = block_tables.shape[1]
    cols = [min((TILE * w) // block_size, mb - 1) for w in range(4)]
    plan = np.zeros((len(ctx), 8), np.int32)
    plan[:, 0] = order
    plan[:, 1] = np.asarray(context_lens, np.int32)[order]
    plan[:, 2:6] = np.asarray(block_tables, np.int32)[order][:, cols]
    return plan


def make_plan(dev, max_ctx, block_size):
    plan = pkv.new_decode_plan(dev["block_tables"].shape[0], "cuda")
    pkv.decode_plan(plan, dev["block_tables"], dev["context_lens"], max_ctx, block_size)
    return plan


def plan_entries(plan, num_seqs):
    return plan[: num_seqs * 32].view(torch.int32).cpu().numpy().reshape(num_seqs, 8)


@pytest.mark.parametrize("num_seqs,max_ctx,min_ctx,bs", [
    (1, 40, 40, 16),
    (60, 1024, 64, 16),
    (300, 90, 0, 16),          # past one chunk of the plan kernel, many equal sizes, empty ones
    (700, 3000, 0, 32),
    (2000, 200, 0, 64),
])
def test_plan_is_the_stable_size_order(num_seqs, max_ctx, min_ctx, bs):
    b = W.random_decode_batch(900 + num_seqs, num_seqs, 8, 8, 64, torch.bfloat16, max_ctx=max_ctx,
                              min_ctx=min_ctx, block_size=bs, store=False)
    say(f"plan S={num_seqs} ctx<={max_ctx} bs={bs}")
    dev = to_device(b)
    plan = make_plan(dev, b.max_ctx, bs)
    torch.cuda.synchronize()
    want = expected_plan(b.pool.block_tables, b.pool.context_lens, b.max_ctx, bs)
    np.testing.assert_array_equal(plan_entries(plan, num_seqs), want)


def test_plan_caps_tiles_and_clamps_lengths():
    """Lengths past 2047 tiles share the top size; a length above the host
    bound counts as the bound (the entry keeps the raw value)."""
    s, mb = 40, 2200
    rng = np.random.default_rng(7)
    ctx = rng.integers(0, mb * 16, size=s).astype(np.int32)
    ctx[:6] = [2047 * 16, 2047 * 16 + 5, 2100 * 16, mb * 16, 16, 0]
    bt = rng.integers(0, 5000, size=(s, mb)).astype(np.int32)
    max_ctx = 2100 * 16
    dev = {"block_tables": torch.as_tensor(bt, device="cuda"),
           "context_lens": torch.as_tensor(ctx, device="cuda")}
    plan = make_plan(dev, max_ctx, 16)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(plan_entries(plan, s), expected_plan(bt, ctx, max_ctx, 16))


CASES = [
    # (num_seqs, hq, hkv, d, max_ctx, min_ctx, block_size): items = num_seqs * hkv against
    # 256 compute units: one item per unit, one or two, more than two
    (20, 16, 8, 128, 500, 0, 16),
    (60, 16, 8, 128, 1024, 64, 16),
    (45, 32, 8, 128, 700, 1, 32),
    (150, 32, 8, 128, 300, 0, 16),
    (90, 12, 4, 64, 400, 0, 16),
    (37, 8, 1, 128, 600, 0, 64),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{c[1]}x{c[2]}-d{c[3]}-bs{c[6]}")
def test_planned_decode(case):
    s, hq, hkv, d, max_ctx, min_ctx, bs = case
    b = W.random_decode_batch(1300 + s + d + bs, s, hq, hkv, d, torch.bfloat16, max_ctx=max_ctx,
                              min_ctx=min_ctx, block_size=bs, store=False)
    say(f"planned decode {case}")
    dev = to_device(b)
    plan = make_plan(dev, b.max_ctx, bs)
    outs = {}
    for part, ws in ((0, None), ("planned", plan)):
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                   workspace=ws, algo="mfma")
        outs[part] = out
    torch.cuda.synchronize()
    assert torch.equal(outs["planned"].view(torch.int16), outs[0].view(torch.int16))
    assert_close(outs["planned"].float().cpu().double().numpy(), oracle_decode(b, store=False),
                 torch.bfloat16, "planned")


@pytest.mark.parametrize("case", CASES[:4], ids=lambda c: f"s{c[0]}-{c[1]}x{c[2]}-d{c[3]}-bs{c[6]}")
def test_planned_decode_store(case):
    s, hq, hkv, d, max_ctx, min_ctx, bs = case
    b = W.random_decode_batch(1700 + s + d + bs, s, hq, hkv, d, torch.bfloat16, max_ctx=max_ctx,
                              min_ctx=min_ctx, block_size=bs)
    b.slot_mapping[2] = -1           # padding: nothing stored, position ctx-1 read from the cache
    say(f"planned decode+store {case}")
    runs = {}
    for part in (0, "planned"):
        dev = to_device(b)
        plan = make_plan(dev, b.max_ctx, bs) if part == "planned" else None
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"],
                                         dev["block_tables"], dev["context_lens"], dev["k_new"],
                                         dev["v_new"], dev["slot_mapping"], b.scale, b.max_ctx,
                                         partition_size=part, workspace=plan)
        torch.cuda.synchronize()
        runs[part] = (out, dev)
    out, dev = runs["planned"]
    kc, vc = oracle_caches(b)
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert W.host_bits(dev["v_cache"]).tobytes() == vc.tobytes()
    assert torch.equal(out.view(torch.int16), runs[0][0].view(torch.int16))
    got = out.float().cpu().double().numpy()
    live = [i for i in range(s) if i != 2]
    assert_close(got[live], oracle_decode(b, caches=(kc, vc), seqs=live), torch.bfloat16, "planned+store")


def test_planned_decode_store_fp8():
    s, hq, hkv, d = 70, 32, 8, 128
    b = W.random_decode_batch_fp8(2100, s, hq, hkv, d, max_ctx=900, min_ctx=0)
    say("planned decode+store over E4M3 caches")
    runs = {}
    for part in (0, "planned"):
        dv = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale",
                                                     "k_new", "v_new", "slot_mapping")}
        dv["block_tables"] = torch.as_tensor(b.pool.block_tables, device="cuda")
        dv["context_lens"] = torch.as_tensor(b.pool.context_lens, device="cuda")
        plan = make_plan(dv, b.max_ctx, b.block_size) if part == "planned" else None
        out = torch.full_like(dv["q"], float("nan"))
        pkv.paged_attention_decode_store_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["k_scale"],
                                             dv["v_scale"], dv["block_tables"], dv["context_lens"],
                                             dv["k_new"], dv["v_new"], dv["slot_mapping"], b.scale,
                                             b.max_ctx, partition_size=part, workspace=plan)
        torch.cuda.synchronize()
        runs[part] = (out, dv)
    out, dv = runs["planned"]
    kc, vc = FP8.kv_cache_store_fp8(W.host_bits(b.k_new), W.host_bits(b.v_new), W.host_bits(b.k_cache),
                                    W.host_bits(b.v_cache), W.host_bits(b.slot_mapping),
                                    W.host_bits(b.k_scale), W.host_bits(b.v_scale), b.block_size)
    np.testing.assert_array_equal(dv["k_cache"].cpu().numpy(), kc)
    np.testing.assert_array_equal(dv["v_cache"].cpu().numpy(), vc)
    assert torch.equal(out.view(torch.int16), runs[0][0].view(torch.int16))
    want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), kc, vc, W.host_bits(b.k_scale),
                                          W.host_bits(b.v_scale), b.pool.block_tables, b.pool.context_lens,
                                          b.scale, b.block_size)
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "planned fp8")


def test_planned_decode_past_the_in_kernel_ranking_limit():
    """5000 sequences: more than the 4096 the kernel ranks in LDS itself,
    which the plan does not need; every row written and right."""
    s = 5000
    b = W.random_decode_batch(3100, s, 8, 8, 64, torch.bfloat16, max_ctx=48, min_ctx=0, store=False)
    say(f"planned decode S={s}")
    dev = to_device(b)
    plan = make_plan(dev, b.max_ctx, b.block_size)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(plan_entries(plan, s),
                                  expected_plan(b.pool.block_tables, b.pool.context_lens, b.max_ctx, b.block_size))
    outs = {}
    for part, ws in ((0, None), ("planned", plan)):
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                   workspace=ws, algo="mfma")
        outs[part] = out
    torch.cuda.synchronize()
    assert torch.equal(outs["planned"].view(torch.int16), outs[0].view(torch.int16))
    assert_close(outs["planned"].float().cpu().double().numpy(), oracle_decode(b, store=False), torch.bfloat16,
                 "planned S=5000")


def test_stale_plan_poisons_only_the_changed_sequences():
    """A plan that no longer matches the lengths or first blocks turns those
    sequences' rows into NaN; every other row equals the single-pass result."""
    s = 50
    b = W.random_decode_batch(2500, s, 16, 8, 128, torch.bfloat16, max_ctx=600, min_ctx=40, store=False)
    b.pool.context_lens[9] = 0
    dev = to_device(b)
    plan = make_plan(dev, b.max_ctx, b.block_size)
    ctx = b.pool.context_lens.copy()
    bt = b.pool.block_tables.copy()
    ctx[3] -= 1                                   # a length that changed
    ctx[9] = 20                                   # an empty sequence that grew
    bt[5, 0], bt[5, 1] = bt[5, 1], bt[5, 0]       # first blocks that changed
    dev["context_lens"].copy_(torch.as_tensor(ctx))
    dev["block_tables"].copy_(torch.as_tensor(bt))
    outs = {}
    for part, ws in ((0, None), ("planned", plan)):
        out = torch.full_like(dev["q"], 7.0)
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                   workspace=ws, algo="mfma")
        outs[part] = out
    torch.cuda.synchronize()
    got = outs["planned"].float().cpu().numpy()
    stale = [3, 5, 9]
    assert np.isnan(got[stale]).all()
    rest = [i for i in range(s) if i not in stale]
    assert torch.equal(outs["planned"][rest].view(torch.int16), outs[0][rest].view(torch.int16))


def test_planned_graph_replays_match_eager():
    """The plan and a few layers' planned fused store + decode captured in one
    graph; every replay (with eager work between them) equals the eager run."""
    wl = W.qwen3_decode(layers=3)
    b0 = wl.batches[0]
    devs = [to_device(b) for b in wl.batches]
    for dv in devs[1:]:
        dv["block_tables"], dv["context_lens"] = devs[0]["block_tables"], devs[0]["context_lens"]
    plan = pkv.new_decode_plan(b0.num_seqs, "cuda")
    plan_launch = pkv.DecodePlanLaunch(plan, devs[0]["block_tables"], devs[0]["context_lens"], b0.max_ctx,
                                       b0.block_size)
    outs = [torch.full_like(dv["q"], float("nan")) for dv in devs]
    launches = [pkv.DecodeStoreLaunch(o, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                      dv["context_lens"], dv["k_new"], dv["v_new"], dv["slot_mapping"],
                                      b.scale, b.max_ctx, partition_size="planned", workspace=plan)
                for o, dv, b in zip(outs, devs, wl.batches)]

    def step():
        plan_launch()
        for f in launches:
            f()

    step()
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    for i, (o, b) in enumerate(zip(eager, wl.batches)):
        assert_close(o.float().cpu().double().numpy(), oracle_decode(b), torch.bfloat16, f"layer {i}")
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for r in range(3):
        for o in outs:
            o.fill_(float("nan"))
        plan.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16)), f"replay {r}"


@pytest.mark.slow
def test_qwen3_layer_planned_store():
    b = W.qwen3_decode(layers=1).batches[0]
    say(f"qwen3 layer planned: S={b.num_seqs}")
    dev = to_device(b)
    plan = make_plan(dev, b.max_ctx, b.block_size)
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["context_lens"], dev["k_new"], dev["v_new"], dev["slot_mapping"],
                                     b.scale, b.max_ctx, partition_size="planned", workspace=plan)
    torch.cuda.synchronize()
    kc, vc = oracle_caches(b)
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert_close(out.float().cpu().double().numpy(), oracle_decode(b, caches=(kc, vc)), torch.bfloat16,
                 "qwen3 planned")

