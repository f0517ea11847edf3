"""GPU tests of the robustness calls: the device-side input checks (integer
reports, compared exactly with counts computed here from their definition),
the workspace initialisation (a garbage-filled workspace, cleared, then
split-K and work-balanced decodes against the oracle), the automatic
partition choice, and the one-call API's reuse of its workspace."""

import numpy as np
import pytest
import torch

import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import binding
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu


def _report(t):
    torch.cuda.synchronize()
    return t.cpu().numpy().tolist()


def _expected_tables(bt, ctx, nb, bs, max_ctx, cu=None, total_q=0, max_q_len=0):
    """The four report entries from their definition (include/pkv.h)."""
    n = len(ctx)
    bad_len = [c < 0 or c > max_ctx for c in ctx]
    bad_ids = []
    for s in range(n):
        used = -(-min(max(int(ctx[s]), 0), max_ctx) // bs)
        bad_ids.append(int(sum(1 for j in range(used) if not 0 <= bt[s][j] < nb)))
    bad_chunk = [False] * n
    if cu is not None:
        for c in range(n):
            rows = cu[c + 1] - cu[c]
            bad_chunk[c] = (rows < 0 or rows > max_q_len or rows > ctx[c] or (c == 0 and cu[0] != 0)
                            or (c == n - 1 and cu[n] != total_q))
    first = [s for s in range(n) if bad_len[s] or bad_ids[s] or bad_chunk[s]]
    return [sum(bad_len), sum(bad_ids), sum(bad_chunk), first[0] if first else n]


def test_check_paged_inputs_clean_and_planted():
    b = W.random_decode_batch(5100, 300, 16, 8, 128, torch.bfloat16, max_ctx=700, min_ctx=0, store=False)
    nb, bs, mb = b.pool.num_blocks, b.block_size, b.max_blocks
    bt, ctx = b.pool.block_tables.copy(), b.pool.context_lens.copy()
    max_ctx = mb * bs
    dev = lambda a: torch.as_tensor(a, device="cuda")
    rep = pkv.check_paged_inputs(dev(bt), dev(ctx), nb, bs, max_ctx)
    assert _report(rep) == [0, 0, 0, 300]
    # plant: lengths outside [0, max_ctx], ids outside the pool among the used
    # entries, and ids outside the pool past the used entries (allowed)
    rng = np.random.default_rng(3)
    ctx[[17, 250]] = [-3, max_ctx + 5]
    live = [s for s in range(300) if 0 < ctx[s] <= max_ctx]
    for s in rng.choice(live, 25, replace=False):
        used = -(-int(ctx[s]) // bs)
        bt[s, rng.integers(0, used)] = rng.choice([nb, nb + 77, -1, -(1 << 30)])
    for s in live[:10]:
        used = -(-int(ctx[s]) // bs)
        if used < mb:
            bt[s, used:] = -5                      # padding past the used entries: not a violation
    want = _expected_tables(bt, ctx, nb, bs, max_ctx)
    say(f"planted tables: want {want}")
    assert _report(pkv.check_paged_inputs(dev(bt), dev(ctx), nb, bs, max_ctx)) == want
    # chunk boundaries
    cu = np.concatenate([[0], np.cumsum(np.minimum(ctx.clip(0), 5))]).astype(np.int32)
    total = int(cu[-1])
    assert _report(pkv.check_paged_inputs(dev(np.ascontiguousarray(b.pool.block_tables)),
                                          dev(np.clip(ctx, 0, max_ctx).astype(np.int32)), nb, bs, max_ctx,
                                          cu_seqlens_q=dev(cu), total_q=total, max_q_len=5))[2] == 0
    cu2 = cu.copy()
    cu2[40] = cu2[41] + 1                        # chunk 39 too long (or chunk 40 negative)
    cu2[-1] += 1                                 # last boundary past total_q
    good_ctx = np.clip(ctx, 0, max_ctx).astype(np.int32)
    want = _expected_tables(b.pool.block_tables, good_ctx, nb, bs, max_ctx, cu2, total, 5)
    got = _report(pkv.check_paged_inputs(dev(np.ascontiguousarray(b.pool.block_tables)), dev(good_ctx), nb, bs,
                                         max_ctx, cu_seqlens_q=dev(cu2), total_q=total, max_q_len=5))
    assert got == want and got[2] >= 2


def _expected_slots(slots, num_slots):
    out = int(np.sum(slots >= num_slots))
    pad = int(np.sum(slots < 0))
    valid = slots[(slots >= 0) & (slots < num_slots)]
    vals, counts = np.unique(valid, return_counts=True)
    dup = int(np.sum(counts - 1))
    dup_slots = set(vals[counts > 1].tolist())
    bad = [t for t, s in enumerate(slots.tolist()) if s >= num_slots or s in dup_slots]
    return [out, dup, pad, bad[0] if bad else len(slots)]


@pytest.mark.parametrize("seed", [0, 1])
def test_check_slots_clean_and_planted(seed):
    wl = W.mixed()
    pre = wl.prefill
    nb, bs = pre.pool.num_blocks, pre.block_size
    slots = W.host_bits(pre.slot_mapping).copy()
    dev = lambda a: torch.as_tensor(a, device="cuda")
    assert _report(pkv.check_slots(dev(slots), nb, bs)) == [0, 0, 0, len(slots)]
    rng = np.random.default_rng(seed)
    t = rng.choice(len(slots), 40, replace=False)
    slots[t[:10]] = -1                              # padding
    slots[t[10:15]] = nb * bs + rng.integers(0, 1000, 5)   # past the pool
    slots[t[15:30]] = slots[t[30:40]].tolist() + slots[t[30:35]].tolist()   # repeated claims
    want = _expected_slots(slots, nb * bs)
    say(f"planted slots: want {want}")
    assert _report(pkv.check_slots(dev(slots), nb, bs)) == want


def test_workspace_init_clears_garbage_for_split_k_and_balanced():
    b = W.random_decode_batch(5200, 40, 32, 8, 128, torch.bfloat16, max_ctx=3000, min_ctx=0, store=False)
    dev = to_device(b)
    want = oracle_decode(b, store=False)
    for part in (256, "balanced"):
        need = pkv.decode_workspace_size(b.num_seqs, 32, 8, 128, b.max_ctx, part)
        ws = torch.randint(-(1 << 31), (1 << 31) - 1, ((need + 3) // 4,), dtype=torch.int32,
                           device="cuda").view(torch.uint8)       # garbage counters
        pkv.decode_workspace_init(ws)
        for call in range(2):
            out = torch.full_like(dev["q"], float("nan"))
            pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                       dev["context_lens"], b.scale, b.max_ctx, partition_size=part, workspace=ws)
            torch.cuda.synchronize()
            assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"init p={part} call {call}")
        counters = 65536 if part == 256 else 4096
        assert int(ws[:4 * counters].view(torch.int32).abs().sum()) == 0


def test_workspace_init_and_decode_in_a_graph():
    """The initialisation is a kernel, not a memset node: an init + split-K
    decode captured together replay with the eager bits every time."""
    b = W.random_decode_batch(5300, 24, 16, 8, 128, torch.bfloat16, max_ctx=2500, min_ctx=100, store=False)
    dev = to_device(b)
    need = pkv.decode_workspace_size(b.num_seqs, 16, 8, 128, b.max_ctx, 128)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.full_like(dev["q"], float("nan"))
    call = pkv.DecodeLaunch(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                            b.scale, b.max_ctx, partition_size=128, workspace=ws)

    def step():
        pkv.decode_workspace_init(ws)
        call()
    step()
    torch.cuda.synchronize()
    eager = out.clone()
    assert_close(eager.float().cpu().double().numpy(), oracle_decode(b, store=False), torch.bfloat16, "eager")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for r in range(4):
        out.fill_(float("nan"))
        ws.fill_(0x5A)                             # garbage between replays, cleared by the replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {r}"


def test_auto_choices_on_this_device():
    """On the MI355X (256 compute units): the long-context batch (256 items)
    takes the work-balanced decode, a few sequences split-K, large or short
    batches one pass."""
    b = W.long_splitk().batches[0]
    part = pkv.decode_auto_partition(b.num_seqs, b.num_kv_heads, b.max_ctx)
    say(f"auto partition for 32 seqs x 8 kv-heads up to {b.max_ctx} tokens: {part}")
    assert part == pkv.PARTITION_BALANCED
    assert pkv.decode_auto_partition(2, 8, 32768) == 2048
    assert pkv.decode_auto_partition(60, 8, 1024) == 0
    assert pkv.decode_auto_partition(256, 8, 4096) == 0


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_auto_work_balanced_choice_and_its_fallback(dtype):
    """A mid-sized batch of long contexts: bf16 runs the work-balanced decode,
    fp32 (vector kernel) the split-K fallback, both in auto's workspace."""
    b = W.random_decode_batch(5450, 20, 32, 8, 128, dtype, max_ctx=6000, min_ctx=0, store=False)
    assert pkv.decode_auto_partition(b.num_seqs, b.num_kv_heads, b.max_ctx) == pkv.PARTITION_BALANCED
    dev = to_device(b)
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                               dev["context_lens"], b.scale, b.max_ctx, partition_size="auto")
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), oracle_decode(b, store=False), dtype, f"auto {dtype}")


@pytest.mark.parametrize("algo,dtype", [("valu", torch.float32), ("mfma", torch.bfloat16)])
def test_auto_on_the_tiny_and_small_batches(algo, dtype):
    for b in (W.tiny().batches[0] if dtype == torch.float32 else
              W.random_decode_batch(5400, 3, 16, 8, 128, dtype, max_ctx=5000, min_ctx=2500),
              W.random_decode_batch(5401, 5, 8, 4, 64, dtype, max_ctx=4000, min_ctx=0)):
        dev = to_device(b)
        if b.k_new is not None:
            pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], dev["slot_mapping"])
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size="auto", algo=algo)
        torch.cuda.synchronize()
        part = pkv.decode_auto_partition(b.num_seqs, b.num_kv_heads, b.max_ctx)
        assert_close(out.float().cpu().double().numpy(), oracle_decode(b), dtype, f"auto ({part}) {algo}")


def test_one_call_api_reuses_its_workspace():
    b = W.random_decode_batch(5500, 20, 32, 8, 128, torch.bfloat16, max_ctx=2000, min_ctx=0, store=False)
    dev = to_device(b)
    want = oracle_decode(b, store=False)
    binding._WS_CACHE.clear()
    ptrs = []
    for part in (64, 128, 64):
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"one-call p={part}")
        ptrs.append(next(iter(binding._WS_CACHE.values())).data_ptr())
    assert len(binding._WS_CACHE) == 1
    assert ptrs[0] == ptrs[1] == ptrs[2]           # made for the first call, which needs the most


def test_split_k_and_work_balanced_alternate_on_one_workspace():
    """Both modes keep their arrival counters in the workspace's first 256 KiB
    and their partial results after it, and leave the counters zero, so one
    workspace serves them in any order. 700 sequences x 8 kv-heads put the
    split-K counters well past the 4096 work-balanced ones, where the
    work-balanced pieces would lie if the layouts did not share the block.
    The one-call functions' cached workspace is checked the same way."""
    b = W.random_decode_batch(5600, 700, 32, 8, 128, torch.bfloat16, max_ctx=2000, min_ctx=0, store=False)
    dev = to_device(b)
    want = oracle_decode(b, store=False)
    order = ("balanced", 256, "balanced", 512, 256, "balanced")
    need = max(pkv.decode_workspace_size(b.num_seqs, 32, 8, 128, b.max_ctx, p) for p in order)
    ws = pkv.new_decode_workspace(need, "cuda")
    for cached in (False, True):
        for part in order:
            say(f"700 seqs, partition {part}, {'cached' if cached else 'one'} workspace")
            out = torch.full_like(dev["q"], float("nan"))
            pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                       dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                       workspace=None if cached else ws, algo="mfma")
            torch.cuda.synchronize()
            assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"partition {part}")
    assert int(ws[:65536 * 4].view(torch.int32).abs().sum()) == 0
