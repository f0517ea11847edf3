"""GPU parity of the shared-prefix decode against the float64 oracle's plain
decode (the same function by definition), through the C ABI."""

import numpy as np
import pytest
import torch

import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu


def run_shared(b, starts, prefixes, dev=None):
    dev = dev or to_device(b)
    out = torch.empty_like(dev["q"])
    gs = torch.as_tensor(np.asarray(starts, np.int32), device="cuda")
    gp = torch.as_tensor(np.asarray(prefixes, np.int32), device="cuda")
    pkv.paged_attention_decode_shared_prefix(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                             dev["context_lens"], gs, gp, b.scale, b.max_ctx,
                                             int(np.diff(starts).max()), int(max(prefixes)))
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


CASES = [
    # (seed, groups, group_size, hq, hkv, shared_blocks, max_ctx, block_size)
    (1, 4, 8, 32, 8, 4, 400, 16),
    (2, 3, 5, 16, 8, 2, 300, 32),
    (3, 6, 2, 8, 8, 3, 500, 16),
    (4, 2, 40, 16, 2, 2, 200, 16),     # group larger than one q-tile of the first pass (G = 8)
    (5, 5, 4, 32, 32, 1, 150, 64),     # G = 1
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"s{c[0]}-{c[1]}x{c[2]}-{c[3]}x{c[4]}-bs{c[7]}")
def test_groups_match_plain_decode(case):
    seed, ng, gsz, hq, hkv, shared, max_ctx, bs = case
    n = ng * gsz
    b = W.random_decode_batch(2000 + seed, n, hq, hkv, 128, torch.bfloat16, max_ctx=max_ctx, min_ctx=0,
                              block_size=bs, store=False, share_group=gsz, shared_blocks=shared)
    starts = np.arange(0, n + 1, gsz)
    prefixes = [shared * bs] * ng
    say(f"shared prefix {case} ctx={b.pool.context_lens.tolist()}")
    assert_close(run_shared(b, starts, prefixes), oracle_decode(b, store=False), torch.bfloat16, "shared")


def test_singletons_and_empty_suffixes():
    """Unshared sequences as groups of one with prefix 0, and a group whose
    members' contexts end exactly at the prefix."""
    b = W.random_decode_batch(2100, 12, 32, 8, 128, torch.bfloat16, max_ctx=300, min_ctx=0, store=False,
                              share_group=4, shared_blocks=3)
    b.pool.context_lens[4:8] = 48                      # group 1: nothing after its 48 shared tokens
    starts = [0, 4, 8, 9, 10, 11, 12]
    prefixes = [48, 48, 0, 0, 0, 0]
    got = run_shared(b, starts, prefixes)
    assert_close(got, oracle_decode(b, store=False), torch.bfloat16, "mixed groups")


def test_prefix_not_a_multiple_of_16_poisons_its_rows():
    b = W.random_decode_batch(2200, 8, 16, 8, 128, torch.bfloat16, max_ctx=200, min_ctx=0, store=False,
                              share_group=4, shared_blocks=2)
    got = run_shared(b, [0, 4, 8], [32, 20])
    assert np.isnan(got[4:]).all()
    assert_close(got[:4], oracle_decode(b, seqs=[0, 1, 2, 3], store=False), torch.bfloat16, "good group")


def test_out_of_pool_block_in_the_prefix_poisons_the_group():
    b = W.random_decode_batch(2300, 8, 16, 8, 128, torch.bfloat16, max_ctx=200, min_ctx=0, store=False,
                              share_group=4, shared_blocks=2)
    b.pool.block_tables[4, 1] = b.pool.num_blocks + 2      # read through the group's first member
    got = run_shared(b, [0, 4, 8], [32, 32])
    assert np.isnan(got[4:]).all()
    assert_close(got[:4], oracle_decode(b, seqs=[0, 1, 2, 3], store=False), torch.bfloat16, "good group")



def test_empty_contexts_give_zero_rows():
    """A sequence with no token (a group of one, prefix 0) gives a zero row,
    as the plain decode does; its neighbours are unaffected."""
    b = W.random_decode_batch(2400, 12, 32, 8, 128, torch.bfloat16, max_ctx=250, min_ctx=1, store=False,
                              share_group=4, shared_blocks=2)
    b.pool.context_lens[9] = 0
    starts = [0, 4, 8, 9, 10, 11, 12]
    prefixes = [32, 32, 0, 0, 0, 0]
    got = run_shared(b, starts, prefixes)
    assert (got[9] == 0).all()
    assert_close(got, oracle_decode(b, store=False), torch.bfloat16, "with an empty context")


def test_repeated_calls_on_one_workspace_agree_exactly():
    """The workspace carries nothing from one call to the next: repeated
    calls give the same bits."""
    b = W.random_decode_batch(2500, 48, 32, 8, 128, torch.bfloat16, max_ctx=900, min_ctx=0, store=False,
                              share_group=8, shared_blocks=20)
    dev = to_device(b)
    starts = np.arange(0, 49, 8)
    prefixes = [320] * 6
    first = run_shared(b, starts, prefixes, dev)
    assert_close(first, oracle_decode(b, store=False), torch.bfloat16, "first call")
    for i in range(4):
        assert np.array_equal(run_shared(b, starts, prefixes, dev), first), f"call {i + 2} differs"


def test_graph_replays_match_eager():
    """Both passes captured in one graph, replayed several times with eager
    calls and synchronisation in between."""
    b = W.random_decode_batch(2600, 24, 32, 8, 128, torch.bfloat16, max_ctx=600, min_ctx=0, store=False,
                              share_group=6, shared_blocks=10)
    dev = to_device(b)
    starts = np.arange(0, 25, 6)
    prefixes = [160] * 4
    want = oracle_decode(b, store=False)
    eager = run_shared(b, starts, prefixes, dev)
    assert_close(eager, want, torch.bfloat16, "eager")
    gs = torch.as_tensor(np.asarray(starts, np.int32), device="cuda")
    gp = torch.as_tensor(np.asarray(prefixes, np.int32), device="cuda")
    out = torch.zeros_like(dev["q"])
    launch = pkv.SharedPrefixDecodeLaunch(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                          dev["context_lens"], gs, gp, b.scale, b.max_ctx, 6, 160)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        launch(s)                      # warm-up on the capture stream
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        launch(s)
    torch.cuda.synchronize()
    for i in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().double().numpy()
        assert np.array_equal(got, eager), f"replay {i} differs from the eager call"
        run_shared(b, starts, prefixes, dev)    # eager work between replays
