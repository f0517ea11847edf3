"""The decode entry point that allocates nothing (pkv_paged_attention_decode_static,
for callers that cannot allocate) against the existing entry point with a
caller workspace (pkv_paged_attention_decode), through the C ABI: the same
bits on two calls in a row, the second with a smaller input, in the split-K,
work-balanced and single-pass modes, and both within tolerance of the
float64 oracle."""

import pytest
import torch

import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_decode, say, to_device

pytestmark = pytest.mark.gpu

MODES = [
    # (dtype, hq, hkv, d, algo, partition)
    (torch.bfloat16, 32, 8, 128, "mfma", 64),
    (torch.bfloat16, 16, 8, 128, "mfma", "balanced"),
    (torch.bfloat16, 16, 4, 64, "mfma", 0),
    (torch.float32, 8, 4, 64, "valu", 128),
    (torch.bfloat16, 32, 8, 128, "valu", 32),
]


def _both(b, dev, algo, part):
    """(static entry point, existing entry point with its own workspace) outputs."""
    ref = torch.full_like(dev["q"], float("nan"))
    ws = None
    need = pkv.decode_workspace_size(b.num_seqs, b.num_q_heads, b.num_kv_heads, b.head_dim, b.max_ctx, part)
    if need:
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    pkv.paged_attention_decode(ref, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                               dev["context_lens"], b.scale, b.max_ctx, partition_size=part, workspace=ws,
                               algo=algo)
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_decode_static(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                      dev["context_lens"], b.scale, b.max_ctx, partition_size=part, algo=algo)
    torch.cuda.synchronize()
    return out, ref


@pytest.mark.parametrize("case", MODES, ids=lambda c: f"{str(c[0])[6:]}-{c[1]}x{c[2]}-d{c[3]}-{c[4]}-p{c[5]}")
def test_static_scratch_matches_the_workspace_entry_point(case):
    dtype, hq, hkv, d, algo, part = case
    for call, (seqs, max_ctx) in enumerate([(37, 1500), (9, 300)]):     # the second call is smaller
        b = W.random_decode_batch(4000 + 7 * call + hq + d, seqs, hq, hkv, d, dtype, max_ctx=max_ctx,
                                  min_ctx=0, store=False)
        say(f"no-alloc decode {case} call {call}: S={seqs} max_ctx={b.max_ctx}")
        dev = to_device(b)
        out, ref = _both(b, dev, algo, part)
        view = torch.int32 if dtype == torch.float32 else torch.int16
        assert torch.equal(out.view(view), ref.view(view)), "static scratch and workspace results differ"
        assert_close(out.float().cpu().double().numpy(), oracle_decode(b, store=False), dtype,
                     f"no-alloc {algo} p={part} call {call}")

