"""Block-table entries past a sequence's last used block are padding: a
serving engine may leave any value there (-1 is common). The kernels may
read such an entry but must never use it, so every launch mode gives the
oracle's result (which reads only the used entries) with the padding set to
-1 or to 2^31 - 1, over bf16 and E4M3 caches, for the decode (plain and with
the store fused), the chunked prefill and the shared-prefix decode.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import assert_close, oracle_caches, say, to_device

pytestmark = pytest.mark.gpu

PADS = [-1, 2 ** 31 - 1]


def _pad(b, value):
    bt = b.pool.block_tables
    for s, c in enumerate(b.pool.context_lens.tolist()):
        bt[s, -(-c // b.block_size):] = value
    return b


@pytest.mark.parametrize("pad", PADS)
def test_decode_bf16_every_mode(pad):
    b = _pad(W.random_decode_batch(8800, 40, 32, 8, 128, torch.bfloat16, max_ctx=900, min_ctx=0, store=True,
                                   block_size=32), pad)
    say(f"padding {pad}: ctx={b.pool.context_lens.tolist()}")
    dev = to_device(b)
    kc, vc = oracle_caches(b)
    want = oracle.paged_attention_decode(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.pool.context_lens,
                                         b.scale, b.block_size)
    # the store fused into the planned decode first, then every mode over the stored caches
    plan = pkv.new_decode_plan(b.num_seqs, "cuda")
    pkv.decode_plan(plan, dev["block_tables"], dev["context_lens"], b.max_ctx, b.block_size)
    out = torch.full_like(dev["q"], float("nan"))
    pkv.paged_attention_decode_store(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                     dev["context_lens"], dev["k_new"], dev["v_new"], dev["slot_mapping"], b.scale,
                                     b.max_ctx, partition_size="planned", workspace=plan)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "planned, store fused")
    for algo, part in [("mfma", 0), ("mfma", "planned"), ("mfma", 128), ("mfma", "balanced"), ("mfma", "auto"),
                       ("valu", 0), ("valu", 128)]:
        out = torch.full_like(dev["q"], float("nan"))
        pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                                   dev["context_lens"], b.scale, b.max_ctx, partition_size=part,
                                   workspace=plan if part == "planned" else None, algo=algo)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"{algo} {part}")


@pytest.mark.parametrize("pad", PADS)
def test_decode_e4m3(pad):
    b = _pad(W.random_decode_batch_fp8(8900, 40, 32, 8, 128, max_ctx=900, min_ctx=0, store=False), pad)
    want = FP8.paged_attention_decode_fp8(W.host_bits(b.q), W.host_bits(b.k_cache), W.host_bits(b.v_cache),
                                          W.host_bits(b.k_scale), W.host_bits(b.v_scale), b.pool.block_tables,
                                          b.pool.context_lens, b.scale, b.block_size)
    dv = {k: getattr(b, k).to("cuda") for k in ("q", "k_cache", "v_cache", "k_scale", "v_scale")}
    bt = torch.as_tensor(b.pool.block_tables, device="cuda")
    cl = torch.as_tensor(b.pool.context_lens, device="cuda")
    for part in (0, "planned", 128):
        ws = None
        if part == "planned":
            ws = pkv.new_decode_plan(b.num_seqs, "cuda")
            pkv.decode_plan(ws, bt, cl, b.max_ctx, b.block_size)
        out = torch.full_like(dv["q"], float("nan"))
        pkv.paged_attention_decode_fp8(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["k_scale"], dv["v_scale"],
                                       bt, cl, b.scale, b.max_ctx, partition_size=part, workspace=ws)
        torch.cuda.synchronize()
        assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, f"E4M3 p={part}")


@pytest.mark.parametrize("pad", PADS)
def test_prefill(pad):
    b = _pad(W.random_prefill_batch(9000, 6, 32, 8, 128, torch.bfloat16, max_rows=70, max_prior=400), pad)
    dv = to_device(b)
    pkv.kv_cache_store(dv["k_new"], dv["v_new"], dv["k_cache"], dv["v_cache"], dv["slot_mapping"])
    kc, vc = oracle_caches(b)
    want = oracle.paged_attention_prefill_chunk(W.host_bits(b.q), kc, vc, b.pool.block_tables, b.cu_seqlens_q,
                                                b.pool.context_lens, b.scale, b.block_size, causal=True)
    out = torch.full_like(dv["q"], float("nan"))
    mq = int(np.diff(b.cu_seqlens_q).max())
    pkv.paged_attention_prefill_chunk(out, dv["q"], dv["k_cache"], dv["v_cache"], dv["block_tables"],
                                      dv["cu_seqlens_q"], dv["context_lens"], b.scale, mq, b.max_ctx, causal=True)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "prefill")


@pytest.mark.parametrize("pad", PADS)
def test_shared_prefix(pad):
    b = _pad(W.random_decode_batch(9100, 32, 32, 8, 128, torch.bfloat16, max_ctx=700, min_ctx=0, store=False,
                                   share_group=4, shared_blocks=6), pad)
    dev = to_device(b)
    want = oracle.paged_attention_decode(W.host_bits(b.q), W.host_bits(b.k_cache), W.host_bits(b.v_cache),
                                         b.pool.block_tables, b.pool.context_lens, b.scale, b.block_size)
    out = torch.full_like(dev["q"], float("nan"))
    prefix = 6 * b.block_size
    pkv.paged_attention_decode_shared_prefix(
        out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
        torch.arange(0, b.num_seqs + 1, 4, dtype=torch.int32, device="cuda"),
        torch.full((b.num_seqs // 4,), prefix, dtype=torch.int32, device="cuda"), b.scale, b.max_ctx, 4, prefix)
    torch.cuda.synchronize()
    assert_close(out.float().cpu().double().numpy(), want, torch.bfloat16, "shared prefix")
