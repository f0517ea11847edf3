"""GPU parity of kv_cache_store: bit-exact against the oracle, every slot."""

import numpy as np
import pytest
import torch

import oracle
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import workloads as W
from tests.gpu_helpers import say, to_device

pytestmark = pytest.mark.gpu


def _check_store(batch, what):
    say(f"store {what}: T={len(batch.slot_mapping)} NB={batch.pool.num_blocks} dtype={batch.q.dtype}")
    dev = to_device(batch)
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                       dev["slot_mapping"])
    torch.cuda.synchronize()
    kc, vc = oracle.kv_cache_store(W.host_bits(batch.k_new), W.host_bits(batch.v_new),
                                   W.host_bits(batch.k_cache), W.host_bits(batch.v_cache),
                                   W.host_bits(batch.slot_mapping), batch.block_size)
    # compare raw bytes: NaN payloads of untouched rows must survive too
    assert W.host_bits(dev["k_cache"]).tobytes() == kc.tobytes()
    assert W.host_bits(dev["v_cache"]).tobytes() == vc.tobytes()


def test_store_tiny_fp32():
    _check_store(W.tiny().batches[0], "tiny")


def test_store_mixed_4224_tokens_bf16():
    _check_store(W.mixed().prefill, "mixed")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("hkv,d", [(1, 64), (2, 128), (8, 128), (3, 64)])
def test_store_shapes_with_padding_slots(dtype, hkv, d):
    b = W.random_decode_batch(11 + hkv, 37, hkv, hkv, d, dtype, max_ctx=200, min_ctx=0)
    slots = b.slot_mapping.clone()
    slots[::5] = -1                      # padding tokens write nothing
    b.slot_mapping = slots
    _check_store(b, f"hkv={hkv} d={d}")


def test_store_skips_slots_outside_the_pool():
    b = W.random_decode_batch(5, 8, 2, 2, 64, torch.float32, max_ctx=60, min_ctx=1)
    nslots = b.pool.num_blocks * b.block_size
    dev = to_device(b)
    before_k = W.host_bits(dev["k_cache"]).copy()
    slots = torch.full((8,), nslots, dtype=torch.int32, device="cuda")
    slots[1] = nslots + 1000
    pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"], slots)
    torch.cuda.synchronize()
    assert W.host_bits(dev["k_cache"]).tobytes() == before_k.tobytes()
