"""Shared pieces of the GPU parity tests: run the HIP path through the C ABI,
run the oracle on the very same host bits, compare."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd.workloads import PagedBatch, host_bits

# Tolerances on max |gpu - oracle|: 1e-5 for fp32 inputs, 2e-2 for bf16 ones.
# bf16: the output is rounded once to bf16 (half an ulp is 2^-9 relative,
# 0.0078 at |out| in [2, 4), 0.0156 in [4, 8)); |out| <= max |V| (about 5.5
# for N(0,1) values at these sizes); fp32 accumulation error is ~1e-6.
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(batch: PagedBatch, device="cuda"):
    d = {
        "q": batch.q.to(device),
        "k_cache": batch.k_cache.to(device),
        "v_cache": batch.v_cache.to(device),
        "block_tables": torch.as_tensor(batch.pool.block_tables, device=device),
        "context_lens": torch.as_tensor(batch.pool.context_lens, device=device),
    }
    if batch.k_new is not None:
        d["k_new"] = batch.k_new.to(device)
        d["v_new"] = batch.v_new.to(device)
        d["slot_mapping"] = batch.slot_mapping.to(device)
    if batch.cu_seqlens_q is not None:
        d["cu_seqlens_q"] = torch.as_tensor(batch.cu_seqlens_q, device=device)
    return d


def gpu_decode(batch: PagedBatch, dev=None, algo="auto", partition_size=0, store=True):
    """Store (if the batch has new rows) then decode on the GPU; returns float64 numpy."""
    dev = dev or to_device(batch)
    if store and batch.k_new is not None:
        pkv.kv_cache_store(dev["k_new"], dev["v_new"], dev["k_cache"], dev["v_cache"],
                           dev["slot_mapping"])
    out = torch.full_like(dev["q"], float("nan"))   # a row no workgroup writes stays NaN
    pkv.paged_attention_decode(out, dev["q"], dev["k_cache"], dev["v_cache"],
                               dev["block_tables"], dev["context_lens"], batch.scale,
                               batch.max_ctx, partition_size=partition_size, algo=algo)
    torch.cuda.synchronize()
    return out.float().cpu().double().numpy()


def oracle_caches(batch: PagedBatch, store=True):
    kc, vc = host_bits(batch.k_cache), host_bits(batch.v_cache)
    if store and batch.k_new is not None:
        kc, vc = oracle.kv_cache_store(host_bits(batch.k_new), host_bits(batch.v_new), kc, vc,
                                       host_bits(batch.slot_mapping), batch.block_size)
    return kc, vc


def oracle_decode(batch: PagedBatch, caches=None, seqs=None, store=True):
    kc, vc = caches if caches is not None else oracle_caches(batch, store)
    q = host_bits(batch.q)
    bt, ctx = batch.pool.block_tables, batch.pool.context_lens
    if seqs is not None:
        q, bt, ctx = q[seqs], bt[seqs], ctx[seqs]
    return oracle.paged_attention_decode(q, kc, vc, bt, ctx, batch.scale, batch.block_size)


def assert_close(got, want, dtype, what=""):
    tol = TOL[dtype]
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want).max() if got.size else 0.0
    say(f"  {what}: max|gpu-oracle| = {err:.3e} (tol {tol:g})")
    assert err <= tol, f"{what}: max abs error {err} > {tol}"
