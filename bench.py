"""Throughput of paged-KV attention on one MI355X.

Headline workload: a Qwen3-0.6B-shaped decode step -- 60 sequences with
contexts U{64..1024}, 16 q / 8 kv heads, head_dim 128, block_size 16, bf16,
28 layers with distinct caches and queries (so the 256 MB last-level cache
cannot serve repeated reads) and one shared block table. One step stores
each sequence's new K/V row and runs decode attention, layer after layer.

value = algorithmic decode bytes per step / step time (GB/s): the K and V
rows inside the contexts, q, out, the block-table entries used and the
context lengths, plus the store's reads and writes. Inputs are resident in
HBM before timing starts.

Also reported on the same JSON line: the roofline of the dominant kernel
(decode, HBM-bound) timed with HIP events on its own stream, a plain-copy
bandwidth measured in the same run, tokens/s, the other standard workloads
(prefix-shared batch, long-context split-K, mixed chunked prefill + decode
with prefill matrix-core utilisation), a parity sample against the CPU
oracle, and the oracle itself timed on a bounded sample of the headline
workload on the host cores (a baseline, not a target).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import paged_attention_kv_store_amd as pkv  # noqa: E402
from paged_attention_kv_store_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, vendor figure


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def decode_bytes(b: W.PagedBatch, unique_blocks=False) -> float:
    e = b.q.element_size()
    hkv, d, bs = b.num_kv_heads, b.head_dim, b.block_size
    ctx = b.pool.context_lens.astype(np.int64)
    if unique_blocks:
        # every distinct (block, row) read once: shared prefix blocks count once
        seen = {}
        for s, c in enumerate(ctx.tolist()):
            nblk = -(-c // bs)
            for j in range(nblk):
                rows = min(bs, c - j * bs)
                blk = int(b.pool.block_tables[s, j])
                seen[blk] = max(seen.get(blk, 0), rows)
        kv_rows = sum(seen.values())
    else:
        kv_rows = int(ctx.sum())
    kv = kv_rows * hkv * d * e * 2
    qo = 2 * b.q.numel() * e
    tables = int((-(-ctx // bs)).sum()) * 4 + len(ctx) * 4
    return float(kv + qo + tables)


def store_bytes(b: W.PagedBatch) -> float:
    if b.k_new is None:
        return 0.0
    t = int((b.slot_mapping >= 0).sum().item())
    row = b.num_kv_heads * b.head_dim * b.q.element_size()
    return float(2 * 2 * t * row + 4 * len(b.slot_mapping))


def prefill_flops(b: W.PagedBatch, causal=True) -> float:
    cu = b.cu_seqlens_q
    tot = 0
    for c in range(len(cu) - 1):
        rows = int(cu[c + 1] - cu[c])
        ctx = int(b.pool.context_lens[c])
        prior = ctx - rows
        pairs = rows * prior + rows * (rows + 1) // 2 if causal else rows * ctx
        tot += pairs
    return float(tot * b.num_q_heads * 4 * b.head_dim)


# --------------------------------------------------------------------------
# device-side workload state
# --------------------------------------------------------------------------

class DecodeCall:
    def __init__(self, b: W.PagedBatch, partition, algo, device, tables=None, lens=None,
                 k_cache=None, v_cache=None):
        self.b = b
        self.q = b.q
        self.kc = b.k_cache if k_cache is None else k_cache
        self.vc = b.v_cache if v_cache is None else v_cache
        self.bt = tables if tables is not None else torch.as_tensor(b.pool.block_tables, device=device)
        self.cl = lens if lens is not None else torch.as_tensor(b.pool.context_lens, device=device)
        self.out = torch.empty_like(b.q)
        self.partition = partition
        self.algo = algo
        self.max_ctx = b.max_ctx
        need = pkv.decode_workspace_size(b.num_seqs, b.num_q_heads, b.head_dim, self.max_ctx,
                                         partition) if partition else 0
        self.ws = torch.empty(max(need, 16), dtype=torch.uint8, device=device)

    def store(self):
        b = self.b
        if b.k_new is not None:
            pkv.kv_cache_store(b.k_new, b.v_new, self.kc, self.vc, b.slot_mapping)

    def decode(self):
        pkv.paged_attention_decode(self.out, self.q, self.kc, self.vc, self.bt, self.cl,
                                   self.b.scale, self.max_ctx, partition_size=self.partition,
                                   workspace=self.ws, algo=self.algo)


def time_region(fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps   # ms


def time_each_launch(fn, launches):
    """Average duration of one launch of fn, events bracketing every launch
    on the stream the kernels run on (torch's current stream)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    fn()
    torch.cuda.synchronize()
    for a, z in evs:
        a.record()
        fn()
        z.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(z) for a, z in evs) / launches


def copy_bandwidth(device, nbytes=2 << 30):
    src = torch.empty(nbytes // 2, dtype=torch.bfloat16, device=device).normal_()
    dst = torch.empty_like(src)
    ms = time_region(lambda: dst.copy_(src), 10, 3)
    return 2 * nbytes / (ms * 1e-3) / 1e9


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# --------------------------------------------------------------------------

def cpu_baseline(b: W.PagedBatch, budget_s=12.0):
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # pragma: no cover
        threadpool_limits = None
    q = W.host_bits(b.q)
    kc, vc = W.host_bits(b.k_cache), W.host_bits(b.v_cache)
    bt, ctx = b.pool.block_tables, b.pool.context_lens
    e = b.q.element_size()
    done_bytes, t_used, seqs = 0.0, 0.0, 0
    ctxm = threadpool_limits(limits=1) if threadpool_limits else None
    try:
        t0 = time.perf_counter()
        while t_used <= budget_s:
            s = seqs % b.num_seqs
            oracle.paged_attention_decode(q[s:s + 1], kc, vc, bt[s:s + 1], ctx[s:s + 1], b.scale,
                                          b.block_size)
            c = int(ctx[s])
            done_bytes += c * b.num_kv_heads * b.head_dim * e * 2 + 2 * b.num_q_heads * b.head_dim * e
            seqs += 1
            t_used = time.perf_counter() - t0
    finally:
        if ctxm is not None:
            ctxm.__exit__(None, None, None)
    return {"value": done_bytes / t_used / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{seqs} sequence decodes (layer 0's {b.num_seqs} sequences, cycled) by the "
                      f"float64 oracle in {t_used:.1f} s on one host core ({seqs / t_used:.1f} seq/s)"}


# --------------------------------------------------------------------------
# secondary workloads
# --------------------------------------------------------------------------

def secondary(device, steps, warmup, decode_algo):
    res = {}
    # prefix-shared Llama-shaped batch: one decode call
    b = W.llama_prefix(device=device).batches[0]
    call = DecodeCall(b, 0, decode_algo, device)
    ms = time_region(call.decode, steps, warmup)
    ub, lb = decode_bytes(b, unique_blocks=True), decode_bytes(b)
    res["llama_prefix"] = {"ms": ms, "unique_GBps": ub / ms / 1e6, "logical_GBps": lb / ms / 1e6,
                           "pct_hbm_peak_unique": 100 * ub / ms / 1e6 / HBM_PEAK_GBS,
                           "tokens_per_s": b.num_seqs / (ms * 1e-3)}
    del call, b
    # long-context split-K
    b = W.long_splitk(device=device).batches[0]
    call = DecodeCall(b, 512, decode_algo, device)
    ms = time_region(call.decode, steps, warmup)
    by = decode_bytes(b)
    res["long_splitk"] = {"ms": ms, "GBps": by / ms / 1e6,
                          "pct_hbm_peak": 100 * by / ms / 1e6 / HBM_PEAK_GBS,
                          "tokens_per_s": b.num_seqs / (ms * 1e-3), "partition": 512}
    del call, b
    # mixed: store, chunked prefill, decode on one stream
    wl = W.mixed(device=device)
    pre, dec = wl.prefill, wl.batches[0]
    bt_pre = torch.as_tensor(pre.pool.block_tables, device=device)
    cu = torch.as_tensor(pre.cu_seqlens_q, device=device)
    cl_pre = torch.as_tensor(pre.pool.context_lens, device=device)
    out_pre = torch.empty_like(pre.q)
    max_q = int(np.diff(pre.cu_seqlens_q).max())
    dcall = DecodeCall(dec, 0, decode_algo, device)

    def store():
        pkv.kv_cache_store(pre.k_new, pre.v_new, pre.k_cache, pre.v_cache, pre.slot_mapping)

    def prefill():
        pkv.paged_attention_prefill_chunk(out_pre, pre.q, pre.k_cache, pre.v_cache, bt_pre, cu,
                                          cl_pre, pre.scale, max_q, pre.max_ctx, causal=True)

    entry = {}
    t_store = time_region(store, steps, warmup)
    t_dec = time_region(dcall.decode, steps, warmup)
    entry["store_ms"] = t_store
    entry["store_GBps"] = store_bytes(pre) / t_store / 1e6
    entry["decode_ms"] = t_dec
    entry["decode_GBps"] = decode_bytes(dec) / t_dec / 1e6
    try:
        t_pre = time_region(prefill, steps, warmup)
        fl = prefill_flops(pre)
        entry["prefill_ms"] = t_pre
        entry["prefill_TFLOPs"] = fl / t_pre / 1e9
        entry["prefill_mfma_util_pct"] = 100 * fl / t_pre / 1e9 / BF16_MFMA_PEAK_TFLOPS
        entry["tokens_per_s"] = 4224 / ((t_store + t_pre + t_dec) * 1e-3)
    except pkv.PkvError as exc:
        entry["prefill"] = f"unavailable: {exc}"
    res["mixed"] = entry
    return res


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--partition", type=int, default=-1,
                    help="decode partition size for the headline step (-1: built-in choice)")
    ap.add_argument("--algo", default="auto", choices=sorted(pkv.DECODE_ALGOS))
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(decode would shard by sequence or kv-head with no exchange; see the design notes)",
              file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    partition = 0 if args.partition < 0 else args.partition

    log("generating the qwen3-shaped decode workload on the GPU")
    wl = W.qwen3_decode(device=device, layers=args.layers)
    calls = [DecodeCall(b, partition, args.algo, device) for b in wl.batches]
    shared_bt, shared_cl = calls[0].bt, calls[0].cl
    for c in calls[1:]:
        c.bt, c.cl = shared_bt, shared_cl
    b0 = wl.batches[0]
    layer_bytes = decode_bytes(b0) + store_bytes(b0)
    step_bytes = layer_bytes * len(calls)

    def step():
        for c in calls:
            c.store()
            c.decode()

    log(f"timing {args.steps} steps ({len(calls)} layers each) after {args.warmup} warmup")
    torch.cuda.synchronize()
    ms = time_region(step, args.steps, args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9

    # dominant kernel: decode on one layer's inputs, events around each launch
    dec_bytes = decode_bytes(b0)
    launches = 28 * 4
    rot = [0]

    def one_decode():
        calls[rot[0] % len(calls)].decode()
        rot[0] += 1

    dec_ms = time_each_launch(one_decode, launches)
    store_ms = time_each_launch(lambda: calls[0].store(), 50)
    copy_gbps = copy_bandwidth(device)

    # parity sample of the timed run's output (layer 0) against the oracle
    import oracle
    seqs = [0, 17, 33, 59]
    okc, ovc = oracle.kv_cache_store(W.host_bits(b0.k_new), W.host_bits(b0.v_new),
                                     W.host_bits(b0.k_cache), W.host_bits(b0.v_cache),
                                     W.host_bits(b0.slot_mapping), b0.block_size)
    calls[0].decode()
    torch.cuda.synchronize()
    want = oracle.paged_attention_decode(W.host_bits(b0.q)[seqs], okc, ovc,
                                         b0.pool.block_tables[seqs], b0.pool.context_lens[seqs],
                                         b0.scale, b0.block_size)
    got = calls[0].out.float().cpu().double().numpy()[seqs]
    parity_err = float(np.abs(got - want).max())
    del okc, ovc

    result = {
        "metric": "decode KV GB/s + % of HBM peak; tokens/s per batch; prefill MFMA util",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_decode", "num_seqs": 60, "context_lens": "U{64..1024}",
                   "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "layers": len(calls), "partition_size": partition, "algo": args.algo,
                   "step": "per layer: kv_cache_store of 60 new rows + paged_attention_decode",
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(b0.num_seqs / (ms * 1e-3), 1),
        "copy_GBps_measured": round(copy_gbps, 1),
        "roofline": {"bound": "hbm", "kernel": "decode (one layer, one launch)",
                     "achieved": round(dec_bytes / (dec_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s",
                     "frac": round(dec_bytes / (dec_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_launch_us": round(dec_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": dec_bytes},
        "store_avg_launch_us": round(store_ms * 1e3, 2),
        "parity_sample_max_abs_err": parity_err,
    }
    if not args.no_secondary:
        del calls, wl
        torch.cuda.empty_cache()
        log("secondary workloads")
        result["secondary"] = secondary(device, max(5, args.steps // 2), 3, args.algo)
    if not args.no_cpu_baseline:
        log("oracle baseline on the host")
        wl1 = W.qwen3_decode(device="cpu", layers=1)
        result["cpu_baseline"] = cpu_baseline(wl1.batches[0])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
