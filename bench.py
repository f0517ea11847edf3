"""Throughput of paged-KV attention on one MI355X.

Headline workload (one "step"): a Qwen3-0.6B-shaped decode step -- 60
sequences with contexts U{64..1024}, 16 q / 8 kv heads, head_dim 128,
block_size 16, bf16, 28 layers with distinct caches and queries (so the
256 MB last-level cache cannot serve repeated reads) and one shared block
table. Per layer the step stores each sequence's new K/V row
(kv_cache_store) and runs decode attention (paged_attention_decode). The
28-layer step is captured once in a HIP graph and replayed, as a serving
engine replays its decode step; every replay used for timing is checked
bit-exact against the eagerly launched step first (--eager times eager
launches instead).

value = algorithmic bytes per step / step time, in GB/s: the K and V rows
inside the contexts, q, out, the block-table entries used and the context
lengths, plus the store's reads and writes. Inputs are resident in HBM
before timing starts.

Also on the same JSON line: the roofline of the dominant kernel (decode,
HBM-bound) from HIP events around each launch on the launch stream, the HBM
traffic that rocprofv3 counters measured for that kernel (from
profiles/decode_qwen3_traffic.json, null if the kernel source changed since),
the bandwidth a plain streaming-read kernel reaches in the same run (over
4 GiB, and over 28 buffers of one decode layer's bytes launched back to back,
the achievable ceiling for a launch of that size), a plain read of each
bandwidth workload's own K/V tiles through its block table (the ceiling of
that access pattern; the line reports the kernel's time as a fraction of
it), tokens/s, the other
standard workloads (prefix-shared batch, long-context decode in the
automatic partition mode, mixed chunked prefill + decode with the prefill's
matrix-core utilisation and a cold-cache store, verification of 4
drafted-token rows per sequence, the headline step over an E4M3 cache), a
parity sample against the CPU oracle, and the oracle itself timed on the
host's cores (a worker pool started before the GPU is touched) for a few
seconds per workload, on the input bits the GPU used (a baseline, not a
target).

Other modes: --pmc-pass runs only the headline decode launches and one
calibration copy of known size (for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE);
--summarize-pmc FETCH_CSV WRITE_CSV turns two such runs into
profiles/decode_qwen3_traffic.json.
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
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

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix cores, vendor figure
CLOCK_HZ = 2.4e9                # MI355X peak engine clock
NUM_SIMDS = 256 * 4             # 256 compute units of 4 SIMDs
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_qwen3_traffic.json")
DECODE_SOURCES = ["decode.hip", "common.h", "device_utils.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_source_hash():
    """Hash of the decode kernel's code: the sources with // comments and
    whitespace removed, so that editing a comment keeps measured counters."""
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        with open(os.path.join(ROOT, "paged_attention_kv_store_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


# --------------------------------------------------------------------------
# algorithmic work
# --------------------------------------------------------------------------

def decode_bytes(b: W.PagedBatch, unique_blocks=False) -> float:
    e = b.k_cache.element_size()        # 1 for E4M3 caches
    hkv, d, bs = b.num_kv_heads, b.head_dim, b.block_size
    ctx = b.pool.context_lens.astype(np.int64)
    if unique_blocks:
        # every distinct (block, row) read once: shared prefix blocks count once
        seen = {}
        for s, c in enumerate(ctx.tolist()):
            for j in range(-(-c // bs)):
                rows = min(bs, c - j * bs)
                blk = int(b.pool.block_tables[s, j])
                seen[blk] = max(seen.get(blk, 0), rows)
        kv_rows = sum(seen.values())
    else:
        kv_rows = int(ctx.sum())
    kv = kv_rows * hkv * d * e * 2
    qo = 2 * b.q.numel() * b.q.element_size()
    tables = int((-(-ctx // bs)).sum()) * 4 + len(ctx) * 4
    return float(kv + qo + tables)


def store_bytes(b: W.PagedBatch) -> float:
    if b.k_new is None:
        return 0.0
    t = int((b.slot_mapping >= 0).sum().item())
    row_in = b.num_kv_heads * b.head_dim * b.k_new.element_size()
    row_out = b.num_kv_heads * b.head_dim * b.k_cache.element_size()
    return float(2 * t * (row_in + row_out) + 4 * len(b.slot_mapping))


def prefill_flops(b: W.PagedBatch, causal=True) -> float:
    cu = b.cu_seqlens_q
    tot = 0
    for c in range(len(cu) - 1):
        rows = int(cu[c + 1] - cu[c])
        ctx = int(b.pool.context_lens[c])
        prior = ctx - rows
        tot += rows * prior + rows * (rows + 1) // 2 if causal else rows * ctx
    return float(tot * b.num_q_heads * 4 * b.head_dim)


# --------------------------------------------------------------------------
# timing helpers (HIP events on torch's current stream, where every launch goes)
# --------------------------------------------------------------------------

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


def time_region_settled(fn, steps, warmup, settle_s=0.3):
    """time_region for a compute-bound kernel: untimed calls of fn for
    settle_s seconds first, so the engine clock has left its idle state
    (the host-side work before it, such as the oracle baseline, leaves the
    GPU idle). The timed calls are the same."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < settle_s:
        for _ in range(4):
            fn()
        torch.cuda.synchronize()
    return time_region(fn, steps, warmup)


def time_each_step(fn, steps):
    """Milliseconds of each of `steps` calls, one HIP event pair around each."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, z in evs:
        a.record()
        fn()
        z.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(z) for a, z in evs]


def gpu_hold(ms):
    """Keep the stream busy for about `ms` so that the launches queued behind
    it run back to back, independent of host launch latency."""
    try:
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))
    except Exception:  # pragma: no cover
        pass


def time_each_launch(fns, rounds):
    """Average duration of one launch: the launches run back to back on the
    stream (queued behind a GPU hold, so host overhead does not enter), one
    HIP event pair brackets them all."""
    for fn in fns:
        fn()
    torch.cuda.synchronize()
    gpu_hold(5.0)
    a = torch.cuda.Event(enable_timing=True)
    z = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(rounds):
        for fn in fns:
            fn()
    z.record()
    torch.cuda.synchronize()
    return a.elapsed_time(z) / (rounds * len(fns))


PROBE_LIB = os.path.join(ROOT, "paged_attention_kv_store_amd", "libpkv_probe.so")
_probe = None


def probe_lib():
    """libpkv_probe.so: the streaming-read kernel (a measurement aid)."""
    global _probe
    if _probe is None:
        import ctypes
        if not os.path.exists(PROBE_LIB):
            raise RuntimeError(f"{PROBE_LIB} is not built; run paged_attention_kv_store_amd/build.py")
        _probe = ctypes.CDLL(PROBE_LIB)
        _probe.pkv_probe_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_void_p]
        _probe.pkv_probe_hbm_read.restype = ctypes.c_int
        _probe.pkv_probe_paged_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                                ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                                ctypes.c_void_p]
        _probe.pkv_probe_paged_read.restype = ctypes.c_int
    return _probe


def hbm_read(buf, workgroups, in_flight, sink):
    rc = probe_lib().pkv_probe_hbm_read(buf.data_ptr(), buf.numel() * buf.element_size(), workgroups, in_flight,
                                        sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"pkv_probe_hbm_read: HIP error {rc}")


PROBE_SHAPES = [(512, 8), (1024, 4), (2048, 8), (2048, 16), (4096, 16)]   # (workgroups, loads in flight)


def read_ceiling(device, layer_bytes, layers, fp8_layer_bytes=None):
    """Bandwidth of a plain streaming read (in-tree kernel, every byte read
    once with 16-byte loads), the best of a few launch shapes: over one 4 GiB
    buffer, and over `layers` distinct buffers of one decode layer's bytes
    launched back to back (as the step's decode launches are); the same for
    the E4M3 layer's bytes when given."""
    sink = torch.zeros(8192, dtype=torch.int32, device=device)
    big = torch.empty(4 << 30, dtype=torch.uint8, device=device).fill_(1)
    best_big = min(time_each_launch([lambda wg=wg, f=f: hbm_read(big, wg, f, sink)], 5)
                   for wg, f in PROBE_SHAPES)
    del big
    torch.cuda.empty_cache()

    def per_layer(nbytes):
        nb = int(nbytes) // 16 * 16
        bufs = [torch.empty(nb, dtype=torch.uint8, device=device).fill_(1) for _ in range(layers)]
        best = min(time_each_launch([lambda b=b, wg=wg, f=f: hbm_read(b, wg, f, sink) for b in bufs], 4)
                   for wg, f in PROBE_SHAPES)
        del bufs
        torch.cuda.empty_cache()
        return nb, best
    nb, best_layer = per_layer(layer_bytes)
    out = {"kernel": "hbm_read_kernel (paged_attention_kv_store_amd/probe/hbm_read.hip), best of "
                     + ", ".join(f"{wg} workgroups x {f} loads in flight" for wg, f in PROBE_SHAPES),
           "GBps_4GiB": round((4 << 30) / (best_big * 1e-3) / 1e9, 1),
           "GBps_layer_bytes": round(nb / (best_layer * 1e-3) / 1e9, 1),
           "layer_bytes_us": round(best_layer * 1e3, 2), "layer_bytes": nb, "layer_buffers": layers}
    if fp8_layer_bytes:
        nb8, best8 = per_layer(fp8_layer_bytes)
        out.update({"GBps_fp8_layer_bytes": round(nb8 / (best8 * 1e-3) / 1e9, 1),
                    "fp8_layer_bytes_us": round(best8 * 1e3, 2), "fp8_layer_bytes": nb8})
    return out


def paged_tile_offsets(b, slice_bytes, device):
    """Byte offset of the first row slice of every 16-token tile of a decode
    layer, kv-head first, then sequence, then tile: the tiles the decode reads,
    for rows of num_kv_heads slices of `slice_bytes` each."""
    bt, ctx, bs, hkv = b.pool.block_tables, b.pool.context_lens.astype(np.int64), b.block_size, b.num_kv_heads
    pitch = hkv * slice_bytes
    seq = np.repeat(np.arange(len(ctx)), (ctx + 15) // 16)
    tok0 = np.concatenate([16 * np.arange((c + 15) // 16) for c in ctx]).astype(np.int64)
    rows = bt[seq, tok0 // bs].astype(np.int64) * bs + tok0 % bs
    offs = (rows[None, :] * pitch + np.arange(hkv, dtype=np.int64)[:, None] * slice_bytes).reshape(-1)
    return torch.as_tensor(offs, dtype=torch.int64, device=device), pitch


def paged_read_ceiling(device, batches):
    """Time of a plain read of one decode layer's K/V tiles in the decode's
    access pattern (16-row tiles of one kv-head's row slices at the cache's
    row pitch, through the block table), split evenly over the waves, with
    nothing computed: in-tree kernel, over the layers' distinct caches launched
    back to back, the best of three grid sizes. Also for rows of one-byte
    elements (the E4M3 layer's pattern), read from the first half of the same
    caches."""
    sink = torch.zeros(8192, dtype=torch.int32, device=device)
    b0 = batches[0]
    out = {"kernel": "paged_read_kernel (paged_attention_kv_store_amd/probe/hbm_read.hip): the layer's "
                     "16-token K and V tiles as the decode reads them, split evenly over the waves, "
                     "nothing computed; best of 512, 1024 and 2048 workgroups of 4 waves"}
    for name, slice_bytes in (("", b0.head_dim * 2), ("fp8_", b0.head_dim)):
        offs, pitch = paged_tile_offsets(b0, slice_bytes, device)
        stream = torch.cuda.current_stream().cuda_stream

        def launch(b, wg):
            rc = probe_lib().pkv_probe_paged_read(b.k_cache.data_ptr(), b.v_cache.data_ptr(), offs.data_ptr(),
                                                  offs.numel(), pitch, slice_bytes, wg, sink.data_ptr(), stream)
            if rc != 0:
                raise RuntimeError(f"pkv_probe_paged_read: HIP error {rc}")
        best = min(time_each_launch([lambda b=b, wg=wg: launch(b, wg) for b in batches], 4) for wg in (512, 1024, 2048))
        nbytes = offs.numel() * 16 * slice_bytes * 2
        out[name + "paged_read_us"] = round(best * 1e3, 2)
        out[name + "paged_read_bytes"] = int(nbytes)
        out[name + "GBps_paged_read"] = round(nbytes / (best * 1e-3) / 1e9, 1)
    return out


def paged_read_ms(b, device):
    """Time of a plain read of one batch's K/V tiles in the decode's order
    (kv-head first, as `paged_read_ceiling`), split evenly over the waves,
    nothing computed: the best of three grid sizes, ten launches each (the
    bandwidth batches exceed the last-level cache)."""
    sink = torch.zeros(8192, dtype=torch.int32, device=device)
    offs, pitch = paged_tile_offsets(b, b.head_dim * 2, device)
    stream = torch.cuda.current_stream().cuda_stream

    def launch(wg):
        rc = probe_lib().pkv_probe_paged_read(b.k_cache.data_ptr(), b.v_cache.data_ptr(), offs.data_ptr(), offs.numel(),
                                              pitch, b.head_dim * 2, wg, sink.data_ptr(), stream)
        if rc != 0:
            raise RuntimeError(f"pkv_probe_paged_read: HIP error {rc}")
    return min(time_each_launch([lambda wg=wg: launch(wg)], 10) for wg in (512, 1024, 2048))


def cold_store_ms(store, device, rounds=10):
    """Median time of one store launch after a 1 GiB streaming read has
    replaced the last-level cache's contents (so neither the new rows nor the
    cache rows it writes are resident), one event pair around the store."""
    sink = torch.zeros(8192, dtype=torch.int32, device=device)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=device).fill_(1)
    times = []
    for _ in range(rounds):
        hbm_read(flush, 2048, 8, sink)
        a = torch.cuda.Event(enable_timing=True)
        z = torch.cuda.Event(enable_timing=True)
        a.record()
        store()
        z.record()
        torch.cuda.synchronize()
        times.append(a.elapsed_time(z))
    del flush
    return float(np.median(times))


# --------------------------------------------------------------------------
# headline workload
# --------------------------------------------------------------------------

class Layer:
    def __init__(self, b: W.PagedBatch, bt, cl, partition, algo, plan=None):
        self.b = b
        self.out = torch.empty_like(b.q)
        self.store = pkv.StoreLaunch(b.k_new, b.v_new, b.k_cache, b.v_cache, b.slot_mapping)
        self.decode = pkv.DecodeLaunch(self.out, b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                                       b.max_ctx, partition_size=partition, algo=algo, workspace=plan)
        self.fused = pkv.DecodeStoreLaunch(self.out, b.q, b.k_cache, b.v_cache, bt, cl, b.k_new,
                                           b.v_new, b.slot_mapping, b.scale, b.max_ctx,
                                           partition_size=partition, algo=algo, workspace=plan)


def parse_partition(v):
    return v if v in ("planned", "balanced") else int(v)


def build_headline(device, layers, partition, algo):
    """The 28 layers, and the step's plan launch (None unless the decode is
    planned: one plan per step, written before the first layer, serves all)."""
    wl = W.qwen3_decode(device=device, layers=layers)
    b0 = wl.batches[0]
    bt = torch.as_tensor(b0.pool.block_tables, device=device)
    cl = torch.as_tensor(b0.pool.context_lens, device=device)
    plan = plan_launch = None
    if partition == "planned":
        plan = pkv.new_decode_plan(b0.num_seqs, device)
        plan_launch = pkv.DecodePlanLaunch(plan, bt, cl, b0.max_ctx, b0.block_size)
        plan_launch()
    return wl, [Layer(b, bt, cl, partition, algo, plan) for b in wl.batches], plan_launch


def capture_step(step, outs, replays=3):
    """Capture `step` in a HIP graph and check replays against eager output."""
    step()
    torch.cuda.synchronize()
    want = [o.clone() for o in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    for _ in range(replays):
        for o in outs:
            o.fill_(float("nan"))          # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            if not torch.equal(o.view(torch.int16), w.view(torch.int16)):
                raise RuntimeError("graph replay differs from the eager step")
    return graph


def load_traffic(dec_bytes):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("decode_source_hash") != decode_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


# --------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the headline workload
# --------------------------------------------------------------------------

def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown CPU"


def baseline_workers():
    # the host share of one GPU is 16 threads; never more than the affinity allows
    return max(1, min(16, len(os.sched_getaffinity(0))))


class OracleBaseline:
    """The float64 oracle timed on the host's cores (oracle/baseline.py, a
    helper process whose worker pool starts before this process touches the
    GPU). Each workload's inputs are copied back from the GPU, so the oracle
    times the very bits the kernels read."""

    def __init__(self, budget_s):
        import subprocess
        self.workers = baseline_workers()
        self.budget_s = budget_s
        self.proc = subprocess.Popen([sys.executable, "-m", "oracle.baseline", str(self.workers)], cwd=ROOT,
                                     stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
        self.ready = None
        self.results = {}

    def _reply(self):
        line = self.proc.stdout.readline()
        if not line:
            raise RuntimeError("the oracle baseline helper ended")
        return json.loads(line)

    def run(self, name, kind, arrays, scale, block_size, work, unit, describe):
        """Time the oracle on a sample of one workload. arrays: host numpy
        (bf16 as uint16 bits); work(units) -> (algorithmic work of the sample,
        tokens or rows of the sample)."""
        import shutil
        import tempfile
        if self.ready is None:
            self.ready = self._reply()
        d = tempfile.mkdtemp(prefix="pkv_baseline_")
        try:
            for k, a in arrays.items():
                np.save(os.path.join(d, k + ".npy"), np.ascontiguousarray(a), allow_pickle=False)
            req = {"kind": kind, "dir": d, "scale": scale, "block_size": block_size, "budget_s": self.budget_s}
            self.proc.stdin.write(json.dumps(req) + "\n")
            self.proc.stdin.flush()
            rep = self._reply()
        finally:
            shutil.rmtree(d, ignore_errors=True)
        if "error" in rep:
            raise RuntimeError(f"oracle baseline on {name}: {rep['error']}")
        amount, items = work(rep["units"])
        self.results[name] = {"value": round(amount / rep["seconds"], 3), "unit": unit,
                              "items_per_s": round(items / rep["seconds"], 2),
                              "seconds": round(rep["seconds"], 2),
                              "sample": f"{describe(rep['units'])}, {rep['passes']:.2f} passes"}
        return self.results[name]

    def close(self):
        try:
            self.proc.stdin.write("quit\n")
            self.proc.stdin.flush()
            self.proc.wait(timeout=60)
        except Exception:  # pragma: no cover
            self.proc.kill()


def decode_arrays(b, k_cache=None, v_cache=None):
    """Host copies of a decode batch's inputs as the GPU holds them."""
    return {"q": W.host_bits(b.q), "k_cache": W.host_bits(b.k_cache if k_cache is None else k_cache),
            "v_cache": W.host_bits(b.v_cache if v_cache is None else v_cache),
            "block_tables": np.ascontiguousarray(b.pool.block_tables), "context_lens": b.pool.context_lens}


def baseline_decode(base, name, b, k_cache=None, v_cache=None):
    if base is None:
        return
    hkv, d, e = b.num_kv_heads, b.head_dim, b.k_cache.element_size()
    ctx = b.pool.context_lens.astype(np.int64)

    def work(units):
        seqs = [u[0] for u in units]
        return float(sum(ctx[s] * hkv * d * e * 2 + 2 * b.num_q_heads * d * b.q.element_size() for s in seqs)) / 1e9, \
            float(len(seqs))
    base.run(name, "decode", decode_arrays(b, k_cache, v_cache), b.scale, b.block_size, work, "GB/s",
             lambda units: f"{len(units)} sequence decodes of the {b.num_seqs} sequences in index order, "
                           f"cycled (float64 oracle, all q-heads)")


def baseline_prefill(base, name, b):
    if base is None:
        return
    cu, ctx = b.cu_seqlens_q, b.pool.context_lens.astype(np.int64)
    g = b.num_q_heads // b.num_kv_heads

    def work(units):
        fl = 0.0
        rows = 0
        for c, _h in units:
            L = int(cu[c + 1] - cu[c])
            prior = int(ctx[c]) - L
            fl += (L * prior + L * (L + 1) // 2) * g * 4 * b.head_dim
            rows += L
        return fl / 1e12, rows / b.num_kv_heads
    arrays = decode_arrays(b)
    arrays["cu_seqlens_q"] = np.asarray(cu, np.int32)
    base.run(name, "prefill", arrays, b.scale, b.block_size, work, "TFLOP/s",
             lambda units: f"{len(units)} (chunk, kv-head) slices of the {len(cu) - 1} chunks x "
                           f"{b.num_kv_heads} kv-heads, chunk by chunk, cycled (float64 oracle, causal)")


# --------------------------------------------------------------------------
# secondary workloads
# --------------------------------------------------------------------------

def balanced_ms(b, bt, cl, steps, warmup):
    """The same decode with the work-balanced kernel (one launch, in-kernel merge)."""
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                           b.max_ctx, partition_size="balanced", algo="mfma")
    return time_region(dec, steps, warmup)


def planned_ms(b, bt, cl, steps, warmup):
    """The same decode in the order of a plan, the plan's launch included
    (one decode call per step here, so nothing amortises it)."""
    plan = pkv.new_decode_plan(b.num_seqs, b.q.device)
    mk = pkv.DecodePlanLaunch(plan, bt, cl, b.max_ctx, b.block_size)
    mk()
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                           b.max_ctx, partition_size="planned", algo="mfma", workspace=plan)

    def run():
        mk()
        dec()
    return time_region(run, steps, warmup)


def fp8_step(device, steps, warmup, bf16_step_ms, partition=0):
    """The headline step over E4M3 caches: per layer, decode with the
    quantising store of the 60 new rows fused in, 28 layers, one graph replay."""
    wl = W.qwen3_decode_fp8(device=device)
    b0 = wl.batches[0]
    bt = torch.as_tensor(b0.pool.block_tables, device=device)
    cl = torch.as_tensor(b0.pool.context_lens, device=device)
    calls, outs = [], []
    plan = mk = None
    if partition == "planned":
        plan = pkv.new_decode_plan(b0.num_seqs, device)
        mk = pkv.DecodePlanLaunch(plan, bt, cl, b0.max_ctx, b0.block_size)
        mk()
    for b in wl.batches:
        out = torch.empty_like(b.q)
        outs.append(out)
        calls.append(pkv.DecodeStoreFp8Launch(out, b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, bt,
                                              cl, b.k_new, b.v_new, b.slot_mapping, b.scale, b.max_ctx,
                                              partition_size=partition, workspace=plan))

    def step():
        if mk is not None:
            mk()
        for c in calls:
            c()
    graph = capture_step(step, outs)
    ms = time_region(graph.replay, steps, warmup)
    per_launch = decode_bytes(b0) + store_bytes(b0)
    dec_ms = time_each_launch(calls, 4)
    return {"ms_per_step": ms, "GBps": per_launch * len(calls) / ms / 1e6,
            "tokens_per_s": b0.num_seqs / (ms * 1e-3), "speedup_vs_bf16_step": bf16_step_ms / ms,
            "decode_avg_launch_us": dec_ms * 1e3, "decode_GBps": per_launch / dec_ms / 1e6,
            "partition": partition, "cache": "E4M3 codes, per-kv-head scales; store fused into decode"}


def secondary(device, steps, warmup, algo, bf16_step_ms, partition=0, base=None):
    res = {"qwen3_fp8": fp8_step(device, steps, warmup, bf16_step_ms, partition)}
    torch.cuda.empty_cache()
    b = W.llama_prefix(device=device).batches[0]
    bt = torch.as_tensor(b.pool.block_tables, device=device)
    cl = torch.as_tensor(b.pool.context_lens, device=device)
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                           b.max_ctx, partition_size=0, algo=algo)
    ms = time_region(dec, steps, warmup)
    ub, lb = decode_bytes(b, unique_blocks=True), decode_bytes(b)
    res["llama_prefix"] = {"ms": ms, "unique_GBps": ub / ms / 1e6, "logical_GBps": lb / ms / 1e6,
                           "pct_hbm_peak_unique": 100 * ub / ms / 1e6 / HBM_PEAK_GBS,
                           "tokens_per_s": b.num_seqs / (ms * 1e-3), "partition": 0,
                           "balanced_ms": balanced_ms(b, bt, cl, steps, warmup),
                           "planned_ms": planned_ms(b, bt, cl, steps, warmup),
                           "shared_prefix_ms": time_region(pkv.SharedPrefixDecodeLaunch(
                               torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl,
                               torch.arange(0, b.num_seqs + 1, 8, dtype=torch.int32, device=device),
                               torch.full((b.num_seqs // 8,), 32 * b.block_size, dtype=torch.int32,
                                          device=device),
                               b.scale, b.max_ctx, 8, 32 * b.block_size), steps, warmup),
                           "paged_read_ms": paged_read_ms(b, device)}
    res["llama_prefix"]["frac_of_paged_read_time"] = res["llama_prefix"]["paged_read_ms"] / ms
    baseline_decode(base, "llama_prefix", b)
    del dec, b
    b = W.long_splitk(device=device).batches[0]
    bt = torch.as_tensor(b.pool.block_tables, device=device)
    cl = torch.as_tensor(b.pool.context_lens, device=device)
    auto_part = pkv.decode_auto_partition(b.num_seqs, b.num_kv_heads, b.max_ctx)
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                           b.max_ctx, partition_size="auto", algo=algo)
    ms = time_region(dec, steps, warmup)
    split_ms = {}
    for part in (512, 1024, 2048):
        d = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale,
                             b.max_ctx, partition_size=part, algo=algo)
        split_ms[str(part)] = time_region(d, steps, warmup)
        del d
    by = decode_bytes(b)
    res["long_splitk"] = {"ms": ms, "GBps": by / ms / 1e6, "pct_hbm_peak": 100 * by / ms / 1e6 / HBM_PEAK_GBS,
                          "tokens_per_s": b.num_seqs / (ms * 1e-3), "partition": "auto",
                          "auto_choice": "balanced" if auto_part == pkv.PARTITION_BALANCED else auto_part,
                          "splitk_ms": split_ms,
                          "balanced_ms": balanced_ms(b, bt, cl, steps, warmup),
                          "planned_ms": planned_ms(b, bt, cl, steps, warmup),
                          "paged_read_ms": paged_read_ms(b, device)}
    res["long_splitk"]["frac_of_paged_read_time"] = res["long_splitk"]["paged_read_ms"] / ms
    baseline_decode(base, "long_splitk", b)
    del dec, b
    wl = W.mixed(device=device)
    pre, db = wl.prefill, wl.batches[0]
    store = pkv.StoreLaunch(pre.k_new, pre.v_new, pre.k_cache, pre.v_cache, pre.slot_mapping)
    prefill = pkv.PrefillLaunch(torch.empty_like(pre.q), pre.q, pre.k_cache, pre.v_cache,
                                torch.as_tensor(pre.pool.block_tables, device=device),
                                torch.as_tensor(pre.cu_seqlens_q, device=device),
                                torch.as_tensor(pre.pool.context_lens, device=device), pre.scale,
                                int(np.diff(pre.cu_seqlens_q).max()), pre.max_ctx, causal=True)
    dec = pkv.DecodeLaunch(torch.empty_like(db.q), db.q, db.k_cache, db.v_cache,
                           torch.as_tensor(db.pool.block_tables, device=device),
                           torch.as_tensor(db.pool.context_lens, device=device), db.scale,
                           db.max_ctx, partition_size=0, algo=algo)
    t_store = time_region(store, steps, warmup)
    t_pre = time_region_settled(prefill, steps, warmup)
    t_dec = time_region(dec, steps, warmup)

    def serial():
        store()
        prefill()
        dec()
    # the same batch with the prefill chunks and the decode sequences on two
    # streams (default priority), both after the store
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()

    def two_streams():
        cur = torch.cuda.current_stream()
        store()
        sa.wait_stream(cur)
        sb.wait_stream(cur)
        with torch.cuda.stream(sa):
            prefill()
        with torch.cuda.stream(sb):
            dec()
        cur.wait_stream(sa)
        cur.wait_stream(sb)
    t_serial = time_region(serial, steps, warmup)
    t_two = time_region(two_streams, steps, warmup)
    t_dec_bal = balanced_ms(db, torch.as_tensor(db.pool.block_tables, device=device),
                            torch.as_tensor(db.pool.context_lens, device=device), steps, warmup)
    t_dec_plan = planned_ms(db, torch.as_tensor(db.pool.block_tables, device=device),
                            torch.as_tensor(db.pool.context_lens, device=device), steps, warmup)
    t_store_cold = cold_store_ms(store, device)
    fl = prefill_flops(pre)
    res["mixed"] = {"store_ms": t_store, "store_GBps": store_bytes(pre) / t_store / 1e6,
                    "store_cold_ms": t_store_cold, "store_cold_GBps": store_bytes(pre) / t_store_cold / 1e6,
                    "prefill_ms": t_pre, "prefill_TFLOPs": fl / t_pre / 1e9,
                    "prefill_mfma_util_pct": 100 * fl / t_pre / 1e9 / BF16_MFMA_PEAK_TFLOPS,
                    "decode_ms": t_dec, "decode_GBps": decode_bytes(db) / t_dec / 1e6,
                    "decode_balanced_ms": t_dec_bal, "decode_planned_ms": t_dec_plan,
                    "tokens_per_s": 4224 / ((t_store + t_pre + t_dec) * 1e-3),
                    "prefill_tokens_per_s": 4096 / (t_pre * 1e-3),
                    "serial_step_ms": t_serial, "two_stream_step_ms": t_two,
                    "tokens_per_s_two_streams": 4224 / (t_two * 1e-3),
                    "decode_paged_read_ms": paged_read_ms(db, device)}
    res["mixed"]["decode_frac_of_paged_read_time"] = res["mixed"]["decode_paged_read_ms"] / t_dec
    baseline_decode(base, "mixed_decode", db)
    baseline_prefill(base, "mixed_prefill", pre)
    del store, prefill, dec, wl, pre, db
    torch.cuda.empty_cache()
    # the same chunked prefill over E4M3 caches (its own draws, same lengths and tables)
    pf = W.mixed_prefill_fp8(device=device)
    pkv.kv_cache_store_fp8(pf.k_new, pf.v_new, pf.k_cache, pf.v_cache, pf.slot_mapping, pf.k_scale,
                           pf.v_scale)
    prefill8 = pkv.PrefillFp8Launch(torch.empty_like(pf.q), pf.q, pf.k_cache, pf.v_cache, pf.k_scale,
                                    pf.v_scale, torch.as_tensor(pf.pool.block_tables, device=device),
                                    torch.as_tensor(pf.cu_seqlens_q, device=device),
                                    torch.as_tensor(pf.pool.context_lens, device=device), pf.scale,
                                    int(np.diff(pf.cu_seqlens_q).max()), pf.max_ctx, causal=True)
    t_pre8 = time_region_settled(prefill8, steps, warmup)
    fl8 = prefill_flops(pf)
    res["mixed"].update({"prefill_fp8_ms": t_pre8, "prefill_fp8_TFLOPs": fl8 / t_pre8 / 1e9,
                         "prefill_fp8_mfma_util_pct": 100 * fl8 / t_pre8 / 1e9 / BF16_MFMA_PEAK_TFLOPS})
    del prefill8, pf
    torch.cuda.empty_cache()
    # verification of drafted tokens: 128 seqs x 4 causal rows, one chunk call
    sv = W.spec_verify(device=device).prefill
    pkv.kv_cache_store(sv.k_new, sv.v_new, sv.k_cache, sv.v_cache, sv.slot_mapping)
    verify = pkv.PrefillLaunch(torch.empty_like(sv.q), sv.q, sv.k_cache, sv.v_cache,
                               torch.as_tensor(sv.pool.block_tables, device=device),
                               torch.as_tensor(sv.cu_seqlens_q, device=device),
                               torch.as_tensor(sv.pool.context_lens, device=device), sv.scale,
                               4, sv.max_ctx, causal=True)
    ms = time_region(verify, steps, warmup)
    by = decode_bytes(sv)
    res["spec_verify"] = {"ms": ms, "GBps": by / ms / 1e6, "pct_hbm_peak": 100 * by / ms / 1e6 / HBM_PEAK_GBS,
                          "rows_per_s": sv.q.shape[0] / (ms * 1e-3), "rows_per_seq": 4,
                          "paged_read_ms": paged_read_ms(sv, device)}
    res["spec_verify"]["frac_of_paged_read_time"] = res["spec_verify"]["paged_read_ms"] / ms
    baseline_prefill(base, "spec_verify", sv)
    return res


# --------------------------------------------------------------------------
# counter passes
# --------------------------------------------------------------------------

CALIB_TOKENS = 65536              # calibration store: 65536 rows of 8 x 128 bf16 (2 KiB) each


def calib_bytes():
    """Bytes the calibration store reads and writes (K and V rows; slots read)."""
    row = 8 * 128 * 2
    return 2 * CALIB_TOKENS * row + 4 * CALIB_TOKENS, 2 * CALIB_TOKENS * row


def _calibration_store(device):
    """A plain copy of known size: kv_cache_store of 65536 new rows into a pool
    of exactly as many slots (identity slots), 256 MiB read and written."""
    k = torch.empty((CALIB_TOKENS, 8, 128), dtype=torch.bfloat16, device=device).normal_()
    v = torch.empty_like(k).normal_()
    kc = torch.empty((CALIB_TOKENS // 16, 16, 8, 128), dtype=torch.bfloat16, device=device)
    vc = torch.empty_like(kc)
    slots = torch.arange(CALIB_TOKENS, dtype=torch.int32, device=device)
    torch.cuda.synchronize()
    pkv.kv_cache_store(k, v, kc, vc, slots)
    torch.cuda.synchronize()


def split_partial_bytes(b, part):
    """Bytes of split-K partials written and read back: (max, sum, D outputs)
    in fp32 per (sequence, q-head, partition) of sequences with more than one
    partition."""
    if not part:
        return 0.0
    parts = -(-b.pool.context_lens.astype(np.int64) // part)
    n = int(parts[parts > 1].sum())
    return float(2 * n * b.num_q_heads * (b.head_dim + 2) * 4)


def pmc_pass(device, layers, partition):
    """Every bandwidth workload's launches, in a fixed order, for rocprofv3
    --pmc FETCH_SIZE / WRITE_SIZE runs, then a plain copy of known size (the
    calibration). Prints the manifest the summary walks: for each segment,
    this library's dispatches in launch order and the algorithmic bytes of
    one call. Repeated launches of a batch read more bytes than the 256 MB
    last-level cache holds, except where noted."""
    segs = []

    def seg(name, calls, per_call, algo_bytes, desc, report=True, extra=0.0):
        segs.append({"name": name, "calls": calls, "dispatches_per_call": per_call,
                     "algorithmic_bytes_per_call": float(algo_bytes), "implementation_bytes_per_call": float(extra),
                     "desc": desc, "report": report})

    wl, lyr, plan_launch = build_headline(device, layers, partition, "auto")
    b0 = wl.batches[0]
    torch.cuda.synchronize()
    if plan_launch is not None:
        plan_launch()
        # build_headline made the plan once already
        seg("qwen3_plan", 2, 1, 0, "decode_plan_kernel", report=False)
    for ly in lyr:
        ly.fused()
    torch.cuda.synchronize()
    seg("qwen3_decode", len(lyr), 1, decode_bytes(b0) + store_bytes(b0),
        f"decode_mfma_kernel, partition {partition}, store fused; {len(lyr)} distinct layers")
    del wl, lyr, plan_launch
    torch.cuda.empty_cache()

    wl = W.qwen3_decode_fp8(device=device, layers=layers)
    b8 = wl.batches[0]
    bt = torch.as_tensor(b8.pool.block_tables, device=device)
    cl = torch.as_tensor(b8.pool.context_lens, device=device)
    plan = pkv.new_decode_plan(b8.num_seqs, device)
    calls = [pkv.DecodeStoreFp8Launch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, b.k_scale, b.v_scale, bt, cl,
                                      b.k_new, b.v_new, b.slot_mapping, b.scale, b.max_ctx,
                                      partition_size="planned", workspace=plan) for b in wl.batches]
    torch.cuda.synchronize()
    pkv.decode_plan(plan, bt, cl, b8.max_ctx, b8.block_size)
    seg("qwen3_fp8_plan", 1, 1, 0, "decode_plan_kernel", report=False)
    for c in calls:
        c()
    torch.cuda.synchronize()
    seg("qwen3_fp8_decode", len(calls), 1, decode_bytes(b8) + store_bytes(b8),
        f"decode_mfma_kernel over E4M3 caches, planned, store fused; {len(calls)} distinct layers")
    del wl, calls, plan, bt, cl
    torch.cuda.empty_cache()

    b = W.llama_prefix(device=device).batches[0]
    bt = torch.as_tensor(b.pool.block_tables, device=device)
    cl = torch.as_tensor(b.pool.context_lens, device=device)
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale, b.max_ctx,
                           partition_size=0)
    shared = pkv.SharedPrefixDecodeLaunch(
        torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl,
        torch.arange(0, b.num_seqs + 1, 8, dtype=torch.int32, device=device),
        torch.full((b.num_seqs // 8,), 32 * b.block_size, dtype=torch.int32, device=device), b.scale, b.max_ctx, 8,
        32 * b.block_size)
    torch.cuda.synchronize()
    for _ in range(3):
        dec()
    torch.cuda.synchronize()
    ub = decode_bytes(b, unique_blocks=True)
    seg("llama_prefix_decode", 3, 1, ub, "decode_mfma_kernel, one pass; algorithmic bytes count shared blocks once "
        f"(logical bytes {decode_bytes(b):.4g})")
    for _ in range(3):
        shared()
    torch.cuda.synchronize()
    sp_extra = float(2 * b.num_seqs * b.num_q_heads * (b.head_dim + 2) * 4 + 8 * b.num_seqs)
    seg("llama_prefix_shared", 3, 2, ub, "prefill_kernel (prefix partials) + decode_mfma_kernel (own tokens, merged)",
        extra=sp_extra)
    del b, bt, cl, dec, shared
    torch.cuda.empty_cache()

    b = W.long_splitk(device=device).batches[0]
    bt = torch.as_tensor(b.pool.block_tables, device=device)
    cl = torch.as_tensor(b.pool.context_lens, device=device)
    part = pkv.decode_auto_partition(b.num_seqs, b.num_kv_heads, b.max_ctx)
    dec = pkv.DecodeLaunch(torch.empty_like(b.q), b.q, b.k_cache, b.v_cache, bt, cl, b.scale, b.max_ctx,
                           partition_size="auto")
    torch.cuda.synchronize()
    seg("long_workspace_init", 1, 1, 0, "zero_ints_kernel (the new workspace's counters)", report=False)
    for _ in range(3):
        dec()
    torch.cuda.synchronize()
    if part == pkv.PARTITION_BALANCED:
        seg("long_splitk_auto", 3, 1, decode_bytes(b), "decode_balanced_kernel (auto's choice): equal tile shares "
            "per wave, split items merged in the same launch (their pieces not counted as extra)")
    else:
        seg("long_splitk_auto", 3, 1, decode_bytes(b), f"decode_mfma_kernel, split-K at {part} tokens (auto), "
            "merged in the same launch", extra=split_partial_bytes(b, part))
    del b, bt, cl, dec
    torch.cuda.empty_cache()

    wl = W.mixed(device=device)
    pre, db = wl.prefill, wl.batches[0]
    pkv.kv_cache_store(pre.k_new, pre.v_new, pre.k_cache, pre.v_cache, pre.slot_mapping)
    torch.cuda.synchronize()
    seg("mixed_store", 1, 1, store_bytes(pre), "kv_store_kernel, 4224 new rows")
    prefill = pkv.PrefillLaunch(torch.empty_like(pre.q), pre.q, pre.k_cache, pre.v_cache,
                                torch.as_tensor(pre.pool.block_tables, device=device),
                                torch.as_tensor(pre.cu_seqlens_q, device=device),
                                torch.as_tensor(pre.pool.context_lens, device=device), pre.scale, 512, pre.max_ctx)
    dec = pkv.DecodeLaunch(torch.empty_like(db.q), db.q, db.k_cache, db.v_cache,
                           torch.as_tensor(db.pool.block_tables, device=device),
                           torch.as_tensor(db.pool.context_lens, device=device), db.scale, db.max_ctx)
    torch.cuda.synchronize()
    for _ in range(2):
        prefill()
    torch.cuda.synchronize()
    seg("mixed_prefill", 2, 1, decode_bytes(pre), "prefill_kernel, 8 chunks x 512 causal rows (algorithmic bytes: "
        "each chunk's K/V once, q, out; the kernel re-reads them per q-tile, mostly from L2)")
    for _ in range(3):
        dec()
    torch.cuda.synchronize()
    seg("mixed_decode", 3, 1, decode_bytes(db), "decode_mfma_kernel, one pass, 128 sequences")
    del wl, pre, db, prefill, dec
    torch.cuda.empty_cache()

    sv = W.spec_verify(device=device).prefill
    pkv.kv_cache_store(sv.k_new, sv.v_new, sv.k_cache, sv.v_cache, sv.slot_mapping)
    torch.cuda.synchronize()
    seg("spec_verify_store", 1, 1, store_bytes(sv), "kv_store_kernel, 512 new rows", report=False)
    verify = pkv.PrefillLaunch(torch.empty_like(sv.q), sv.q, sv.k_cache, sv.v_cache,
                               torch.as_tensor(sv.pool.block_tables, device=device),
                               torch.as_tensor(sv.cu_seqlens_q, device=device),
                               torch.as_tensor(sv.pool.context_lens, device=device), sv.scale, 4, sv.max_ctx)
    torch.cuda.synchronize()
    for _ in range(3):
        verify()
    torch.cuda.synchronize()
    seg("spec_verify", 3, 1, decode_bytes(sv), "prefill_kernel, 128 sequences x 4 causal rows")
    del sv, verify
    torch.cuda.empty_cache()

    _calibration_store(device)
    seg("calibration", 1, 1, 0, "kv_store_kernel, 65536 rows of 2 KiB, identity slots", report=False)
    print(json.dumps({"pmc_pass": "done", "segments": segs, "calibration_read_write_bytes": calib_bytes(),
                      "decode_source_hash": decode_source_hash()}))


PREFILL_COUNTERS = ["SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_VALU",
                    "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_SALU",
                    "GRBM_GUI_ACTIVE"]


def prefill_pmc_pass(device, launches=3):
    """The mixed workload's chunked prefill (8 x 512 causal rows after 0..8K
    cached tokens), launched a few times after its store, for counters."""
    pre = W.mixed(device=device).prefill
    pkv.kv_cache_store(pre.k_new, pre.v_new, pre.k_cache, pre.v_cache, pre.slot_mapping)
    call = pkv.PrefillLaunch(torch.empty_like(pre.q), pre.q, pre.k_cache, pre.v_cache,
                             torch.as_tensor(pre.pool.block_tables, device=device),
                             torch.as_tensor(pre.cu_seqlens_q, device=device),
                             torch.as_tensor(pre.pool.context_lens, device=device), pre.scale,
                             int(np.diff(pre.cu_seqlens_q).max()), pre.max_ctx, causal=True)
    torch.cuda.synchronize()
    for _ in range(launches):
        call()
    torch.cuda.synchronize()
    print(json.dumps({"prefill_pmc_pass": "done", "launches": launches,
                      "flops_per_launch": prefill_flops(pre)}))


def summarize_prefill_pmc(counter_csv, trace_csv, out_md, command):
    """Markdown summary of a --prefill-pmc-pass run under rocprofv3 --pmc
    (PREFILL_COUNTERS) with --kernel-trace: counter means over the prefill
    dispatches, their durations, and the matrix-core busy fraction."""
    vals = {}
    for r in csv.DictReader(open(counter_csv)):
        if "prefill_kernel" in r["Kernel_Name"]:
            vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    dur = [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
           for r in csv.DictReader(open(trace_csv)) if "prefill_kernel" in r["Kernel_Name"]]
    mean = {k: float(np.mean(v)) for k, v in vals.items()}
    us = float(np.median(dur))
    pre = W.mixed(device="cpu").prefill
    fl = prefill_flops(pre)
    simd_cycles = us * 1e-6 * CLOCK_HZ * NUM_SIMDS
    busy = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / simd_cycles
    # GRBM_GUI_ACTIVE sums the busy cycles of the 8 XCDs at the running clock
    clock = mean["GRBM_GUI_ACTIVE"] / 8 / (us * 1e-6)
    busy_at_clock = mean["SQ_VALU_MFMA_BUSY_CYCLES"] / (mean["GRBM_GUI_ACTIVE"] * NUM_SIMDS // 8)
    valu = mean["SQ_INSTS_VALU"] - mean["SQ_INSTS_MFMA"]
    lines = [
        "# Chunked prefill on the matrix cores: counters, mixed workload", "",
        "Kernel: `prefill_kernel<4>` (bf16, head_dim 128, 32 q / 8 kv heads), the mixed workload's",
        "prefill part: 8 chunks of 512 query rows, causal, after 0..8K cached tokens per chunk",
        "(the chunk's own rows stored first), block_size 16.", "",
        "Commands (from the repository root on one MI355X):", "", "```", command, "```", "",
        "| quantity | value |", "|---|---|",
        f"| dispatches | {len(dur)} |",
        f"| duration (median, kernel trace) | {us:.1f} us |",
        f"| useful FLOPs (QK^T and PV over visible keys) | {fl:.4g} |",
        f"| useful rate | {fl / (us * 1e-6) / 1e12:.0f} TFLOP/s = {100 * fl / (us * 1e-6) / 1e12 / BF16_MFMA_PEAK_TFLOPS:.1f}% of 2.5 PFLOP/s |",
        f"| SQ_VALU_MFMA_BUSY_CYCLES / (duration x {NUM_SIMDS} SIMDs x {CLOCK_HZ / 1e9:.1f} GHz) | {100 * busy:.1f}% |",
        f"| engine clock during the kernel, GRBM_GUI_ACTIVE / 8 XCDs / duration | {clock / 1e9:.2f} GHz |",
        f"| SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x {NUM_SIMDS // 8} SIMDs per XCD) | {100 * busy_at_clock:.1f}% |",
        f"| MFMA instructions | {mean['SQ_INSTS_MFMA']:.4g} |",
        f"| other vector ALU instructions | {valu:.4g} ({valu / mean['SQ_INSTS_MFMA']:.2f} per MFMA) |",
        f"| of which transcendental (exp2) | {mean['SQ_INSTS_VALU_TRANS_F32']:.4g} |",
        f"| scalar ALU instructions | {mean['SQ_INSTS_SALU']:.4g} |",
        f"| LDS instructions | {mean['SQ_INSTS_LDS']:.4g} |",
        f"| LDS bank-conflict cycles | {mean['SQ_LDS_BANK_CONFLICT']:.4g} |",
        f"| GRBM_GUI_ACTIVE | {mean['GRBM_GUI_ACTIVE']:.4g} |", "",
        "The busy fraction counts the row-sum MFMA (P times a ones column) too, which the useful",
        "FLOPs leave out: two of every 34 MFMAs of a full 32-key step. Under this load the engine",
        "runs below its 2.4 GHz peak clock, so the fraction of the cycles it actually ran is the",
        "higher of the two busy figures; the useful rate is against the 2.4 GHz vendor peak.",
    ]
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def summarize_counters(kernel, out_md, title, command, *csvs):
    """Means per dispatch of every counter that rocprofv3 --pmc runs recorded
    for kernels whose name contains `kernel`, and each wave-cycle counter as a
    share of SQ_WAVE_CYCLES."""
    vals = {}
    for path in csvs:
        for r in csv.DictReader(open(path)):
            if kernel in r["Kernel_Name"]:
                vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    mean = {k: float(np.mean(v)) for k, v in vals.items()}
    lines = [f"# {title}", "", "Commands (on one MI355X; R is the repository root):", "", "```", command, "```", "",
             "| counter | mean per dispatch | share of SQ_WAVE_CYCLES |", "|---|---|---|"]
    wc = mean.get("SQ_WAVE_CYCLES")
    for k in sorted(mean):
        share = f"{100 * mean[k] / wc:.1f}%" if wc and (k.startswith("SQ_WAIT") or k.startswith("SQ_ACTIVE_INST")) else ""
        lines.append(f"| {k} | {mean[k]:.4g} | {share} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


def summarize_pmc(fetch_csv, write_csv, manifest, command):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of every segment of a
    --pmc-pass run, each scaled by (known bytes / counter reading) of the
    calibration copy that ends the pass. Writes profiles/decode_qwen3_traffic.*
    (the headline decode, read back by the benchmark while the decode
    source is unchanged) and profiles/hbm_traffic_all_workloads.md."""
    man = None
    for line in open(manifest):
        line = line.strip()
        if line.startswith("{") and '"pmc_pass"' in line:
            man = json.loads(line)
    if man is None:
        raise RuntimeError(f"{manifest}: no pmc-pass manifest line")

    def ours(path, counter):
        rows = [r for r in csv.DictReader(open(path)) if r.get("Counter_Name") == counter and "pkv::" in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Dispatch_Id"]))
        return [(r["Kernel_Name"].split("(")[0].replace("void ", ""), float(r["Counter_Value"]) * 1024.0)
                for r in rows]
    fetch, write = ours(fetch_csv, "FETCH_SIZE"), ours(write_csv, "WRITE_SIZE")
    need = sum(sg["calls"] * sg["dispatches_per_call"] for sg in man["segments"])
    if len(fetch) != need or len(write) != need:
        raise RuntimeError(f"expected {need} dispatches of this library, found {len(fetch)} / {len(write)}")
    read_known, write_known = man["calibration_read_write_bytes"]
    fr, fw = read_known / fetch[-1][1], write_known / write[-1][1]
    rows, i = [], 0
    for sg in man["segments"]:
        n = sg["calls"] * sg["dispatches_per_call"]
        f_seg, w_seg = fetch[i:i + n], write[i:i + n]
        i += n
        if not sg["report"]:
            continue
        kernels = sorted(set(k for k, _ in f_seg))
        f_call = sum(v for _, v in f_seg) * fr / sg["calls"]
        w_call = sum(v for _, v in w_seg) * fw / sg["calls"]
        rows.append(dict(sg, kernels=kernels, fetch=f_call, write=w_call, fetch_raw=sum(v for _, v in f_seg) / sg["calls"],
                         write_raw=sum(v for _, v in w_seg) / sg["calls"]))
    head = next(r for r in rows if r["name"] == "qwen3_decode")
    out = {
        "kernel": "decode_mfma_kernel (planned single pass, store of the 60 new rows fused), qwen3-shaped layer",
        "decode_source_hash": man["decode_source_hash"],
        "fetch_bytes_raw_per_launch": head["fetch_raw"], "write_bytes_raw_per_launch": head["write_raw"],
        "calibration": {"kernel": "kv_store_kernel, 65536 rows of 2 KiB, identity slots", "read_bytes": read_known,
                        "write_bytes": write_known, "fetch_raw": fetch[-1][1], "write_raw": write[-1][1],
                        "fetch_factor": fr, "write_factor": fw},
        "hbm_bytes_per_launch": head["fetch"] + head["write"],
        "algorithmic_bytes_per_launch": head["algorithmic_bytes_per_call"],
        "launches_averaged": head["calls"],
        "command": command,
    }
    if out["decode_source_hash"] != decode_source_hash():
        raise RuntimeError("the decode sources changed since the counter pass")
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    with open(TRAFFIC_FILE[:-5] + ".md", "w") as f:
        f.write(traffic_markdown(out))
    lines = ["# HBM traffic of every bandwidth workload (rocprofv3 counters)", "",
             "Counters FETCH_SIZE and WRITE_SIZE per dispatch of this library's kernels, in two passes over the same",
             "launches, each scaled by the reading of a plain copy of known size that ends the pass",
             f"(fetch factor {fr:.3f}, write factor {fw:.3f}); per call (a call of the shared-prefix decode is two",
             "dispatches). Algorithmic bytes are those the benchmark divides by time; implementation bytes are what",
             "the method does not need but this implementation moves on purpose (split-K and shared-prefix partials,",
             "written and read back).", "", "Commands (from the repository root on one MI355X):", "", "```", command,
             "```", "",
             "| workload | kernels | calls | HBM read / call | HBM write / call | algorithmic / call | implementation extra | traffic / (algorithmic + extra) |",
             "|---|---|---|---|---|---|---|---|"]
    for r in rows:
        tot = r["fetch"] + r["write"]
        base = r["algorithmic_bytes_per_call"] + r["implementation_bytes_per_call"]
        lines.append(f"| {r['name']}: {r['desc']} | {', '.join('`' + k + '`' for k in r['kernels'])} | {r['calls']} | "
                     f"{r['fetch']:,.0f} | {r['write']:,.0f} | {r['algorithmic_bytes_per_call']:,.0f} | "
                     f"{r['implementation_bytes_per_call']:,.0f} | {tot / base:.3f} |")
    lines += ["", "Repeated calls of one batch (every workload but the two 28-layer steps) read the same bytes again;",
              "every such batch is larger than the 256 MB last-level cache except the store, whose line is therefore",
              "a warm figure. The shared-prefix row's algorithmic bytes count each shared block once, as the",
              "prefix-shared decode's line in the benchmark does."]
    md = os.path.join(os.path.dirname(TRAFFIC_FILE), "hbm_traffic_all_workloads.md")
    with open(md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(json.dumps(out))
    print(f"wrote {md}")


def traffic_markdown(t):
    c = t["calibration"]
    return f"""# HBM traffic of the decode kernel, Qwen3-shaped layer

Kernel: `decode_mfma_kernel<128, 4>` (single pass with items in the order of the step's plan, the
store of the 60 new K/V rows fused into it, as the benchmark's step launches it), one layer of the Qwen3-0.6B-shaped decode step
(60 sequences, contexts U{{64..1024}}, 16 q / 8 kv heads, head_dim 128, block_size 16, bf16),
{t['launches_averaged']} launches on distinct layer caches (4.7 GB in total, so the 256 MB last-level cache
cannot hold them).

Commands (on one MI355X; R is the repository root):

```
{t['command']}
```

Calibration: the last dispatch of each pass is a plain copy of known size, a `kv_store_kernel`
moving 65536 rows of 2 KiB with identity slots ({c['read_bytes']:,} bytes read including the slot
array, {c['write_bytes']:,} bytes written). The counters read {int(c['fetch_raw']):,} bytes fetched
(factor {c['fetch_factor']:.3f}) and {int(c['write_raw']):,} bytes written (factor {c['write_factor']:.3f}) for it;
the decode readings are scaled by the same factors.

| quantity | bytes per launch |
|---|---|
| FETCH_SIZE, raw (mean of {t['launches_averaged']} launches) | {int(t['fetch_bytes_raw_per_launch']):,} |
| WRITE_SIZE, raw (mean of {t['launches_averaged']} launches) | {int(t['write_bytes_raw_per_launch']):,} |
| HBM bytes, calibrated | {int(t['hbm_bytes_per_launch']):,} |
| algorithmic bytes (K/V rows in context, q, out, table entries, lengths, the fused store's rows and slots) | {int(t['algorithmic_bytes_per_launch']):,} |
| traffic / algorithmic | {t['hbm_bytes_per_launch'] / t['algorithmic_bytes_per_launch']:.3f} |

The written bytes are the output (60 x 16 x 128 bf16 = 245,760) plus the 60 stored K and V rows
(245,760). Machine-readable values: `decode_qwen3_traffic.json` (bench.py reports them as
`traffic` only while the decode kernel's source hash, {t['decode_source_hash']}, matches).
"""


def summarize_trace(stats_csv, trace_csv, out_md, command):
    """Short markdown summary of a rocprofv3 --kernel-trace --stats run."""
    stats = list(csv.DictReader(open(stats_csv)))
    lines = [f"# Kernel trace: {os.path.basename(out_md)[:-3]}", "",
             "Command (from the repository root on one MI355X):", "", "```", command, "```", "",
             "## rocprofv3 --stats (all kernels of the run)", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in stats[:14]:
        name = r["Name"].split("(")[0].replace("void ", "")[:70]
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.2f} |")
    groups = {}
    for r in csv.DictReader(open(trace_csv)):
        name = r["Kernel_Name"]
        if "pkv::" not in name:
            continue
        key = (name.split("(")[0].replace("void ", ""), r["Grid_Size_X"], r["Grid_Size_Y"], r["Grid_Size_Z"])
        groups.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines += ["", "## This library's kernels by launch shape (from the kernel trace)", "",
              "| kernel | grid (threads x, y, z) | launches | median us | mean us |", "|---|---|---|---|---|"]
    for (name, gx, gy, gz), v in groups.items():
        v.sort()
        lines.append(f"| `{name}` | {gx}, {gy}, {gz} | {len(v)} | {v[len(v) // 2]:.2f} | {sum(v) / len(v):.2f} |")
    with open(out_md, "w") as f:
        f.write("\n".join(lines) + "\n")
    print(f"wrote {out_md}")


# --------------------------------------------------------------------------

def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--partition", type=parse_partition, default="planned",
                    help="decode partition size for the step: 'planned' (items in the order of a plan "
                         "made once per step), 0 (one pass, items ranked in the kernel), a multiple of "
                         "16 (split-K) or 'balanced'")
    ap.add_argument("--algo", default="auto", choices=sorted(pkv.DECODE_ALGOS))
    ap.add_argument("--layers", type=int, default=28)
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of graph replay")
    ap.add_argument("--unfused", action="store_true",
                    help="store and decode as two launches per layer instead of the fused call")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=3.0,
                    help="seconds of wall time the oracle baseline spends on each workload")
    ap.add_argument("--pmc-pass", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "PASS_STDOUT", "COMMAND"))
    ap.add_argument("--summarize-trace", nargs=4, metavar=("STATS_CSV", "TRACE_CSV", "OUT_MD", "COMMAND"))
    ap.add_argument("--prefill-pmc-pass", action="store_true")
    ap.add_argument("--summarize-prefill-pmc", nargs=4, metavar=("COUNTER_CSV", "TRACE_CSV", "OUT_MD", "COMMAND"))
    ap.add_argument("--summarize-counters", nargs="+", metavar="ARG",
                    help="KERNEL OUT_MD TITLE COMMAND CSV [CSV ...]: means of the counters of one kernel")
    args = ap.parse_args()

    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc)
        return
    if args.summarize_trace:
        summarize_trace(*args.summarize_trace)
        return
    if args.summarize_prefill_pmc:
        summarize_prefill_pmc(*args.summarize_prefill_pmc)
        return
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(decode would shard by sequence or kv-head with no exchange)", file=sys.stderr)
        sys.exit(2)
    # the oracle baseline's worker processes start before anything touches the GPU
    base = None if args.no_cpu_baseline else OracleBaseline(args.cpu_budget)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    device = torch.device("cuda:0")
    torch.cuda.set_device(device)
    if args.pmc_pass:
        pmc_pass(device, args.layers, args.partition)
        return
    if args.prefill_pmc_pass:
        prefill_pmc_pass(device)
        return

    log("generating the qwen3-shaped decode workload on the GPU")
    wl, lyr, plan_launch = build_headline(device, args.layers, args.partition, args.algo)
    b0 = wl.batches[0]
    step_bytes = (decode_bytes(b0) + store_bytes(b0)) * len(lyr)

    def make_plan():
        if plan_launch is not None:
            plan_launch()

    if args.unfused:
        def step():
            make_plan()
            for ly in lyr:
                ly.store()
                ly.decode()
    else:
        def step():
            make_plan()
            for ly in lyr:
                ly.fused()

    if args.eager:
        run = step
    else:
        log("capturing the step in a HIP graph; checking replays against the eager step")
        graph = capture_step(step, [ly.out for ly in lyr])
        run = graph.replay
    log(f"timing {args.steps} steps ({len(lyr)} layers each) after {args.warmup} warmup")
    ms = time_region(run, args.steps, args.warmup)
    value = step_bytes / (ms * 1e-3) / 1e9
    per_step = sorted(time_each_step(run, args.steps))

    # dominant kernel: decode (fused with the store unless --unfused), one launch per layer
    dec_bytes = decode_bytes(b0) + (0.0 if args.unfused else store_bytes(b0))
    dec_ms = time_each_launch([ly.decode if args.unfused else ly.fused for ly in lyr], 4)
    store_ms = time_each_launch([ly.store for ly in lyr], 2)
    plan_us = time_each_launch([plan_launch], 20) * 1e3 if plan_launch is not None else None
    # the E4M3 layer moves the same rows with one byte per cache element
    kv_elems = float(b0.pool.context_lens.astype(np.int64).sum()) * b0.num_kv_heads * b0.head_dim
    stored = float(int((b0.slot_mapping >= 0).sum().item())) * b0.num_kv_heads * b0.head_dim
    fp8_bytes = decode_bytes(b0) + store_bytes(b0) - 2 * kv_elems - 2 * stored
    ceiling = read_ceiling(device, dec_bytes, len(lyr), fp8_bytes)
    ceiling["paged_read"] = paged_read_ceiling(device, wl.batches)
    achieved = dec_bytes / (dec_ms * 1e-3) / 1e9

    # parity sample of layer 0's output against the oracle
    import oracle
    seqs = [0, 17, 33, 59]
    okc, ovc = oracle.kv_cache_store(W.host_bits(b0.k_new), W.host_bits(b0.v_new),
                                     W.host_bits(b0.k_cache), W.host_bits(b0.v_cache),
                                     W.host_bits(b0.slot_mapping), b0.block_size)
    run()
    torch.cuda.synchronize()
    want = oracle.paged_attention_decode(W.host_bits(b0.q)[seqs], okc, ovc,
                                         b0.pool.block_tables[seqs], b0.pool.context_lens[seqs],
                                         b0.scale, b0.block_size)
    got = lyr[0].out.float().cpu().double().numpy()[seqs]
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
        "ms_per_step_median_min_max": [round(float(np.median(per_step)), 4), round(per_step[0], 4),
                                       round(per_step[-1], 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_decode", "num_seqs": 60, "context_lens": "U{64..1024}",
                   "num_q_heads": 16, "num_kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "layers": len(lyr), "partition_size": args.partition, "algo": args.algo,
                   "step": (("decode_plan once, then " if plan_launch is not None else "") +
                            ("per layer: kv_cache_store of 60 new rows, then paged_attention_decode"
                             if args.unfused else
                             "per layer: paged_attention_decode_store (store of 60 new rows fused)")),
                   "launch": "eager" if args.eager else "hip graph replay",
                   "parallelism": "single GPU"},
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(b0.num_seqs / (ms * 1e-3), 1),
        "hbm_read_ceiling": ceiling,
        "roofline": {"bound": "hbm",
                     "kernel": "decode_mfma_kernel (one layer per launch%s)" % (
                         "" if args.unfused else ", store fused"),
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": load_traffic(dec_bytes),
                     "avg_launch_us": round(dec_ms * 1e3, 2),
                     "algorithmic_bytes_per_launch": dec_bytes,
                     "frac_of_read_ceiling_same_bytes": round(achieved / ceiling["GBps_layer_bytes"], 4),
                     "frac_of_paged_read_time": round(ceiling["paged_read"]["paged_read_us"] / (dec_ms * 1e3), 4)},
        "store_avg_launch_us": round(store_ms * 1e3, 2),
        "plan_avg_launch_us": None if plan_us is None else round(plan_us, 2),
        "parity_sample_max_abs_err": parity_err,
    }
    if base is not None:
        log("oracle baseline on the host: the headline's layer 0")
        baseline_decode(base, "qwen3_decode", b0)
    if not args.no_secondary:
        del lyr, wl
        if not args.eager:
            del graph, run
        torch.cuda.empty_cache()
        log("secondary workloads")
        result["secondary"] = secondary(device, max(5, args.steps // 2), 3, args.algo, ms, args.partition, base)
        f8 = result["secondary"].get("qwen3_fp8")
        if f8 and f8.get("decode_avg_launch_us"):
            f8["frac_of_paged_read_time"] = round(ceiling["paged_read"]["fp8_paged_read_us"] /
                                                  f8["decode_avg_launch_us"], 4)
    if base is not None:
        base.close()
        head = base.results["qwen3_decode"]
        result["cpu_baseline"] = {
            "value": head["value"], "unit": head["unit"], "cores": base.workers, "kind": "oracle",
            "sample": f"the float64 oracle (numpy, one BLAS thread per worker process, {base.workers} worker "
                      f"processes) on the host's {cpu_model()}, on the GPU's own input bits: "
                      f"{head['sample']}, of the headline's layer 0 in {head['seconds']} s "
                      f"({head['items_per_s']} sequences/s); each workload below likewise for about "
                      f"{args.cpu_budget:g} s",
            "per_workload": base.results}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
