"""The float64 oracle over whole full-size workloads, spread over host worker
processes.

Every (sequence, q-head) row of the oracle's decode, and every (chunk,
kv-head) slice of its chunked prefill, depends on its own inputs only, so the
rows are computed by the unchanged oracle functions in independent worker
processes and put back in place. Inputs reach the workers as memory-mapped
.npy files (no copy of the caches per worker). The workers are started with
the "spawn" method, as fresh interpreters that import numpy and the oracle
only, so they never touch the GPU state of the test process.

This module imports no torch: it is what each worker imports.
"""

from __future__ import annotations

import atexit
import concurrent.futures as cf
import multiprocessing as mp
import os
import shutil
import tempfile

import numpy as np

import oracle
from oracle import fp8_cache as FP8

_POOL = None
_DIRS = []


def workers() -> int:
    # the host share of one GPU is 16 threads; never more than the affinity allows
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _pool():
    global _POOL
    if _POOL is None:
        # one BLAS thread per worker; set before the first worker starts
        for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
            os.environ[k] = "1"
        _POOL = cf.ProcessPoolExecutor(max_workers=workers(), mp_context=mp.get_context("spawn"))
        atexit.register(shutdown)
    return _POOL


def shutdown():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None
    while _DIRS:
        shutil.rmtree(_DIRS.pop(), ignore_errors=True)


class Staged:
    """Host arrays written once as .npy files that workers memory-map."""

    def __init__(self, **arrays):
        self.dir = tempfile.mkdtemp(prefix="pkv_oracle_")
        _DIRS.append(self.dir)
        self.paths = {}
        for name, a in arrays.items():
            path = os.path.join(self.dir, name + ".npy")
            np.save(path, np.ascontiguousarray(a), allow_pickle=False)
            self.paths[name] = path

    def close(self):
        shutil.rmtree(self.dir, ignore_errors=True)
        if self.dir in _DIRS:
            _DIRS.remove(self.dir)


def _load(paths):
    return {k: np.load(p, mmap_mode="r", allow_pickle=False) for k, p in paths.items()}


# ---- worker tasks ------------------------------------------------------------

def _decode_task(paths, seqs, scale, block_size):
    a = _load(paths)
    seqs = np.asarray(seqs)
    if "k_scale" in a:
        out = FP8.paged_attention_decode_fp8(np.asarray(a["q"][seqs]), a["k_cache"], a["v_cache"],
                                             np.asarray(a["k_scale"]), np.asarray(a["v_scale"]),
                                             np.asarray(a["block_tables"][seqs]),
                                             np.asarray(a["context_lens"][seqs]), scale, block_size)
    else:
        out = oracle.paged_attention_decode(np.asarray(a["q"][seqs]), a["k_cache"], a["v_cache"],
                                            np.asarray(a["block_tables"][seqs]),
                                            np.asarray(a["context_lens"][seqs]), scale, block_size)
    return seqs, out


def _prefill_task(paths, chunk, kv_head, scale, block_size, causal):
    """Chunk `chunk`, the q-heads of kv-head `kv_head` only, over that kv-head's
    cache columns: the oracle's chunked prefill with Hq/Hkv q-heads and one
    kv-head, which is exactly that slice of the full result."""
    a = _load(paths)
    cu = np.asarray(a["cu_seqlens_q"])
    lo, hi = int(cu[chunk]), int(cu[chunk + 1])
    hq, hkv = a["q"].shape[1], a["k_cache"].shape[2]
    g = hq // hkv
    q = np.asarray(a["q"][lo:hi, kv_head * g:(kv_head + 1) * g])
    kc = a["k_cache"][:, :, kv_head:kv_head + 1]
    vc = a["v_cache"][:, :, kv_head:kv_head + 1]
    bt = np.asarray(a["block_tables"][chunk:chunk + 1])
    ctx = np.asarray(a["context_lens"][chunk:chunk + 1])
    one = np.array([0, hi - lo], dtype=np.int32)
    if "k_scale" in a:
        ks = np.asarray(a["k_scale"][kv_head:kv_head + 1])
        vs = np.asarray(a["v_scale"][kv_head:kv_head + 1])
        out = FP8.paged_attention_prefill_chunk_fp8(q, kc, vc, ks, vs, bt, one, ctx, scale, block_size,
                                                    causal=causal)
    else:
        out = oracle.paged_attention_prefill_chunk(q, kc, vc, bt, one, ctx, scale, block_size,
                                                   causal=causal)
    return chunk, kv_head, out


# ---- drivers -------------------------------------------------------------------

def decode(q, k_cache, v_cache, block_tables, context_lens, scale, block_size, k_scale=None,
           v_scale=None):
    """oracle.paged_attention_decode (or its E4M3 form when scales are given)
    over every sequence; float64 [S, Hq, D]."""
    arrays = dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                  context_lens=context_lens)
    if k_scale is not None:
        arrays.update(k_scale=k_scale, v_scale=v_scale)
    st = Staged(**arrays)
    try:
        ctx = np.asarray(context_lens, np.int64)
        n = len(ctx)
        # about equal numbers of tokens per task, several tasks per worker
        tasks = max(1, min(n, 4 * workers()))
        order = np.argsort(-ctx, kind="stable")
        buckets = [[] for _ in range(tasks)]
        load = np.zeros(tasks)
        for s in order.tolist():
            i = int(np.argmin(load))
            buckets[i].append(s)
            load[i] += ctx[s] + 1
        out = np.zeros(np.asarray(q).shape, dtype=np.float64)
        futs = [_pool().submit(_decode_task, st.paths, sorted(b), float(scale), int(block_size))
                for b in buckets if b]
        for f in futs:
            seqs, part = f.result()
            out[seqs] = part
        return out
    finally:
        st.close()


def prefill(q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens, scale, block_size,
            causal=True, k_scale=None, v_scale=None):
    """oracle.paged_attention_prefill_chunk (or its E4M3 form) over every
    chunk; float64 [Tq, Hq, D]."""
    arrays = dict(q=q, k_cache=k_cache, v_cache=v_cache, block_tables=block_tables,
                  cu_seqlens_q=cu_seqlens_q, context_lens=context_lens)
    if k_scale is not None:
        arrays.update(k_scale=k_scale, v_scale=v_scale)
    st = Staged(**arrays)
    try:
        hq, hkv = np.asarray(q).shape[1], np.asarray(k_cache).shape[2]
        g = hq // hkv
        cu = np.asarray(cu_seqlens_q)
        ctx = np.asarray(context_lens, np.int64)
        # the largest chunks first, so the long tasks start early
        jobs = sorted(((c, h) for c in range(len(cu) - 1) for h in range(hkv)),
                      key=lambda ch: -int(ctx[ch[0]]) * int(cu[ch[0] + 1] - cu[ch[0]]))
        futs = [_pool().submit(_prefill_task, st.paths, c, h, float(scale), int(block_size), bool(causal))
                for c, h in jobs]
        out = np.zeros(np.asarray(q).shape, dtype=np.float64)
        for f in futs:
            c, h, part = f.result()
            out[cu[c]:cu[c + 1], h * g:(h + 1) * g] = part
        return out
    finally:
        st.close()
