"""The float64 oracle timed on the host's cores: the CPU baseline that the
benchmark reports beside the GPU's numbers.

TEST INFRASTRUCTURE: started only by the benchmark's CPU-baseline leg. It
runs the oracle's own functions, unchanged, over a bounded sample of a
workload, spread over worker processes (one BLAS thread each), and reports
how much of the workload's algorithmic work the sample covered per second.
It does no attention arithmetic of its own.

Run as a helper process (python -m oracle.baseline WORKERS): the worker pool
starts at once, before the parent touches the GPU. The parent then writes
one JSON request per line on stdin and reads one JSON reply per line:
  {"kind": "decode", "dir": D, "scale": s, "block_size": bs, "budget_s": t}
  {"kind": "prefill", "dir": D, "scale": s, "block_size": bs, "budget_s": t}
where D holds q.npy, k_cache.npy, v_cache.npy, block_tables.npy,
context_lens.npy (and cu_seqlens_q.npy for a prefill), as the GPU saw them
(bf16 as uint16 bit patterns). Decode work is taken sequence by sequence in
index order, a prefill's (chunk, kv-head) slices chunk by chunk, cycling
through the workload again after a full pass, until the time budget is
spent; the reply lists the units done (with repeats) and the wall time.
"""

from __future__ import annotations

import concurrent.futures as cf
import json
import os
import sys
import time


_MAPPED = {}


def _load(d):
    """The workload's arrays, memory-mapped once per worker (the latest
    workload only)."""
    import numpy as np
    if d not in _MAPPED:
        _MAPPED.clear()
        _MAPPED[d] = {name[:-4]: np.load(os.path.join(d, name), mmap_mode="r", allow_pickle=False)
                      for name in os.listdir(d) if name.endswith(".npy")}
    return _MAPPED[d]


def _decode_task(d, seqs, scale, block_size):
    import numpy as np
    from oracle import paged_attention_decode
    a = _load(d)
    seqs = np.asarray(seqs)
    paged_attention_decode(np.asarray(a["q"][seqs]), a["k_cache"], a["v_cache"], np.asarray(a["block_tables"][seqs]),
                           np.asarray(a["context_lens"][seqs]), scale, block_size)
    return len(seqs)


def _prefill_task(d, chunk, kv_head, scale, block_size):
    import numpy as np
    from oracle import paged_attention_prefill_chunk
    a = _load(d)
    cu = np.asarray(a["cu_seqlens_q"])
    lo, hi = int(cu[chunk]), int(cu[chunk + 1])
    g = a["q"].shape[1] // a["k_cache"].shape[2]
    paged_attention_prefill_chunk(np.asarray(a["q"][lo:hi, kv_head * g:(kv_head + 1) * g]),
                                  a["k_cache"][:, :, kv_head:kv_head + 1], a["v_cache"][:, :, kv_head:kv_head + 1],
                                  np.asarray(a["block_tables"][chunk:chunk + 1]), np.array([0, hi - lo], np.int32),
                                  np.asarray(a["context_lens"][chunk:chunk + 1]), scale, block_size, causal=True)
    return 1


def _warm():
    import numpy  # noqa: F401
    import oracle  # noqa: F401
    return os.getpid()


def _run(pool, workers, req):
    """Submit tasks in workload order, keeping every worker busy, until the
    budget is spent; then wait for the ones in flight. Returns the sample."""
    import numpy as np
    d, scale, bs, budget = req["dir"], float(req["scale"]), int(req["block_size"]), float(req["budget_s"])
    a = _load(d)
    ctx = np.asarray(a["context_lens"], np.int64)
    if req["kind"] == "decode":
        units = [(s,) for s in range(len(ctx))]
        submit = lambda u: pool.submit(_decode_task, d, [u[0]], scale, bs)
    else:
        hkv = a["k_cache"].shape[2]
        units = [(c, h) for c in range(len(ctx)) for h in range(hkv)]
        submit = lambda u: pool.submit(_prefill_task, d, u[0], u[1], scale, bs)
    t0 = time.perf_counter()
    done, pending, i = [], {}, 0
    # units in workload order, cycled after a full pass, until the budget is spent
    while time.perf_counter() - t0 < budget or pending:
        while len(pending) < 2 * workers and time.perf_counter() - t0 < budget:
            u = units[i % len(units)]
            pending[submit(u)] = u
            i += 1
        if not pending:
            break
        fin, _ = cf.wait(list(pending), return_when=cf.FIRST_COMPLETED)
        for f in fin:
            f.result()
            done.append(pending.pop(f))
    return {"units": done, "passes": len(done) / len(units), "seconds": time.perf_counter() - t0}


def main():
    workers = int(sys.argv[1]) if len(sys.argv) > 1 else 1
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    import multiprocessing as mp
    pool = cf.ProcessPoolExecutor(max_workers=workers, mp_context=mp.get_context("spawn"))
    pids = set(f.result() for f in [pool.submit(_warm) for _ in range(4 * workers)])
    print(json.dumps({"ready": True, "workers": workers, "worker_pids": len(pids)}), flush=True)
    for line in sys.stdin:
        line = line.strip()
        if not line or line == "quit":
            break
        try:
            reply = _run(pool, workers, json.loads(line))
        except Exception as e:  # reported to the parent, which decides
            reply = {"error": repr(e)}
        print(json.dumps(reply), flush=True)
    pool.shutdown(wait=True)


if __name__ == "__main__":
    main()
