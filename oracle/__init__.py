"""Plain CPU float64 oracle for paged-KV attention.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code with it. Every function here is pinned by the CPU tests
(closed forms, hand-worked golden cases, brute force, an independent library
attention routine and invariants); no function is left unpinned.
"""

from .paged_attention import (  # noqa: F401
    attend_rows,
    gather_context,
    kv_cache_store,
    paged_attention_decode,
    paged_attention_prefill_chunk,
    to_f64,
)
