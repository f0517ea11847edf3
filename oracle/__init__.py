"""Plain CPU float64 oracle for paged-KV attention.

TEST INFRASTRUCTURE: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package. The HIP library never calls it and
shares no code with it. Every function here is pinned by the CPU tests
(closed forms, hand-worked golden cases, brute force, an independent library
attention routine and invariants); no function is left unpinned.

oracle.fp8_cache holds the E4M3-quantised cache (store with per-kv-head
scales, decode over dequantised rows), pinned in tests/test_oracle_fp8.py.
"""

from .paged_attention import (  # noqa: F401
    attend_rows,
    gather_context,
    kv_cache_store,
    paged_attention_decode,
    paged_attention_prefill_chunk,
    to_f64,
)
from . import fp8_cache  # noqa: F401,E402
