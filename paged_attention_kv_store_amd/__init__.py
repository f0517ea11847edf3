"""Paged-KV attention for MI355X (gfx950).

The compute path is a C-ABI shared library of hand-written HIP kernels
(csrc/, interface in include/pkv.h); this package is its thin ctypes binding
plus the seeded input generators. Importing the package does not load the
library; the first call does, and raises if it has not been built.
"""

from .binding import (  # noqa: F401
    DECODE_ALGOS,
    PARTITION_AUTO,
    PARTITION_BALANCED,
    PARTITION_PLANNED,
    DecodeFp8Launch,
    DecodeLaunch,
    DecodePlanLaunch,
    DecodeStoreFp8Launch,
    DecodeStoreLaunch,
    PkvError,
    PrefillFp8Launch,
    PrefillLaunch,
    SharedPrefixDecodeLaunch,
    StoreFp8Launch,
    StoreLaunch,
    check_paged_inputs,
    check_slots,
    decode_auto_partition,
    decode_plan,
    decode_plan_size,
    decode_workspace_init,
    decode_workspace_size,
    kv_cache_store,
    kv_cache_store_fp8,
    lib,
    library_path,
    new_decode_plan,
    new_decode_workspace,
    paged_attention_decode,
    paged_attention_decode_fp8,
    paged_attention_decode_shared_prefix,
    paged_attention_decode_static,
    paged_attention_decode_store,
    paged_attention_decode_store_fp8,
    paged_attention_prefill_chunk,
    paged_attention_prefill_chunk_fp8,
)
