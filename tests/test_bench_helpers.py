"""Host-side helpers of the benchmark (no GPU): the tile list of the
paged-read ceiling names exactly the tiles the decode reads."""

import torch

import bench
from paged_attention_kv_store_amd import workloads as W


def test_paged_tile_offsets_list_every_tile_once_in_bounds():
    b = W.random_decode_batch(5, 23, 32, 8, 128, torch.bfloat16, max_ctx=700, min_ctx=0, block_size=32)
    bt, ctx, bs = b.pool.block_tables, b.pool.context_lens, b.block_size
    for slice_bytes in (256, 128):
        offs, pitch = bench.paged_tile_offsets(b, slice_bytes, "cpu")
        want = [(int(bt[s][16 * t // bs]) * bs + (16 * t) % bs) * pitch + g * slice_bytes
                for g in range(b.num_kv_heads) for s in range(len(ctx)) for t in range((int(ctx[s]) + 15) // 16)]
        assert pitch == b.num_kv_heads * slice_bytes
        assert offs.numpy().tolist() == want
        # the last byte a tile's read touches stays inside the pool (rows of `pitch` bytes)
        if want:
            assert int(offs.max()) + 15 * pitch + slice_bytes <= b.pool.num_blocks * bs * pitch
