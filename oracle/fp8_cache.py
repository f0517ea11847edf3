"""CPU float64 oracle for a float8 (E4M3) paged KV cache.

TEST INFRASTRUCTURE, like the rest of this package: only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may use it, and it
shares nothing with the HIP library.

The pages list support for quantized models among vLLM's features
("Building a minimal vLLM implementation", the feature list that opens the
page) and fix nothing further. The readings taken here:

  * element format: OCP 8-bit E4M3 ("fn" variant): 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent field 0 holds subnormals
    m/8 * 2^-6; no infinities; the codes 0x7f and 0xff are NaN; the largest
    finite magnitude is 448 (code 0x7e);
  * one float32 scale per kv-head for K and one for V: the cache holds
    e4m3(x / scale) and stands for e4m3_value * scale;
  * quantisation: t = x / scale as one correctly rounded float32 division,
    then t rounded to the nearest E4M3 value, ties to the even code; |t| at
    or above 448 saturates to +-448 (the format has no infinity; clamping
    keeps an outlier finite instead of turning it into NaN); NaN gives 0x7f;
  * attention over the cache is the ordinary definition applied to the
    dequantised rows, so this module only turns codes into values and hands
    them to the same attention routine as the bf16 oracle.
"""

from __future__ import annotations

import numpy as np

from .paged_attention import attend_rows, kv_cache_store, paged_attention_prefill_chunk, to_f64

__all__ = [
    "E4M3_MAX",
    "E4M3_TABLE",
    "e4m3_value",
    "e4m3_encode",
    "quantize_rows",
    "kv_cache_store_fp8",
    "dequantize",
    "paged_attention_decode_fp8",
    "paged_attention_prefill_chunk_fp8",
]

E4M3_MAX = 448.0


def e4m3_value(code) -> np.ndarray:
    """Value of 8-bit E4M3 codes, from the field layout (float64, NaN for 0x7f/0xff)."""
    c = np.asarray(code, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exponent = (c >> 3) & 0xF
    mantissa = c & 0x7
    subnormal = mantissa / 8.0 * 2.0 ** -6
    normal = (1.0 + mantissa / 8.0) * 2.0 ** (exponent - 7)
    value = sign * np.where(exponent == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, value)


E4M3_TABLE = e4m3_value(np.arange(256))
_POS_VALUES = E4M3_TABLE[:0x7F]          # codes 0x00 .. 0x7e: 0 .. 448, increasing


def e4m3_encode(t) -> np.ndarray:
    """Nearest E4M3 code of each value (ties to the even code), saturating.

    The non-negative finite codes 0x00..0x7e are the format's values in
    increasing order, so the candidates for |t| are the table entries just
    below and just above it; the nearer wins and a tie goes to the code with
    an even last bit (an even mantissa). The sign bit is copied, so -0.0 and
    negative values that round to zero keep it.
    """
    t = np.asarray(t, dtype=np.float64)
    a = np.minimum(np.abs(np.nan_to_num(t, nan=0.0)), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS_VALUES, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo) | np.where(np.signbit(t), 0x80, 0)
    code = np.where(np.isnan(t), 0x7F, code)
    return code.astype(np.uint8)


def quantize_rows(x, scale) -> np.ndarray:
    """Codes of rows x [T, Hkv, D] (float32, or bf16 bit patterns) with one
    scale per kv-head: e4m3(float32(x) / float32(scale[g]))."""
    xf = to_f64(x).astype(np.float32)                 # exact: bf16 and f32 are f32 values
    s = np.asarray(scale, dtype=np.float32)[None, :, None]
    return e4m3_encode(xf / s)                         # numpy float32 division is IEEE


def kv_cache_store_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, block_size):
    """Quantise new K/V rows with the per-kv-head scales and write their codes
    into the slots (the same slot rule as the unquantised store)."""
    return kv_cache_store(quantize_rows(k, k_scale), quantize_rows(v, v_scale), k_cache, v_cache,
                          slot_mapping, block_size)


def dequantize(codes, scale) -> np.ndarray:
    """Values of cache rows [..., Hkv, D] of codes: e4m3_value * scale[g]."""
    return E4M3_TABLE[np.asarray(codes)] * np.asarray(scale, dtype=np.float64)[:, None]


def paged_attention_decode_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                               scale, block_size):
    """Decode attention over E4M3 caches: each sequence's rows are gathered
    (position p in block table[p // block_size], row p % block_size),
    dequantised, and attended to exactly as in the unquantised decode."""
    qf = to_f64(q)
    num_seqs, num_q_heads, head_dim = qf.shape
    kc, vc = np.asarray(k_cache), np.asarray(v_cache)
    num_kv_heads = kc.shape[2]
    group = num_q_heads // num_kv_heads
    assert group * num_kv_heads == num_q_heads
    out = np.zeros((num_seqs, num_q_heads, head_dim), dtype=np.float64)
    for s in range(num_seqs):
        ctx = int(context_lens[s])
        if ctx == 0:
            continue
        positions = np.arange(ctx)
        physical = np.asarray(block_tables[s])[positions // block_size]
        keys = dequantize(kc[physical, positions % block_size], k_scale)
        values = dequantize(vc[physical, positions % block_size], v_scale)
        for h in range(num_q_heads):
            g = h // group
            out[s, h] = attend_rows(qf[s, h][None, :], keys[:, g], values[:, g], scale, [ctx])[0]
    return out


def paged_attention_prefill_chunk_fp8(q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                      cu_seqlens_q, context_lens, scale, block_size, causal=True):
    """Chunked prefill over E4M3 caches: the caches are dequantised (code
    value times the kv-head's scale) and the unquantised prefill definition
    is applied to them unchanged (same chunk, position and mask rules)."""
    kd = E4M3_TABLE[np.asarray(k_cache)] * np.asarray(k_scale, dtype=np.float64)[None, None, :, None]
    vd = E4M3_TABLE[np.asarray(v_cache)] * np.asarray(v_scale, dtype=np.float64)[None, None, :, None]
    return paged_attention_prefill_chunk(q, kd, vd, block_tables, cu_seqlens_q, context_lens, scale,
                                         block_size, causal=causal)
