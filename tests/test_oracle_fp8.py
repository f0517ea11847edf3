"""Pins of the E4M3 KV-cache oracle (CPU only).

The format table and the rounding are checked against torch's own
float8_e4m3fn conversion (an independent library routine), hand-decoded
codes, closed forms (saturation, round trips, the half-gap error bound) and
the unquantised oracle on dequantised caches. A planted slip in the module's
source must fail at least one of these checks.
"""

import inspect
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import fp8_cache as FP8

# hand-decoded codes: (code, value) from the field layout
HAND = [(0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0), (0x01, 2.0 ** -9),
        (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x3C, 1.5), (0x40, 2.0), (0x77, 240.0),
        (0x78, 256.0), (0x30, 0.5), (0x5F, 30.0)]


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_codes_saturated(x):
    """torch rounds past 448 to NaN; the cache reading saturates first."""
    return _torch_codes(np.clip(np.asarray(x, dtype=np.float32), -448, 448))


def _rounding_probe():
    """Every finite value, every midpoint between neighbours, points just off
    the midpoints, and random magnitudes, with both signs; all inside +-448."""
    v = FP8.E4M3_TABLE[:0x7F]
    mid = (v[:-1] + v[1:]) / 2
    rng = np.random.default_rng(0)
    x = np.concatenate([v, mid, np.nextafter(mid.astype(np.float32), np.float32(0)),
                        np.nextafter(mid.astype(np.float32), np.float32(1000)),
                        rng.uniform(0, 448, 4000), np.exp(rng.uniform(-14, 6, 4000))])
    x = np.concatenate([x, -x]).astype(np.float32)
    return x[np.abs(x) <= 448]


def check_table(mod):
    torch_vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    same = (mod.E4M3_TABLE == torch_vals) | (np.isnan(mod.E4M3_TABLE) & np.isnan(torch_vals))
    assert same.all()
    for code, val in HAND:
        assert mod.E4M3_TABLE[code] == val, hex(code)
    assert np.isnan(mod.E4M3_TABLE[0x7F]) and np.isnan(mod.E4M3_TABLE[0xFF])
    assert np.signbit(mod.E4M3_TABLE[0x80])


def check_encode_matches_torch(mod):
    x = _rounding_probe()
    np.testing.assert_array_equal(mod.e4m3_encode(x), _torch_codes(x))


def check_encode_closed_forms(mod):
    # saturation: the format has no infinity; outliers clamp to +-448
    big = np.array([448.0, 449.0, 463.9, 464.0, 480.0, 1e6, np.inf, -464.0, -1e30, -np.inf])
    np.testing.assert_array_equal(mod.e4m3_encode(big), [0x7E] * 7 + [0xFE] * 3)
    assert mod.e4m3_encode(np.array([np.nan]))[0] == 0x7F
    # ties to even: 2^-10 lies halfway between 0 and 2^-9; 1.5 * 2^-9 between codes 1 and 2
    np.testing.assert_array_equal(mod.e4m3_encode(np.array([2.0 ** -10, 1.5 * 2.0 ** -9, 2.5 * 2.0 ** -9,
                                                            1.0625, 1.1875, -1.0625])),
                                  [0x00, 0x02, 0x02, 0x38, 0x3A, 0xB8])
    # every finite code round-trips; the error is at most half the local gap
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F])
    np.testing.assert_array_equal(mod.e4m3_encode(mod.E4M3_TABLE[codes]), codes)
    x = np.random.default_rng(1).uniform(-448, 448, 5000)
    got = mod.E4M3_TABLE[mod.e4m3_encode(x)]
    mag = np.abs(x)
    gap = np.where(mag < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(mag, 2.0 ** -6))) - 3))
    assert (np.abs(got - x) <= gap / 2 + 1e-15).all()


def check_quantized_store(mod, seed=3):
    rng = np.random.default_rng(seed)
    nb, bs, hkv, d, t = 6, 4, 3, 8, 9
    k = rng.normal(0, 3, (t, hkv, d)).astype(np.float32)
    v = rng.normal(0, 3, (t, hkv, d)).astype(np.float32)
    ks = np.array([0.01, 0.02, 0.5], np.float32)
    vs = np.array([0.03, 0.007, 1.0], np.float32)
    kc = rng.integers(0, 256, (nb, bs, hkv, d)).astype(np.uint8)
    vc = rng.integers(0, 256, (nb, bs, hkv, d)).astype(np.uint8)
    slots = np.array([0, 5, -1, 23, 7, 12, -3, 1, 18])
    kc2, vc2 = mod.kv_cache_store_fp8(k, v, kc, vc, slots, ks, vs, bs)
    written = set()
    for i, s in enumerate(slots):
        if s < 0:
            continue
        written.add(int(s))
        b, r = divmod(int(s), bs)
        np.testing.assert_array_equal(kc2[b, r], _torch_codes_saturated(k[i] / ks[:, None]))
        np.testing.assert_array_equal(vc2[b, r], _torch_codes_saturated(v[i] / vs[:, None]))
    for s in range(nb * bs):
        if s not in written:
            b, r = divmod(s, bs)
            assert (kc2[b, r] == kc[b, r]).all() and (vc2[b, r] == vc[b, r]).all()
    # bf16 bit patterns are upcast exactly before the division
    kb = (k.view(np.uint32) >> 16).astype(np.uint16)
    kf = (kb.astype(np.uint32) << 16).view(np.float32)
    np.testing.assert_array_equal(mod.quantize_rows(kb, ks), _torch_codes_saturated(kf / ks[None, :, None]))


def check_decode_is_dequantised_decode(mod, seed=5):
    rng = np.random.default_rng(seed)
    nb, bs, hkv, hq, d, s = 12, 4, 2, 4, 8, 4
    kc = rng.integers(0, 0x7F, (nb, bs, hkv, d)).astype(np.uint8) | (rng.integers(0, 2, (nb, bs, hkv, d)) << 7).astype(np.uint8)
    vc = rng.integers(0, 0x7F, (nb, bs, hkv, d)).astype(np.uint8) | (rng.integers(0, 2, (nb, bs, hkv, d)) << 7).astype(np.uint8)
    ks = np.array([0.05, 0.002], np.float32)
    vs = np.array([0.01, 0.3], np.float32)
    q = rng.normal(0, 1, (s, hq, d))
    tables = np.stack([rng.permutation(nb)[:5] for _ in range(s)])
    ctx = np.array([1, 7, 20, 0])
    got = mod.paged_attention_decode_fp8(q, kc, vc, ks, vs, tables, ctx, 0.3, bs)
    kd = mod.E4M3_TABLE[kc] * ks.astype(np.float64)[None, None, :, None]
    vd = mod.E4M3_TABLE[vc] * vs.astype(np.float64)[None, None, :, None]
    want = oracle.paged_attention_decode(q, kd, vd, tables, ctx, 0.3, bs)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    # one-token context: the output is the dequantised V row, exactly
    b0 = tables[0, 0]
    np.testing.assert_array_equal(got[0, :2], np.repeat(mod.E4M3_TABLE[vc[b0, 0, :1]], 2, axis=0) * vs[0])
    assert (got[3] == 0).all()


def _codes(rng, shape):
    """Random finite E4M3 codes of both signs (never 0x7f / 0xff)."""
    return (rng.integers(0, 0x7F, shape) | (rng.integers(0, 2, shape) << 7)).astype(np.uint8)


def check_prefill_pins(mod, seed=9):
    rng = np.random.default_rng(seed)
    nb, bs, hkv, hq, d = 16, 4, 2, 4, 8
    kc, vc = _codes(rng, (nb, bs, hkv, d)), _codes(rng, (nb, bs, hkv, d))
    ks = np.array([0.04, 0.003], np.float32)
    vs = np.array([0.02, 0.5], np.float32)
    ctx = np.array([9, 14, 5])
    rows = np.array([4, 1, 5])                       # the last chunk has no earlier tokens
    cu = np.concatenate([[0], np.cumsum(rows)])
    tables = np.stack([rng.permutation(nb)[:5] for _ in range(3)])
    q = rng.normal(0, 1, (int(cu[-1]), hq, d))
    got = mod.paged_attention_prefill_chunk_fp8(q, kc, vc, ks, vs, tables, cu, ctx, 0.4, bs)
    # row i of a chunk is single-row decode over the first ctx - L + i + 1 keys
    for c in range(3):
        for i in range(rows[c]):
            r = cu[c] + i
            want = mod.paged_attention_decode_fp8(q[r:r + 1], kc, vc, ks, vs, tables[c:c + 1],
                                                  np.array([ctx[c] - rows[c] + i + 1]), 0.4, bs)
            np.testing.assert_allclose(got[r], want[0], rtol=0, atol=1e-12)
    # non-causal: every row sees all ctx keys, so the last row is unchanged
    nc = mod.paged_attention_prefill_chunk_fp8(q, kc, vc, ks, vs, tables, cu, ctx, 0.4, bs, causal=False)
    for c in range(3):
        np.testing.assert_allclose(nc[cu[c + 1] - 1], got[cu[c + 1] - 1], rtol=0, atol=1e-12)
    # identical keys: the weights are uniform, the output is the mean of the visible V rows
    kc_same = np.broadcast_to(kc[:1, :1], kc.shape).copy()
    same = mod.paged_attention_prefill_chunk_fp8(q, kc_same, vc, ks, vs, tables, cu, ctx, 0.4, bs)
    for i in range(rows[0]):
        n_vis = ctx[0] - rows[0] + i + 1
        pos = np.arange(n_vis)
        vrows = mod.E4M3_TABLE[vc[tables[0][pos // bs], pos % bs]]      # [n_vis, hkv, d]
        for h in range(hq):
            np.testing.assert_allclose(same[i, h], vrows[:, h // 2].mean(0) * vs[h // 2], rtol=1e-12, atol=1e-15)


CHECKS = [check_table, check_encode_matches_torch, check_encode_closed_forms, check_quantized_store,
          check_decode_is_dequantised_decode, check_prefill_pins]


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(FP8)


MUTANTS = {
    "exponent_bias_8": ("2.0 ** (exponent - 7)", "2.0 ** (exponent - 8)"),
    "subnormal_scale_wrong": ("mantissa / 8.0 * 2.0 ** -6", "mantissa / 8.0 * 2.0 ** -7"),
    "nan_code_missing": ("(c & 0x7F) == 0x7F, np.nan", "(c & 0xFF) == 0xFF, np.nan"),
    "ties_to_upper": ("(d_hi == d_lo) & (hi % 2 == 0)", "(d_hi == d_lo)"),
    "ties_to_lower": ("(d_hi == d_lo) & (hi % 2 == 0)", "(d_hi == d_lo) & False"),
    "overflow_to_nan": ("code = np.where(np.isnan(t), 0x7F, code)",
                        "code = np.where(np.isnan(t) | (np.abs(t) > E4M3_MAX), 0x7F, code)"),
    "nan_not_canonical": ("code = np.where(np.isnan(t), 0x7F, code)", "code = code"),
    "sign_dropped": ("| np.where(np.signbit(t), 0x80, 0)", "| 0"),
    "scale_multiplied": ("return e4m3_encode(xf / s)", "return e4m3_encode(xf * s)"),
    "k_scale_for_v": ("quantize_rows(v, v_scale)", "quantize_rows(v, k_scale)"),
    "dequantize_unscaled": ("E4M3_TABLE[np.asarray(codes)] * np.asarray(scale, dtype=np.float64)[:, None]",
                            "E4M3_TABLE[np.asarray(codes)]"),
    "gather_row_from_block": ("kc[physical, positions % block_size]", "kc[physical, positions // block_size]"),
    "values_with_k_scale": ("dequantize(vc[physical, positions % block_size], v_scale)",
                            "dequantize(vc[physical, positions % block_size], k_scale)"),
    "prefill_v_scaled_by_k": ("vd = E4M3_TABLE[np.asarray(v_cache)] * np.asarray(v_scale,",
                              "vd = E4M3_TABLE[np.asarray(v_cache)] * np.asarray(k_scale,"),
    "prefill_k_unscaled": ("kd = E4M3_TABLE[np.asarray(k_cache)] * np.asarray(k_scale, dtype=np.float64)[None, None, :, None]",
                           "kd = E4M3_TABLE[np.asarray(k_cache)] * 1.0"),
    "prefill_not_causal": ("block_size, causal=causal)", "block_size, causal=False)"),
}


def _mutant(old, new):
    src = inspect.getsource(FP8)
    assert old in src, f"mutation target not found: {old!r}"
    mod = types.ModuleType("oracle.fp8_mutant")
    mod.__dict__["__package__"] = "oracle"
    exec(compile(src.replace(old, new), "<fp8_mutant>", "exec"), mod.__dict__)
    return mod


def test_unmutated_source_passes():
    mod = _mutant("", "")
    for check in CHECKS:
        check(mod)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    mod = _mutant(*MUTANTS[name])
    caught = False
    for check in CHECKS:
        try:
            check(mod)
        except Exception:
            caught = True
            break
    assert caught, f"mutant {name} passed every pin"
