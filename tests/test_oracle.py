"""Pins of the CPU oracle to things other than itself.

Each check below is a function of the oracle module so that the mutation test
(test_oracle_mutations.py) can run the same checks against deliberately broken
copies of the oracle and show that every planted mistake fails at least one.

Pins used:
  * hand-worked golden cases (tests/golden/hand_worked.json), derived by hand;
  * an independent library routine: torch's scaled_dot_product_attention in
    float64 on the CPU, over K/V gathered by a separate indexing route
    (a flat row index built with torch) and heads expanded with
    repeat_interleave, with an explicit boolean causal mask;
  * brute force with pure-Python loops, math.exp and math.fsum;
  * invariants and closed forms: block-id permutation invariance (bit-exact),
    context 1 returns the V row exactly, identical keys or scale 0 give the
    mean of V, a 1-row chunk equals decode, NaN in dead rows never leaks.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import paged_attention as ORACLE

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_worked.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _arr(x):
    return np.asarray(x, dtype=np.float64)


# ----------------------------------------------------------------------------
# checks (each takes the module under test)
# ----------------------------------------------------------------------------

def check_golden(mod):
    g = _golden()
    for case in g["decode"]:
        out = mod.paged_attention_decode(
            _arr(case["q"]), _arr(case["k_cache"]), _arr(case["v_cache"]),
            np.asarray(case["block_tables"]), np.asarray(case["context_lens"]),
            case["scale"], case["block_size"])
        np.testing.assert_allclose(out, _arr(case["expected"]), atol=1e-12, rtol=0,
                                   err_msg=case["name"])
    for case in g["prefill"]:
        for causal, key in ((True, "expected_causal"), (False, "expected_full")):
            out = mod.paged_attention_prefill_chunk(
                _arr(case["q"]), _arr(case["k_cache"]), _arr(case["v_cache"]),
                np.asarray(case["block_tables"]), np.asarray(case["cu_seqlens_q"]),
                np.asarray(case["context_lens"]), case["scale"], case["block_size"],
                causal=causal)
            np.testing.assert_allclose(out, _arr(case[key]), atol=1e-12, rtol=0,
                                       err_msg=case["name"] + key)
    for case in g["store"]:
        shape = (case["num_blocks"], case["block_size"]) + np.asarray(case["k"]).shape[1:]
        kc, vc = mod.kv_cache_store(_arr(case["k"]), _arr(case["v"]), np.zeros(shape),
                                    np.zeros(shape), np.asarray(case["slot_mapping"]),
                                    case["block_size"])
        np.testing.assert_array_equal(kc, _arr(case["expected_k_cache"]))
        np.testing.assert_array_equal(vc, _arr(case["expected_v_cache"]))
    bits = np.asarray(g["bf16"]["bits"], dtype=np.uint16)
    want = np.asarray([float(v) for v in g["bf16"]["values"]], dtype=np.float64)
    np.testing.assert_array_equal(mod.to_f64(bits), want)


def _random_case(seed, num_seqs=5, hq=8, hkv=2, d=8, bs=4, max_ctx=37, nb=None):
    rng = np.random.default_rng(seed)
    ctx = rng.integers(1, max_ctx + 1, size=num_seqs)
    ctx[0] = max_ctx
    need = -(-ctx // bs)
    nb = nb or int(need.sum()) + 3
    perm = rng.permutation(nb)
    mb = int(need.max())
    tables = np.full((num_seqs, mb), perm[-1])
    c = 0
    for s in range(num_seqs):
        tables[s, :need[s]] = perm[c:c + need[s]]
        c += need[s]
    kc = rng.standard_normal((nb, bs, hkv, d))
    vc = rng.standard_normal((nb, bs, hkv, d))
    q = rng.standard_normal((num_seqs, hq, d))
    return q, kc, vc, tables, ctx


def _torch_gather(cache, table, ctx, bs):
    """Independent gather: flat row ids built with torch arithmetic."""
    cache_t = torch.as_tensor(cache, dtype=torch.float64)
    nb, _, hkv, d = cache_t.shape
    flat = cache_t.reshape(nb * bs, hkv, d)
    pos = torch.arange(int(ctx))
    tbl = torch.as_tensor(np.asarray(table), dtype=torch.long)
    rows = tbl.index_select(0, torch.div(pos, bs, rounding_mode="floor")) * bs + torch.remainder(pos, bs)
    return flat.index_select(0, rows)


def _sdpa(q_rows, keys, values, scale, mask):
    """torch SDPA, float64 CPU. q_rows [Hq, L, D]; keys/values [Hkv, ctx, D]."""
    hq = q_rows.shape[0]
    group = hq // keys.shape[0]
    k = keys.repeat_interleave(group, dim=0)
    v = values.repeat_interleave(group, dim=0)
    return torch.nn.functional.scaled_dot_product_attention(
        q_rows[None], k[None], v[None], attn_mask=mask, scale=scale)[0]


def check_sdpa_decode(mod, seed=0, **kw):
    q, kc, vc, tables, ctx = _random_case(seed, **kw)
    bs = kc.shape[1]
    scale = 0.37
    out = mod.paged_attention_decode(q, kc, vc, tables, ctx, scale, bs)
    for s in range(len(ctx)):
        keys = _torch_gather(kc, tables[s], ctx[s], bs).permute(1, 0, 2)
        values = _torch_gather(vc, tables[s], ctx[s], bs).permute(1, 0, 2)
        qs = torch.as_tensor(q[s], dtype=torch.float64)[:, None, :]
        ref = _sdpa(qs, keys, values, scale, None)[:, 0, :].numpy()
        np.testing.assert_allclose(out[s], ref, atol=1e-12, rtol=0)


def check_sdpa_prefill(mod, seed=0, causal=True, hq=8, hkv=2, d=8, bs=4):
    rng = np.random.default_rng(seed + 100)
    rows = np.array([1, 7, 13, 4])
    prior = np.array([0, 9, 2, 21])
    ctx = rows + prior
    need = -(-ctx // bs)
    nb = int(need.sum()) + 2
    perm = rng.permutation(nb)
    tables = np.full((len(ctx), int(need.max())), perm[-1])
    c = 0
    for s in range(len(ctx)):
        tables[s, :need[s]] = perm[c:c + need[s]]
        c += need[s]
    kc = rng.standard_normal((nb, bs, hkv, d))
    vc = rng.standard_normal((nb, bs, hkv, d))
    cu = np.concatenate([[0], np.cumsum(rows)])
    q = rng.standard_normal((int(cu[-1]), hq, d))
    scale = 0.29
    out = mod.paged_attention_prefill_chunk(q, kc, vc, tables, cu, ctx, scale, bs, causal=causal)
    for s in range(len(ctx)):
        keys = _torch_gather(kc, tables[s], ctx[s], bs).permute(1, 0, 2)
        values = _torch_gather(vc, tables[s], ctx[s], bs).permute(1, 0, 2)
        qs = torch.as_tensor(q[cu[s]:cu[s + 1]], dtype=torch.float64).permute(1, 0, 2)
        if causal:
            i = torch.arange(int(rows[s]))[:, None]
            j = torch.arange(int(ctx[s]))[None, :]
            mask = j <= (int(prior[s]) + i)
        else:
            mask = None
        ref = _sdpa(qs, keys, values, scale, mask).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[cu[s]:cu[s + 1]], ref, atol=1e-12, rtol=0)


def _brute(q, kc, vc, table, ctx, scale, bs, group, visible=None):
    """Pure-Python attention for one query row set of one sequence."""
    res = []
    nq, hq, d = len(q), len(q[0]), len(q[0][0])
    for i in range(nq):
        per_head = []
        for h in range(hq):
            g = h // group
            m = ctx if visible is None else visible[i]
            logits = []
            for p in range(m):
                b = int(table[p // bs])
                r = p % bs
                logits.append(scale * math.fsum(q[i][h][x] * kc[b][r][g][x] for x in range(d)))
            if not logits:
                per_head.append([0.0] * d)
                continue
            top = max(logits)
            w = [math.exp(x - top) for x in logits]
            tot = math.fsum(w)
            row = []
            for x in range(d):
                acc = math.fsum(w[p] * vc[int(table[p // bs])][p % bs][g][x] for p in range(m))
                row.append(acc / tot)
            per_head.append(row)
        res.append(per_head)
    return np.asarray(res)


def check_brute_force(mod, seed=3):
    rng = np.random.default_rng(seed)
    bs, hkv, hq, d = 4, 2, 4, 4
    group = hq // hkv
    for ctx in list(range(1, 2 * bs + 2)) + [2 * bs + 7]:
        need = -(-ctx // bs)
        nb = need + 2
        perm = rng.permutation(nb)
        table = np.concatenate([perm[:need], [perm[-1]]])
        kc = rng.standard_normal((nb, bs, hkv, d))
        vc = rng.standard_normal((nb, bs, hkv, d))
        q = rng.standard_normal((1, hq, d))
        out = mod.paged_attention_decode(q, kc, vc, table[None], np.array([ctx]), 0.8, bs)
        want = _brute(q.tolist(), kc.tolist(), vc.tolist(), table, ctx, 0.8, bs, group)
        np.testing.assert_allclose(out[0], want[0], atol=1e-12, rtol=0)
        # the same context as a causal chunk of up to 3 rows
        rows = min(3, ctx)
        qq = rng.standard_normal((rows, hq, d))
        out = mod.paged_attention_prefill_chunk(qq, kc, vc, table[None], np.array([0, rows]),
                                                np.array([ctx]), 0.8, bs, causal=True)
        vis = [ctx - rows + i + 1 for i in range(rows)]
        want = _brute(qq.tolist(), kc.tolist(), vc.tolist(), table, ctx, 0.8, bs, group, vis)
        np.testing.assert_allclose(out, want, atol=1e-12, rtol=0)


def check_permutation_invariance(mod, seed=5):
    q, kc, vc, tables, ctx = _random_case(seed)
    bs = kc.shape[1]
    out = mod.paged_attention_decode(q, kc, vc, tables, ctx, 0.5, bs)
    pi = np.random.default_rng(seed + 1).permutation(kc.shape[0])
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    out2 = mod.paged_attention_decode(q, kc2, vc2, pi[tables], ctx, 0.5, bs)
    np.testing.assert_array_equal(out, out2)


def check_closed_forms(mod, seed=7):
    q, kc, vc, tables, ctx = _random_case(seed)
    bs = kc.shape[1]
    hq, hkv = q.shape[1], kc.shape[2]
    group = hq // hkv
    # context 1: the single V row, exactly
    ctx1 = np.ones_like(ctx)
    out = mod.paged_attention_decode(q, kc, vc, tables, ctx1, 0.9, bs)
    for s in range(len(ctx)):
        for h in range(hq):
            np.testing.assert_array_equal(out[s, h], vc[tables[s, 0], 0, h // group])
    # scale 0, and identical keys: the mean of the visible V rows
    kc_same = np.broadcast_to(kc[:1, :1], kc.shape).copy()
    for keys, scale in ((kc, 0.0), (kc_same, 1.3)):
        out = mod.paged_attention_decode(q, keys, vc, tables, ctx, scale, bs)
        for s in range(len(ctx)):
            pos = np.arange(ctx[s])
            rows = vc[tables[s][pos // bs], pos % bs]          # [ctx, Hkv, D]
            mean = rows.mean(axis=0)
            for h in range(hq):
                np.testing.assert_allclose(out[s, h], mean[h // group], atol=1e-12, rtol=0)


def check_prefill_matches_decode(mod, seed=11):
    q, kc, vc, tables, ctx = _random_case(seed)
    bs = kc.shape[1]
    # a chunk of L rows: row i equals decode with context prior + i + 1
    for s in range(len(ctx)):
        rows = min(5, int(ctx[s]))
        rng = np.random.default_rng(seed + s)
        qq = rng.standard_normal((rows,) + q.shape[1:])
        out = mod.paged_attention_prefill_chunk(qq, kc, vc, tables[s:s + 1],
                                                np.array([0, rows]), ctx[s:s + 1], 0.6, bs)
        prior = int(ctx[s]) - rows
        for i in range(rows):
            dec = mod.paged_attention_decode(qq[i:i + 1], kc, vc, tables[s:s + 1],
                                             np.array([prior + i + 1]), 0.6, bs)
            np.testing.assert_allclose(out[i], dec[0], atol=1e-13, rtol=0)


def check_store(mod, seed=13):
    rng = np.random.default_rng(seed)
    nb, bs, hkv, d = 6, 4, 2, 3
    sentinel = rng.standard_normal((nb, bs, hkv, d)).astype(np.float32)
    k = rng.standard_normal((5, hkv, d)).astype(np.float32)
    v = rng.standard_normal((5, hkv, d)).astype(np.float32)
    slots = np.array([23, -1, 0, 9, -5])
    kc, vc = mod.kv_cache_store(k, v, sentinel, sentinel, slots, bs)
    touched = np.zeros((nb, bs), dtype=bool)
    for t, s in enumerate(slots):
        if s >= 0:
            np.testing.assert_array_equal(kc[s // bs, s % bs], k[t])
            np.testing.assert_array_equal(vc[s // bs, s % bs], v[t])
            touched[s // bs, s % bs] = True
    np.testing.assert_array_equal(kc[~touched], sentinel[~touched])
    np.testing.assert_array_equal(vc[~touched], sentinel[~touched])
    # bf16 bit patterns pass through untouched, NaN payloads included
    bits = rng.integers(0, 1 << 16, size=(nb, bs, hkv, d)).astype(np.uint16)
    kb = rng.integers(0, 1 << 16, size=(5, hkv, d)).astype(np.uint16)
    kc, _ = mod.kv_cache_store(kb, kb, bits, bits, slots, bs)
    assert kc[23 // bs, 23 % bs].tobytes() == kb[0].tobytes()
    assert kc[0, 0].tobytes() == kb[2].tobytes()


def check_poison_does_not_leak(mod, seed=17):
    q, kc, vc, tables, ctx = _random_case(seed)
    bs = kc.shape[1]
    kp, vp = kc.copy(), vc.copy()
    live = np.zeros(kc.shape[:2], dtype=bool)
    for s in range(len(ctx)):
        pos = np.arange(ctx[s])
        live[tables[s][pos // bs], pos % bs] = True
    kp[~live] = np.nan
    vp[~live] = np.nan
    out = mod.paged_attention_decode(q, kp, vp, tables, ctx, 0.5, bs)
    ref = mod.paged_attention_decode(q, kc, vc, tables, ctx, 0.5, bs)
    assert np.isfinite(out).all()
    np.testing.assert_array_equal(out, ref)


CHECKS = [check_golden, check_sdpa_decode, check_sdpa_prefill,
          lambda m: check_sdpa_prefill(m, causal=False), check_brute_force,
          check_permutation_invariance, check_closed_forms,
          check_prefill_matches_decode, check_store, check_poison_does_not_leak]


# ----------------------------------------------------------------------------
# tests on the oracle itself
# ----------------------------------------------------------------------------

def test_golden():
    check_golden(ORACLE)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_sdpa_decode(seed):
    check_sdpa_decode(ORACLE, seed)


def test_sdpa_decode_no_gqa_and_wide_groups():
    check_sdpa_decode(ORACLE, 4, hq=4, hkv=4)
    check_sdpa_decode(ORACLE, 5, hq=16, hkv=2, bs=16, max_ctx=70)


@pytest.mark.parametrize("causal", [True, False])
def test_sdpa_prefill(causal):
    check_sdpa_prefill(ORACLE, causal=causal)


def test_brute_force():
    check_brute_force(ORACLE)


def test_permutation_invariance():
    check_permutation_invariance(ORACLE)


def test_closed_forms():
    check_closed_forms(ORACLE)


def test_prefill_matches_decode():
    check_prefill_matches_decode(ORACLE)


def test_store():
    check_store(ORACLE)


def test_store_rejects_duplicates_and_out_of_pool():
    z = np.zeros((2, 2, 1, 1))
    k = np.ones((2, 1, 1))
    with pytest.raises(ValueError):
        ORACLE.kv_cache_store(k, k, z, z, np.array([1, 1]), 2)
    with pytest.raises(IndexError):
        ORACLE.kv_cache_store(k, k, z, z, np.array([0, 4]), 2)


def test_poison_does_not_leak():
    check_poison_does_not_leak(ORACLE)


def test_bf16_inputs_upcast_exactly():
    """bf16 caches given as bit patterns equal the same values given in fp64."""
    q, kc, vc, tables, ctx = _random_case(19)
    bs = kc.shape[1]
    to_bits = lambda x: (torch.as_tensor(x, dtype=torch.float32).to(torch.bfloat16)
                         .view(torch.int16).numpy().view(np.uint16))
    qb, kb, vb = to_bits(q), to_bits(kc), to_bits(vc)
    out_bits = ORACLE.paged_attention_decode(qb, kb, vb, tables, ctx, 0.5, bs)
    as64 = lambda b: torch.as_tensor(b.view(np.int16)).view(torch.bfloat16).double().numpy()
    out_f64 = ORACLE.paged_attention_decode(as64(qb), as64(kb), as64(vb), tables, ctx, 0.5, bs)
    np.testing.assert_array_equal(out_bits, out_f64)


def test_package_exports():
    for name in ("kv_cache_store", "paged_attention_decode", "paged_attention_prefill_chunk",
                 "gather_context", "to_f64"):
        assert callable(getattr(oracle, name))
