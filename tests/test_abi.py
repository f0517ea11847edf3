"""The C-ABI library loads, exports every symbol include/pkv.h declares, and
rejects invalid arguments on the host before launching anything (CPU only:
no call here reaches a kernel)."""

import ctypes
import os
import re

import pytest

import paged_attention_kv_store_amd as pkv
from paged_attention_kv_store_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkv.h")

needs_lib = pytest.mark.skipif(not os.path.exists(pkv.library_path()),
                               reason="libpkv.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_symbols() == binding.exported_symbols()


@needs_lib
def test_library_exports_every_declared_symbol():
    lib = pkv.lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.pkv_version() >= 100


def _decode(lib, **over):
    args = dict(out=1024, q=1024, k=1024, v=1024, bt=1024, cl=1024, S=4, MB=16, max_ctx=256,
                NB=64, bs=16, Hq=8, Hkv=4, D=64, scale=0.125, part=0, ws=None, ws_bytes=0,
                dtype=0, algo=0, stream=None)
    args.update(over)
    a = args
    return lib.pkv_paged_attention_decode(a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"],
                                          a["S"], a["MB"], a["max_ctx"], a["NB"], a["bs"],
                                          a["Hq"], a["Hkv"], a["D"], a["scale"], a["part"],
                                          a["ws"], a["ws_bytes"], a["dtype"], a["algo"],
                                          a["stream"])


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(S=-1), binding.PKV_EINVAL),
    (dict(Hq=6, Hkv=4), binding.PKV_EINVAL),
    (dict(Hkv=0), binding.PKV_EINVAL),
    (dict(D=96), binding.PKV_EUNSUPPORTED),
    (dict(bs=8), binding.PKV_EUNSUPPORTED),
    (dict(bs=512), binding.PKV_EUNSUPPORTED),
    (dict(dtype=7), binding.PKV_EINVAL),
    (dict(max_ctx=257), binding.PKV_EINVAL),
    (dict(part=24), binding.PKV_EINVAL),
    (dict(part=-16), binding.PKV_EINVAL),
    (dict(part=64), binding.PKV_EWORKSPACE),
    (dict(part=64, ws=1024, ws_bytes=100), binding.PKV_EWORKSPACE),
    (dict(algo=2, dtype=0), binding.PKV_EUNSUPPORTED),
    (dict(algo=9), binding.PKV_EINVAL),
    (dict(Hq=36, Hkv=2, algo=1, dtype=1), binding.PKV_EUNSUPPORTED),
    (dict(Hq=34, Hkv=2, algo=2, dtype=1), binding.PKV_EUNSUPPORTED),
    (dict(q=None), binding.PKV_EINVAL),
    (dict(q=1028), binding.PKV_EINVAL),
    (dict(scale=float("nan")), binding.PKV_EINVAL),
    (dict(S=70000), binding.PKV_EUNSUPPORTED),
    (dict(S=9000, Hq=64, Hkv=8, part=16, max_ctx=256, MB=16), binding.PKV_EUNSUPPORTED),   # 72000 pairs
    (dict(part=-1), binding.PKV_EUNSUPPORTED),                       # balanced needs bf16
    (dict(part=-1, dtype=1, algo=1), binding.PKV_EUNSUPPORTED),      # ... and the MFMA kernel
    (dict(part=-1, dtype=1, S=9000), binding.PKV_EUNSUPPORTED),      # at most 8192 sequences
    (dict(part=-1, dtype=1), binding.PKV_EWORKSPACE),
    (dict(part=-1, dtype=1, ws=1040, ws_bytes=1 << 30), binding.PKV_EINVAL),   # 256-byte alignment
    (dict(part=-1, dtype=1, out=1032), binding.PKV_EINVAL),          # out 16-byte aligned
    (dict(part=-4), binding.PKV_EINVAL),
    (dict(part=-2), binding.PKV_EUNSUPPORTED),                       # planned needs the MFMA kernel
    (dict(part=-2, dtype=1), binding.PKV_EWORKSPACE),                # ... and its plan
    (dict(part=-2, dtype=1, ws=1024, ws_bytes=4 * 32 - 1), binding.PKV_EWORKSPACE),
    (dict(part=-2, dtype=1, ws=1032, ws_bytes=1 << 20), binding.PKV_EINVAL),   # 16-byte alignment
])
def test_decode_rejects(over, code):
    lib = pkv.lib()
    assert _decode(lib, **over) == code
    assert lib.pkv_last_error()


@needs_lib
def test_decode_empty_batch_is_a_no_op():
    assert _decode(pkv.lib(), S=0, out=None, q=None) == binding.PKV_OK


def _plan(lib, **over):
    a = dict(plan=1024, plan_bytes=1 << 20, bt=1024, cl=1024, S=4, MB=16, max_ctx=256, bs=16, stream=None)
    a.update(over)
    return lib.pkv_decode_plan(a["plan"], a["plan_bytes"], a["bt"], a["cl"], a["S"], a["MB"], a["max_ctx"],
                               a["bs"], a["stream"])


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(S=-1), binding.PKV_EINVAL),
    (dict(S=70000), binding.PKV_EINVAL),
    (dict(bs=8), binding.PKV_EUNSUPPORTED),
    (dict(bs=512), binding.PKV_EUNSUPPORTED),
    (dict(MB=0), binding.PKV_EINVAL),
    (dict(max_ctx=257), binding.PKV_EINVAL),
    (dict(plan=None), binding.PKV_EINVAL),
    (dict(cl=None), binding.PKV_EINVAL),
    (dict(plan_bytes=4 * 32 - 4), binding.PKV_EWORKSPACE),
    (dict(plan=1032), binding.PKV_EINVAL),
    (dict(cl=1026), binding.PKV_EINVAL),
])
def test_plan_rejects(over, code):
    lib = pkv.lib()
    assert _plan(lib, **over) == code
    assert lib.pkv_last_error()


@needs_lib
def test_plan_empty_batch_is_a_no_op():
    assert _plan(pkv.lib(), S=0, plan=None, bt=None, cl=None) == binding.PKV_OK


@needs_lib
def test_plan_size():
    lib = pkv.lib()
    # eight int32 per sequence: sequence, length, four first blocks, two spare
    assert pkv.decode_plan_size(60) == 60 * 32
    assert lib.pkv_decode_plan_size(0) == 0
    assert pkv.decode_workspace_size(60, 16, 8, 128, 1024, "planned") == 60 * 32
    assert pkv.decode_workspace_size(60, 16, 8, 128, 1024, binding.PARTITION_PLANNED) == 60 * 32


@needs_lib
def test_workspace_size():
    lib = pkv.lib()
    # 32 seqs x 32 heads x ceil(32768/512)=64 partitions x (128 + 2) floats
    # 65536 counters first, then partials (m, l, o) per (seq, q-head, partition)
    assert pkv.decode_workspace_size(32, 32, 8, 128, 32768, 512) == 65536 * 4 + 32 * 32 * 64 * 130 * 4
    assert pkv.decode_workspace_size(32, 32, 8, 128, 512, 512) == 0      # one partition
    assert pkv.decode_workspace_size(32, 32, 8, 128, 513, 512) == 65536 * 4 + 32 * 32 * 2 * 130 * 4
    assert lib.pkv_decode_workspace_size(4, 8, 4, 64, 100, 0) == 0
    assert lib.pkv_decode_workspace_size(4, 8, 3, 64, 100, 0) == 0       # Hq not a multiple of Hkv
    # work-balanced: the 256 KiB counter block that split-K uses too (its first
    # 4096 counters), then 2 pieces per wave of the largest grid (4096 waves),
    # each G*D + 2G floats rounded up to 4; no dependence on num_seqs or
    # max_context_len
    counters = 65536 * 4
    assert pkv.decode_workspace_size(32, 32, 8, 128, 4096, "balanced") == \
        counters + 2 * 4096 * (4 * 128 + 8) * 4
    assert pkv.decode_workspace_size(60, 16, 8, 128, 1024, -1) == counters + 2 * 4096 * 260 * 4
    assert pkv.decode_workspace_size(7000, 16, 8, 128, 9, -1) == counters + 2 * 4096 * 260 * 4
    assert pkv.decode_workspace_size(3, 3, 1, 64, 10, -1) == counters + 2 * 4096 * 200 * 4


def _store(lib, **over):
    a = dict(k=1024, v=1024, kc=1024, vc=1024, slots=1024, T=4, NB=64, bs=16, Hkv=4, D=64,
             dtype=0, stream=None)
    a.update(over)
    return lib.pkv_kv_cache_store(a["k"], a["v"], a["kc"], a["vc"], a["slots"], a["T"], a["NB"],
                                  a["bs"], a["Hkv"], a["D"], a["dtype"], a["stream"])


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(T=-1), binding.PKV_EINVAL),
    (dict(NB=0), binding.PKV_EINVAL),
    (dict(dtype=3), binding.PKV_EINVAL),
    (dict(Hkv=1, D=2, dtype=1), binding.PKV_EUNSUPPORTED),
    (dict(k=None), binding.PKV_EINVAL),
    (dict(kc=1032), binding.PKV_EINVAL),
])
def test_store_rejects(over, code):
    lib = pkv.lib()
    assert _store(lib, **over) == code
    assert lib.pkv_last_error()


@needs_lib
def test_store_zero_tokens_is_a_no_op():
    assert _store(pkv.lib(), T=0, k=None, v=None) == binding.PKV_OK


def _prefill(lib, **over):
    a = dict(out=1024, q=1024, k=1024, v=1024, bt=1024, cu=1024, cl=1024, S=2, Tq=64, maxq=32,
             MB=16, max_ctx=256, NB=64, bs=16, Hq=32, Hkv=8, D=128, scale=0.08, causal=1,
             dtype=1, stream=None)
    a.update(over)
    return lib.pkv_paged_attention_prefill_chunk(a["out"], a["q"], a["k"], a["v"], a["bt"],
                                                 a["cu"], a["cl"], a["S"], a["Tq"], a["maxq"],
                                                 a["MB"], a["max_ctx"], a["NB"], a["bs"],
                                                 a["Hq"], a["Hkv"], a["D"], a["scale"],
                                                 a["causal"], a["dtype"], a["stream"])


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(S=-1), binding.PKV_EINVAL),
    (dict(dtype=0), binding.PKV_EUNSUPPORTED),
    (dict(D=64), binding.PKV_EUNSUPPORTED),
    (dict(Hq=24, Hkv=8), binding.PKV_EUNSUPPORTED),
    (dict(Hq=30, Hkv=8), binding.PKV_EINVAL),
    (dict(max_ctx=300), binding.PKV_EINVAL),
    (dict(maxq=300, max_ctx=256), binding.PKV_EINVAL),
    (dict(cu=None), binding.PKV_EINVAL),
    (dict(out=1030), binding.PKV_EINVAL),
    (dict(NB=1 << 28, bs=32), binding.PKV_EUNSUPPORTED),        # 2^33 pool rows
])
def test_prefill_rejects(over, code):
    lib = pkv.lib()
    assert _prefill(lib, **over) == code
    assert lib.pkv_last_error()


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        binding.lib()


@needs_lib
def test_fused_store_rejects_missing_rows():
    lib = pkv.lib()
    rc = lib.pkv_paged_attention_decode_store(1024, 1024, 1024, 1024, 1024, 1024, None, 1024, 1024,
                                              4, 16, 256, 64, 16, 8, 4, 64, 0.125, 0, None, 0, 0, 0,
                                              None)
    assert rc == binding.PKV_EINVAL and b"null" in lib.pkv_last_error()
    rc = lib.pkv_paged_attention_decode_store(1024, 1024, 1024, 1024, 1024, 1024, 1032, 1024, 1024,
                                              4, 16, 256, 64, 16, 8, 4, 64, 0.125, 0, None, 0, 0, 0,
                                              None)
    assert rc == binding.PKV_EINVAL


def _shared(lib, **over):
    a = dict(out=1024, q=1024, k=1024, v=1024, bt=1024, cl=1024, gs=1024, gp=1024, NG=2, GS=4, PL=64,
             S=8, MB=16, max_ctx=256, NB=64, bs=16, Hq=32, Hkv=8, D=128, scale=0.08, ws=1024,
             ws_bytes=1 << 20, stream=None)
    a.update(over)
    return lib.pkv_paged_attention_decode_shared_prefix(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["gs"], a["gp"], a["NG"], a["GS"], a["PL"],
        a["S"], a["MB"], a["max_ctx"], a["NB"], a["bs"], a["Hq"], a["Hkv"], a["D"], a["scale"], a["ws"],
        a["ws_bytes"], a["stream"])


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(S=-1), binding.PKV_EINVAL),
    (dict(D=64), binding.PKV_EUNSUPPORTED),
    (dict(Hq=24, Hkv=8), binding.PKV_EUNSUPPORTED),
    (dict(bs=48), binding.PKV_EUNSUPPORTED),
    (dict(PL=300), binding.PKV_EINVAL),
    (dict(NG=0), binding.PKV_EINVAL),
    (dict(gs=None), binding.PKV_EINVAL),
    (dict(ws_bytes=100), binding.PKV_EWORKSPACE),
    (dict(ws=1032), binding.PKV_EINVAL),
])
def test_shared_prefix_rejects(over, code):
    lib = pkv.lib()
    assert _shared(lib, **over) == code
    assert lib.pkv_last_error()


@needs_lib
def test_shared_prefix_workspace_size():
    assert pkv.lib().pkv_decode_shared_prefix_workspace_size(8, 32, 128) == 8 * 32 * 130 * 4 + 8 * 4


def test_static_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define PKV_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == binding.STATIC_SCRATCH_BYTES


@needs_lib
@pytest.mark.parametrize("over,code", [
    (dict(S=4096, MB=2048, max_ctx=32768, Hq=32, Hkv=8, D=128, part=16, dtype=1, algo=2),
     binding.PKV_EWORKSPACE),                       # split-K partials beyond the static scratch
    (dict(part=-2), binding.PKV_EINVAL),            # the planned decode reads a caller's plan
    (dict(S=-1, part=64), binding.PKV_EINVAL),
    (dict(Hq=6, Hkv=4, part=64), binding.PKV_EINVAL),
])
def test_static_decode_rejects_on_the_host(over, code):
    """The entry point without a workspace rejects these before any launch
    (no device is touched: the pointers are placeholders)."""
    a = dict(out=1024, q=1024, k=1024, v=1024, bt=1024, cl=1024, S=4, MB=16, max_ctx=256, NB=64, bs=16,
             Hq=8, Hkv=4, D=64, scale=0.125, part=0, dtype=0, algo=0, stream=None)
    a.update(over)
    rc = pkv.lib().pkv_paged_attention_decode_static(
        a["out"], a["q"], a["k"], a["v"], a["bt"], a["cl"], a["S"], a["MB"], a["max_ctx"], a["NB"], a["bs"],
        a["Hq"], a["Hkv"], a["D"], a["scale"], a["part"], a["dtype"], a["algo"], a["stream"])
    assert rc == code, pkv.lib().pkv_last_error()
    if code == binding.PKV_EWORKSPACE:
        assert b"static scratch" in pkv.lib().pkv_last_error()


@needs_lib
def test_static_decode_empty_batch_is_a_no_op():
    rc = pkv.lib().pkv_paged_attention_decode_static(None, None, None, None, None, None, 0, 16, 0, 64, 16, 8, 4,
                                                     64, 0.125, 64, 0, 0, None)
    assert rc == binding.PKV_OK


@needs_lib
def test_auto_partition_rule():
    """PKV_PARTITION_AUTO: one pass when the items fill two workgroups per
    compute unit or contexts are short; the work-balanced decode from half a
    workgroup per unit; below that split-K at the power of two in [512, 2048]
    nearest above one partition per unit. (Without a GPU the library assumes
    256 compute units.)"""
    cus = 256
    auto = pkv.decode_auto_partition
    bal = binding.PARTITION_BALANCED
    assert auto(60, 8, 1024) == 0                 # short contexts
    assert auto(256, 8, 4096) == 0                # 2048 items
    assert auto(64, 8, 32768) == 0                # 512 items = 2 per unit
    assert auto(32, 8, 32768) == bal              # 256 items: one per unit
    assert auto(16, 8, 8192) == bal               # 128 items: half a workgroup per unit
    assert auto(8, 8, 8192) == 2048               # 64 items x 8192 / 256 units = 2048 tokens
    assert auto(1, 8, 32768) == 1024              # 8 x 32768 / 256
    assert auto(1, 8, 4096) == 512                # the floor
    assert auto(1, 1, 3000) == 512
    assert auto(2, 8, 32768) == 2048              # 16 x 32768 / 256 = 2048
    assert auto(4, 8, 32768) == 2048              # the ceiling (4096 would be one per unit)
    # (recompute the rule here for more sizes)
    for s, hkv, ctx in [(32, 8, 32768), (1, 8, 4096), (4, 8, 8192), (2, 4, 2100), (100, 2, 5000),
                        (15, 8, 9000), (17, 8, 3000), (3, 2, 40000)]:
        items = s * hkv
        if items >= 2 * cus or ctx <= 2048:
            want = 0
        elif 2 * items >= cus:
            want = bal
        else:
            part = 512
            while part < 2048 and part < -(-items * ctx // cus):
                part *= 2
            want = part if -(-ctx // part) > 1 else 0
        assert auto(s, hkv, ctx) == want, (s, hkv, ctx)
    assert pkv.lib().pkv_decode_auto_partition(0, 8, 100) == 0
    # the workspace of "auto" covers the choice and, for a work-balanced
    # choice, the split-K fallback of calls that cannot take it
    assert pkv.decode_workspace_size(8, 32, 8, 128, 8192, "auto") == \
        pkv.decode_workspace_size(8, 32, 8, 128, 8192, 2048)
    both = max(pkv.decode_workspace_size(32, 32, 8, 128, 32768, "balanced"),
               pkv.decode_workspace_size(32, 32, 8, 128, 32768, 2048))
    assert pkv.decode_workspace_size(32, 32, 8, 128, 32768, "auto") == both
    assert pkv.decode_workspace_size(60, 16, 8, 128, 1024, "auto") == 0


@needs_lib
def test_workspace_init_rejects():
    lib = pkv.lib()
    assert lib.pkv_decode_workspace_init(None, 0, None) == binding.PKV_OK
    assert lib.pkv_decode_workspace_init(None, 64, None) == binding.PKV_EINVAL
    assert lib.pkv_decode_workspace_init(1026, 64, None) == binding.PKV_EINVAL


@needs_lib
def test_checks_reject_on_the_host():
    lib = pkv.lib()
    E = binding.PKV_EINVAL
    # block_tables, context_lens, cu, S, MB, max_ctx, total_q, max_q_len, NB, bs, report, stream
    assert lib.pkv_check_paged_inputs(1024, 1024, None, -1, 16, 256, 0, 0, 64, 16, 1024, None) == E
    assert lib.pkv_check_paged_inputs(1024, 1024, None, 4, 16, 257, 0, 0, 64, 16, 1024, None) == E
    assert lib.pkv_check_paged_inputs(1024, 1024, None, 4, 16, 256, 0, 0, 0, 16, 1024, None) == E
    assert lib.pkv_check_paged_inputs(1024, 1024, None, 4, 16, 256, 0, 0, 64, 16, None, None) == E
    assert lib.pkv_check_paged_inputs(None, 1024, None, 4, 16, 256, 0, 0, 64, 16, 1024, None) == E
    assert lib.pkv_check_paged_inputs(1024, 1026, None, 4, 16, 256, 0, 0, 64, 16, 1024, None) == E
    assert lib.pkv_check_slots_workspace_size(64, 16) == 2 * 32 * 4
    assert lib.pkv_check_slots_workspace_size(3, 16) == 2 * 2 * 4
    assert lib.pkv_check_slots_workspace_size(0, 16) == 0
    # slot_mapping, T, NB, bs, workspace, ws_bytes, report, stream
    assert lib.pkv_check_slots(1024, -1, 64, 16, 1024, 256, 1024, None) == E
    assert lib.pkv_check_slots(1024, 4, 64, 16, 1024, 255, 1024, None) == binding.PKV_EWORKSPACE
    assert lib.pkv_check_slots(1024, 4, 64, 16, None, 256, 1024, None) == binding.PKV_EWORKSPACE
    assert lib.pkv_check_slots(1024, 4, 64, 16, 1024, 256, None, None) == E
    assert lib.pkv_check_slots(None, 4, 64, 16, 1024, 256, 1024, None) == E
