"""ctypes binding of libpkv.so (include/pkv.h), with the same entry-point names.

Argument marshalling only: shape and dtype checks on torch tensors, then the
raw device pointers, sizes and the current HIP stream go to the C ABI. Every
step of the computation runs in the library's HIP kernels. torch supplies
device memory and streams; nothing here computes on the data. If the library
has not been built, every call raises.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
_lock = threading.Lock()
_lib = None

PKV_OK, PKV_EINVAL, PKV_EUNSUPPORTED, PKV_EWORKSPACE, PKV_EHIP = 0, -1, -2, -3, -4
PKV_F32, PKV_BF16 = 0, 1
DECODE_ALGOS = {"auto": 0, "valu": 1, "mfma": 2}
PARTITION_BALANCED = -1      # partition_size selecting the work-balanced decode
PARTITION_PLANNED = -2       # partition_size selecting the planned decode (workspace = the plan)
PARTITION_AUTO = -3          # partition_size chosen by the library from the host-side sizes
STATIC_SCRATCH_BYTES = 64 << 20   # PKV_STATIC_SCRATCH_BYTES: the library's per-device decode scratch

_i32 = ctypes.c_int32
_vp = ctypes.c_void_p
_SIGNATURES = {
    "pkv_version": ([], ctypes.c_int),
    "pkv_last_error": ([], ctypes.c_char_p),
    "pkv_kv_cache_store": ([_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _vp],
                           ctypes.c_int),
    "pkv_decode_workspace_size": ([_i32, _i32, _i32, _i32, _i32, _i32], ctypes.c_size_t),
    "pkv_decode_plan_size": ([_i32], ctypes.c_size_t),
    "pkv_decode_workspace_init": ([_vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "pkv_decode_auto_partition": ([_i32, _i32, _i32], _i32),
    "pkv_check_paged_inputs": ([_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp], ctypes.c_int),
    "pkv_check_slots_workspace_size": ([_i32, _i32], ctypes.c_size_t),
    "pkv_check_slots": ([_vp, _i32, _i32, _i32, _vp, ctypes.c_size_t, _vp, _vp], ctypes.c_int),
    "pkv_decode_plan": ([_vp, ctypes.c_size_t, _vp, _vp, _i32, _i32, _i32, _i32, _vp], ctypes.c_int),
    "pkv_paged_attention_decode": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                    _i32, _i32, _i32, ctypes.c_float, _i32, _vp, ctypes.c_size_t,
                                    ctypes.c_int, _i32, _vp], ctypes.c_int),
    "pkv_paged_attention_decode_store": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                          _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_float, _i32,
                                          _vp, ctypes.c_size_t, ctypes.c_int, _i32, _vp], ctypes.c_int),
    "pkv_paged_attention_decode_static": ([_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                           _i32, _i32, _i32, ctypes.c_float, _i32, ctypes.c_int, _i32, _vp],
                                          ctypes.c_int),
    "pkv_kv_cache_store_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                ctypes.c_int, _vp], ctypes.c_int),
    "pkv_paged_attention_decode_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32,
                                        _i32, _i32, _i32, _i32, ctypes.c_float, _i32, _vp,
                                        ctypes.c_size_t, _vp], ctypes.c_int),
    "pkv_paged_attention_decode_store_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                              ctypes.c_float, _i32, _vp, ctypes.c_size_t, _vp],
                                             ctypes.c_int),
    "pkv_decode_shared_prefix_workspace_size": ([_i32, _i32, _i32], ctypes.c_size_t),
    "pkv_paged_attention_decode_shared_prefix": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                                  _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                  ctypes.c_float, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "pkv_paged_attention_prefill_chunk": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32,
                                           _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                           ctypes.c_float, _i32, ctypes.c_int, _vp], ctypes.c_int),
    "pkv_paged_attention_prefill_chunk_fp8": ([_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32,
                                               _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                               ctypes.c_float, _i32, _vp], ctypes.c_int),
}


class PkvError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"pkv status {status}: {message}")
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def lib():
    """Load libpkv.so once; raise if it is missing (no fallback exists)."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise RuntimeError(
                        f"{_LIB_PATH} is not built; run paged_attention_kv_store_amd/build.py")
                handle = ctypes.CDLL(_LIB_PATH)
                for name, (args, res) in _SIGNATURES.items():
                    fn = getattr(handle, name)
                    fn.argtypes = args
                    fn.restype = res
                _lib = handle
    return _lib


def exported_symbols():
    return sorted(_SIGNATURES)


def _check(status):
    if status != PKV_OK:
        raise PkvError(status, lib().pkv_last_error().decode(errors="replace"))


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return PKV_F32
    if t.dtype == torch.bfloat16:
        return PKV_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _dev(*ts):
    for t in ts:
        _need(t.is_cuda, "tensors must be on the GPU")
        _need(t.is_contiguous(), "tensors must be contiguous")


def kv_cache_store(k, v, k_cache, v_cache, slot_mapping, stream=None):
    """Copy k[t], v[t] into the cache row named by slot_mapping[t] (in place)."""
    _dev(k, v, k_cache, v_cache, slot_mapping)
    _need(k.dim() == 3 and v.shape == k.shape, "k, v must be [T, Hkv, D]")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
    _need(k_cache.shape[2:] == k.shape[1:], "cache and new rows disagree on heads/dims")
    _need(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (k.shape[0],),
          "slot_mapping must be int32 [T]")
    _need(k.dtype == v.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    nb, bs, hkv, d = k_cache.shape
    _check(lib().pkv_kv_cache_store(_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(slot_mapping), k.shape[0], nb, bs, hkv, d,
                                    _dtype_code(k), _stream(stream)))


def _partition(partition_size):
    if partition_size == "balanced":
        return PARTITION_BALANCED
    if partition_size == "planned":
        return PARTITION_PLANNED
    if partition_size == "auto":
        return PARTITION_AUTO
    return int(partition_size)


def decode_plan_size(num_seqs):
    return int(lib().pkv_decode_plan_size(num_seqs))


def new_decode_plan(num_seqs, device):
    """A device buffer for decode_plan (uint8, pkv_decode_plan_size bytes)."""
    return torch.empty(max(decode_plan_size(num_seqs), 16), dtype=torch.uint8, device=device)


class DecodePlanLaunch:
    """decode_plan with fixed tensors: one C call per launch."""

    def __init__(self, plan, block_tables, context_lens, max_context_len, block_size):
        _dev(plan, block_tables, context_lens)
        _need(plan.dtype == torch.uint8 and plan.is_contiguous(), "plan must be a contiguous uint8 tensor")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2, "block_tables must be int32 [S, MB]")
        _need(context_lens.dtype == torch.int32 and context_lens.shape == (block_tables.shape[0],),
              "context_lens must be int32 [S]")
        _need(block_tables.is_contiguous() and context_lens.is_contiguous(), "index arrays must be contiguous")
        self._keep = (plan, block_tables, context_lens)
        self._args = (_ptr(plan), plan.numel(), _ptr(block_tables), _ptr(context_lens),
                      block_tables.shape[0], block_tables.shape[1], int(max_context_len), int(block_size))

    def __call__(self, stream=None):
        _check(lib().pkv_decode_plan(*self._args, _stream(stream)))


def decode_plan(plan, block_tables, context_lens, max_context_len, block_size, stream=None):
    """Order the step's sequences by size, largest first, into `plan` (see
    new_decode_plan); decode calls with partition_size="planned" and
    workspace=plan then use it, for as long as context_lens and block_tables
    stay as they were."""
    DecodePlanLaunch(plan, block_tables, context_lens, max_context_len, block_size)(stream)
    return plan


def decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len,
                          partition_size):
    return int(lib().pkv_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               max_context_len, _partition(partition_size)))


def decode_workspace_init(workspace, stream=None):
    """Zero the arrival counters of a decode workspace (a uint8 device
    tensor) with a kernel on the stream; the rest needs no initial contents."""
    _dev(workspace)
    _check(lib().pkv_decode_workspace_init(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                           _stream(stream)))
    return workspace


def decode_auto_partition(num_seqs, num_kv_heads, max_context_len):
    """The partition_size that partition_size="auto" resolves to on the current device."""
    return int(lib().pkv_decode_auto_partition(num_seqs, num_kv_heads, int(max_context_len)))


def new_decode_workspace(nbytes, device, stream=None):
    """A decode workspace of nbytes with its counters cleared (torch.empty plus
    pkv_decode_workspace_init: one small kernel, no memset)."""
    ws = torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)
    return decode_workspace_init(ws, stream)


# Workspaces of the one-call functions (paged_attention_decode and friends
# without a workspace argument): one per (device, stream), grown when a call
# needs more. Calls on one stream are ordered, so they may share it; every
# call leaves its counters zero.
_WS_CACHE = {}


def _cached_workspace(need, device, stream):
    key = (torch.device(device).index, _stream(stream).value)
    ws = _WS_CACHE.get(key)
    if ws is None or ws.numel() < need:
        ws = new_decode_workspace(need, device, stream)
        _WS_CACHE[key] = ws
    return ws


def _decode_workspace(workspace, s, hq, hkv, d, max_context_len, partition, device, stream=None,
                      cached=False):
    """The caller's workspace, or one for the call when it needs it: the
    one-call functions reuse a cached workspace per (device, stream), the
    prepared launches own theirs; both are cleared once when made."""
    need = decode_workspace_size(s, hq, hkv, d, max_context_len, partition) if partition else 0
    _need(partition != PARTITION_PLANNED or workspace is not None,
          "the planned decode takes its plan (written by decode_plan) as workspace")
    if need and workspace is None:
        workspace = _cached_workspace(need, device, stream) if cached else new_decode_workspace(need, device, stream)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return workspace, ws_bytes


def paged_attention_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                           max_context_len, partition_size=0, workspace=None, algo="auto",
                           stream=None):
    """One query row per sequence over its paged context; writes out [S, Hq, D].

    max_context_len is a host-side bound on context_lens (it sizes the grid).
    partition_size: 0 (one pass per sequence and kv-head), a positive multiple
    of 16 (split-K), "balanced" / PARTITION_BALANCED (work-balanced decode),
    "planned" / PARTITION_PLANNED (one pass in the order of the plan passed as
    `workspace`, written by decode_plan), or "auto" / PARTITION_AUTO.
    The workspace those need is taken from `workspace` (a uint8 device tensor
    whose first 256 KiB, the arrival counters, are zero before its first
    split-K or work-balanced use: new_decode_workspace makes one so) or, when
    omitted, from a workspace cached per (device, stream) and grown as calls
    need, which split-K and work-balanced calls share in any order.
    """
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [S, Hq, D]")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
          "context_lens must be int32 [S]")
    _need(k_cache.shape[3] == q.shape[2], "head_dim mismatch")
    s, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    part = _partition(partition_size)
    workspace, ws_bytes = _decode_workspace(workspace, s, hq, hkv, d, max_context_len, part, q.device, stream,
                                            cached=True)
    _check(lib().pkv_paged_attention_decode(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        s, block_tables.shape[1], int(max_context_len), nb, bs, hq, hkv, d, float(scale),
        part, _ptr(workspace), ws_bytes, _dtype_code(q), DECODE_ALGOS[algo],
        _stream(stream)))
    return out


def paged_attention_decode_static(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                                  max_context_len, partition_size=0, algo="auto", stream=None):
    """paged_attention_decode without a workspace: split-K and work-balanced
    modes use the library's own per-device scratch (PKV_STATIC_SCRATCH_BYTES),
    so nothing is allocated. Calls that overlap in time on one device race."""
    _dev(out, q, k_cache, v_cache, block_tables, context_lens)
    _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [S, Hq, D]")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
          and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, MB]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
          "context_lens must be int32 [S]")
    _need(k_cache.shape[3] == q.shape[2], "head_dim mismatch")
    s, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    _check(lib().pkv_paged_attention_decode_static(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(context_lens),
        s, block_tables.shape[1], int(max_context_len), nb, bs, hq, hkv, d, float(scale),
        _partition(partition_size), _dtype_code(q), DECODE_ALGOS[algo], _stream(stream)))
    return out


def paged_attention_decode_store(out, q, k_cache, v_cache, block_tables, context_lens, k_new,
                                 v_new, slot_mapping, scale, max_context_len, partition_size=0,
                                 workspace=None, algo="auto", stream=None):
    """Store one new K/V row per sequence (at its slot, which must be position
    context_lens[s]-1) and run decode, in one launch; writes out and the caches."""
    DecodeStoreLaunch(out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                      slot_mapping, scale, max_context_len, partition_size, algo,
                      workspace, _cache_workspace=True)(stream)
    return out


def _check_fp8_cache(k_cache, v_cache, k_scale, v_scale):
    _need(k_cache.dtype == v_cache.dtype == torch.uint8 and k_cache.dim() == 4
          and v_cache.shape == k_cache.shape, "E4M3 caches must be uint8 [NB, bs, Hkv, D]")
    hkv = k_cache.shape[2]
    _need(k_scale.dtype == v_scale.dtype == torch.float32 and k_scale.shape == (hkv,)
          and v_scale.shape == (hkv,), "k_scale, v_scale must be float32 [Hkv]")


def kv_cache_store_fp8(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale, stream=None):
    """Quantise new K/V rows (bf16 or fp32 [T, Hkv, D]) to E4M3 codes with one
    scale per kv-head and write them into uint8 caches [NB, bs, Hkv, D]."""
    StoreFp8Launch(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale)(stream)


def paged_attention_decode_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                               context_lens, scale, max_context_len, partition_size=0,
                               workspace=None, stream=None):
    """Decode over E4M3 caches (uint8 [NB, bs, Hkv, D], scales float32 [Hkv]);
    q and out bf16 [S, Hq, D]."""
    DecodeFp8Launch(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, scale,
                    max_context_len, partition_size, workspace, _cache_workspace=True)(stream)
    return out


def paged_attention_decode_store_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                     context_lens, k_new, v_new, slot_mapping, scale,
                                     max_context_len, partition_size=0, workspace=None, stream=None):
    """Quantise and store one new row per sequence (bf16 k_new / v_new
    [S, Hkv, D], at the slot of position context_lens[s]-1) and decode over
    the E4M3 caches, in one launch."""
    DecodeStoreFp8Launch(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, k_new,
                         v_new, slot_mapping, scale, max_context_len, partition_size, workspace,
                         _cache_workspace=True)(stream)
    return out


def paged_attention_decode_shared_prefix(out, q, k_cache, v_cache, block_tables, context_lens,
                                         group_starts, group_prefix_lens, scale, max_context_len,
                                         max_group_size, max_prefix_len, workspace=None,
                                         stream=None):
    """Decode where groups of consecutive sequences share their first blocks:
    group j is sequences group_starts[j] .. group_starts[j+1]-1 (int32 device
    [NG+1]) sharing group_prefix_lens[j] tokens (int32 device [NG])."""
    SharedPrefixDecodeLaunch(out, q, k_cache, v_cache, block_tables, context_lens, group_starts,
                             group_prefix_lens, scale, max_context_len, max_group_size,
                             max_prefix_len, workspace)(stream)
    return out


def paged_attention_prefill_chunk(out, q, k_cache, v_cache, block_tables, cu_seqlens_q,
                                  context_lens, scale, max_q_len, max_context_len, causal=True,
                                  stream=None):
    """Packed query chunks over their paged contexts; writes out [Tq, Hq, D]."""
    _dev(out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens)
    _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [Tq, Hq, D]")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
    _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2, "block_tables must be int32")
    n = block_tables.shape[0]
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (n + 1,),
          "cu_seqlens_q must be int32 [S+1]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (n,),
          "context_lens must be int32 [S]")
    tq, hq, d = q.shape
    nb, bs, hkv, _ = k_cache.shape
    _check(lib().pkv_paged_attention_prefill_chunk(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(cu_seqlens_q),
        _ptr(context_lens), n, tq, int(max_q_len), block_tables.shape[1], int(max_context_len),
        nb, bs, hq, hkv, d, float(scale), int(bool(causal)), _dtype_code(q), _stream(stream)))
    return out


# --------------------------------------------------------------------------
# Prepared launches: arguments checked and marshalled once, then each call is
# a single C-ABI call with the cached arguments on the current (or a given)
# stream. For serving loops and graph capture, where per-call Python work
# would otherwise dominate short kernels.
# --------------------------------------------------------------------------

class _Prepared:
    _fn = None
    _args = ()

    def __call__(self, stream=None):
        _check(getattr(lib(), self._fn)(*self._args, _stream(stream)))


class StoreLaunch(_Prepared):
    """kv_cache_store with fixed tensors."""

    def __init__(self, k, v, k_cache, v_cache, slot_mapping):
        _dev(k, v, k_cache, v_cache, slot_mapping)
        _need(k.dim() == 3 and v.shape == k.shape, "k, v must be [T, Hkv, D]")
        _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
        _need(k_cache.shape[2:] == k.shape[1:], "cache and new rows disagree on heads/dims")
        _need(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (k.shape[0],),
              "slot_mapping must be int32 [T]")
        _need(k.dtype == v.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
        nb, bs, hkv, d = k_cache.shape
        self._keep = (k, v, k_cache, v_cache, slot_mapping)
        self._fn = "pkv_kv_cache_store"
        self._args = (_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
                      k.shape[0], nb, bs, hkv, d, _dtype_code(k))


class DecodeLaunch(_Prepared):
    """paged_attention_decode with fixed tensors; owns its workspace."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, scale,
                 max_context_len, partition_size=0, algo="auto", workspace=None, _cache_workspace=False):
        _dev(out, q, k_cache, v_cache, block_tables, context_lens)
        _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [S, Hq, D]")
        _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
        _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
              and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, MB]")
        _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
              "context_lens must be int32 [S]")
        s, hq, d = q.shape
        nb, bs, hkv, _ = k_cache.shape
        part = _partition(partition_size)
        workspace, ws_bytes = _decode_workspace(workspace, s, hq, hkv, d, max_context_len, part,
                                                q.device, cached=_cache_workspace)
        self._keep = (out, q, k_cache, v_cache, block_tables, context_lens, workspace)
        self._fn = "pkv_paged_attention_decode"
        self._args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                      _ptr(context_lens), s, block_tables.shape[1], int(max_context_len), nb, bs,
                      hq, hkv, d, float(scale), part, _ptr(workspace), ws_bytes,
                      _dtype_code(q), DECODE_ALGOS[algo])


def _prefill_args(out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens):
    """Checks shared by the prefill entry points; returns (n, Tq, Hq, D, NB, bs, Hkv)."""
    _dev(out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens)
    _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [Tq, Hq, D]")
    _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2, "block_tables must be int32")
    n = block_tables.shape[0]
    _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (n + 1,),
          "cu_seqlens_q must be int32 [S+1]")
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (n,),
          "context_lens must be int32 [S]")
    return (n,) + tuple(q.shape) + tuple(k_cache.shape[:3])


def paged_attention_prefill_chunk_fp8(out, q, k_cache, v_cache, k_scale, v_scale, block_tables,
                                      cu_seqlens_q, context_lens, scale, max_q_len, max_context_len,
                                      causal=True, stream=None):
    """Chunked prefill over E4M3 caches (uint8 [NB, bs, Hkv, D], scales float32
    [Hkv]); bf16 q and out [Tq, Hq, D]."""
    _check_fp8_cache(k_cache, v_cache, k_scale, v_scale)
    _need(q.dtype == torch.bfloat16, "q must be bf16")
    n, tq, hq, d, nb, bs, hkv = _prefill_args(out, q, k_cache, v_cache, block_tables, cu_seqlens_q,
                                              context_lens)
    _check(lib().pkv_paged_attention_prefill_chunk_fp8(
        _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
        _ptr(block_tables), _ptr(cu_seqlens_q), _ptr(context_lens), n, tq, int(max_q_len),
        block_tables.shape[1], int(max_context_len), nb, bs, hq, hkv, d, float(scale),
        int(bool(causal)), _stream(stream)))
    return out


class PrefillLaunch(_Prepared):
    """paged_attention_prefill_chunk with fixed tensors."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens, scale,
                 max_q_len, max_context_len, causal=True):
        _dev(out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens)
        _need(q.dim() == 3 and out.shape == q.shape and out.dtype == q.dtype, "q/out must be [Tq, Hq, D]")
        _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape, "caches must be [NB, bs, Hkv, D]")
        _need(q.dtype == k_cache.dtype == v_cache.dtype, "dtypes must match")
        n = block_tables.shape[0]
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2, "block_tables must be int32")
        _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (n + 1,),
              "cu_seqlens_q must be int32 [S+1]")
        _need(context_lens.dtype == torch.int32 and context_lens.shape == (n,),
              "context_lens must be int32 [S]")
        tq, hq, d = q.shape
        nb, bs, hkv, _ = k_cache.shape
        self._keep = (out, q, k_cache, v_cache, block_tables, cu_seqlens_q, context_lens)
        self._fn = "pkv_paged_attention_prefill_chunk"
        self._args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                      _ptr(cu_seqlens_q), _ptr(context_lens), n, tq, int(max_q_len),
                      block_tables.shape[1], int(max_context_len), nb, bs, hq, hkv, d,
                      float(scale), int(bool(causal)), _dtype_code(q))


class PrefillFp8Launch(_Prepared):
    """paged_attention_prefill_chunk_fp8 with fixed tensors."""

    def __init__(self, out, q, k_cache, v_cache, k_scale, v_scale, block_tables, cu_seqlens_q,
                 context_lens, scale, max_q_len, max_context_len, causal=True):
        _check_fp8_cache(k_cache, v_cache, k_scale, v_scale)
        _need(q.dtype == torch.bfloat16, "q must be bf16")
        n, tq, hq, d, nb, bs, hkv = _prefill_args(out, q, k_cache, v_cache, block_tables,
                                                  cu_seqlens_q, context_lens)
        self._keep = (out, q, k_cache, v_cache, k_scale, v_scale, block_tables, cu_seqlens_q,
                      context_lens)
        self._fn = "pkv_paged_attention_prefill_chunk_fp8"
        self._args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                      _ptr(block_tables), _ptr(cu_seqlens_q), _ptr(context_lens), n, tq, int(max_q_len),
                      block_tables.shape[1], int(max_context_len), nb, bs, hq, hkv, d, float(scale),
                      int(bool(causal)))


class DecodeStoreLaunch(_Prepared):
    """paged_attention_decode_store with fixed tensors; owns its workspace."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, k_new, v_new,
                 slot_mapping, scale, max_context_len, partition_size=0, algo="auto",
                 workspace=None, _cache_workspace=False):
        base = DecodeLaunch(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                            max_context_len, partition_size, algo, workspace, _cache_workspace)
        _dev(k_new, v_new, slot_mapping)
        s, _, d = q.shape
        hkv = k_cache.shape[2]
        _need(k_new.shape == (s, hkv, d) and v_new.shape == k_new.shape, "k_new, v_new must be [S, Hkv, D]")
        _need(k_new.dtype == v_new.dtype == q.dtype, "dtypes must match")
        _need(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (s,), "slot_mapping must be int32 [S]")
        a = base._args
        self._keep = base._keep + (k_new, v_new, slot_mapping)
        self._fn = "pkv_paged_attention_decode_store"
        self._args = a[:6] + (_ptr(k_new), _ptr(v_new), _ptr(slot_mapping)) + a[6:]


class StoreFp8Launch(_Prepared):
    """kv_cache_store_fp8 with fixed tensors."""

    def __init__(self, k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale):
        _dev(k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale)
        _check_fp8_cache(k_cache, v_cache, k_scale, v_scale)
        _need(k.dim() == 3 and v.shape == k.shape and k.dtype == v.dtype, "k, v must be [T, Hkv, D]")
        _need(k_cache.shape[2:] == k.shape[1:], "cache and new rows disagree on heads/dims")
        _need(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (k.shape[0],),
              "slot_mapping must be int32 [T]")
        nb, bs, hkv, d = k_cache.shape
        self._keep = (k, v, k_cache, v_cache, slot_mapping, k_scale, v_scale)
        self._fn = "pkv_kv_cache_store_fp8"
        self._args = (_ptr(k), _ptr(v), _ptr(k_cache), _ptr(v_cache), _ptr(slot_mapping),
                      _ptr(k_scale), _ptr(v_scale), k.shape[0], nb, bs, hkv, d, _dtype_code(k))


class DecodeFp8Launch(_Prepared):
    """paged_attention_decode_fp8 with fixed tensors; owns its split-K workspace."""

    def __init__(self, out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                 scale, max_context_len, partition_size=0, workspace=None, _cache_workspace=False):
        _dev(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens)
        _check_fp8_cache(k_cache, v_cache, k_scale, v_scale)
        _need(q.dim() == 3 and out.shape == q.shape and q.dtype == out.dtype == torch.bfloat16,
              "q/out must be bf16 [S, Hq, D]")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
              and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, MB]")
        _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
              "context_lens must be int32 [S]")
        _need(k_cache.shape[3] == q.shape[2], "head_dim mismatch")
        s, hq, d = q.shape
        nb, bs, hkv, _ = k_cache.shape
        part = _partition(partition_size)
        workspace, ws_bytes = _decode_workspace(workspace, s, hq, hkv, d, max_context_len, part,
                                                q.device, cached=_cache_workspace)
        self._keep = (out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, workspace)
        self._fn = "pkv_paged_attention_decode_fp8"
        self._args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(k_scale), _ptr(v_scale),
                      _ptr(block_tables), _ptr(context_lens), s, block_tables.shape[1],
                      int(max_context_len), nb, bs, hq, hkv, d, float(scale), part,
                      _ptr(workspace), ws_bytes)


class DecodeStoreFp8Launch(_Prepared):
    """paged_attention_decode_store_fp8 with fixed tensors; owns its split-K workspace."""

    def __init__(self, out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens, k_new,
                 v_new, slot_mapping, scale, max_context_len, partition_size=0, workspace=None,
                 _cache_workspace=False):
        base = DecodeFp8Launch(out, q, k_cache, v_cache, k_scale, v_scale, block_tables, context_lens,
                               scale, max_context_len, partition_size, workspace, _cache_workspace)
        _dev(k_new, v_new, slot_mapping)
        s, _, d = q.shape
        hkv = k_cache.shape[2]
        _need(k_new.shape == (s, hkv, d) and v_new.shape == k_new.shape, "k_new, v_new must be [S, Hkv, D]")
        _need(k_new.dtype == v_new.dtype == torch.bfloat16, "k_new, v_new must be bf16")
        _need(slot_mapping.dtype == torch.int32 and slot_mapping.shape == (s,), "slot_mapping must be int32 [S]")
        a = base._args
        self._keep = base._keep + (k_new, v_new, slot_mapping)
        self._fn = "pkv_paged_attention_decode_store_fp8"
        self._args = a[:8] + (_ptr(k_new), _ptr(v_new), _ptr(slot_mapping)) + a[8:]


class SharedPrefixDecodeLaunch(_Prepared):
    """paged_attention_decode_shared_prefix with fixed tensors; owns its workspace."""

    def __init__(self, out, q, k_cache, v_cache, block_tables, context_lens, group_starts,
                 group_prefix_lens, scale, max_context_len, max_group_size, max_prefix_len,
                 workspace=None):
        _dev(out, q, k_cache, v_cache, block_tables, context_lens, group_starts, group_prefix_lens)
        _need(q.dim() == 3 and out.shape == q.shape and q.dtype == out.dtype == torch.bfloat16,
              "q/out must be bf16 [S, Hq, D]")
        _need(k_cache.dim() == 4 and v_cache.shape == k_cache.shape and k_cache.dtype == q.dtype,
              "caches must be bf16 [NB, bs, Hkv, D]")
        _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2
              and block_tables.shape[0] == q.shape[0], "block_tables must be int32 [S, MB]")
        _need(context_lens.dtype == torch.int32 and context_lens.shape == (q.shape[0],),
              "context_lens must be int32 [S]")
        ng = group_prefix_lens.shape[0]
        _need(group_starts.dtype == group_prefix_lens.dtype == torch.int32 and group_prefix_lens.dim() == 1
              and group_starts.shape == (ng + 1,), "group_starts int32 [NG+1], group_prefix_lens int32 [NG]")
        s, hq, d = q.shape
        nb, bs, hkv, _ = k_cache.shape
        need = int(lib().pkv_decode_shared_prefix_workspace_size(s, hq, d))
        if workspace is None and need:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        self._keep = (out, q, k_cache, v_cache, block_tables, context_lens, group_starts,
                      group_prefix_lens, workspace)
        self._fn = "pkv_paged_attention_decode_shared_prefix"
        self._args = (_ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
                      _ptr(context_lens), _ptr(group_starts), _ptr(group_prefix_lens), ng,
                      int(max_group_size), int(max_prefix_len), s, block_tables.shape[1],
                      int(max_context_len), nb, bs, hq, hkv, d, float(scale), _ptr(workspace), ws_bytes)


# --------------------------------------------------------------------------
# Checks of device-held inputs (debugging): each returns the device report
# (int32 [4]); see include/pkv.h for what each entry counts.
# --------------------------------------------------------------------------

def check_paged_inputs(block_tables, context_lens, num_blocks, block_size, max_context_len,
                       cu_seqlens_q=None, total_q=0, max_q_len=0, report=None, stream=None):
    """Count lengths outside [0, max_context_len], used table entries outside
    the pool and (with cu_seqlens_q) impossible chunk row counts."""
    _dev(block_tables, context_lens)
    _need(block_tables.dtype == torch.int32 and block_tables.dim() == 2, "block_tables must be int32 [S, MB]")
    n = block_tables.shape[0]
    _need(context_lens.dtype == torch.int32 and context_lens.shape == (n,), "context_lens must be int32 [S]")
    if cu_seqlens_q is not None:
        _dev(cu_seqlens_q)
        _need(cu_seqlens_q.dtype == torch.int32 and cu_seqlens_q.shape == (n + 1,),
              "cu_seqlens_q must be int32 [S+1]")
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=block_tables.device)
    _check(lib().pkv_check_paged_inputs(_ptr(block_tables), _ptr(context_lens), _ptr(cu_seqlens_q), n,
                                        block_tables.shape[1], int(max_context_len), int(total_q),
                                        int(max_q_len), int(num_blocks), int(block_size), _ptr(report),
                                        _stream(stream)))
    return report


def check_slots(slot_mapping, num_blocks, block_size, workspace=None, report=None, stream=None):
    """Count slots past the pool, repeated claims of a slot and padding slots."""
    _dev(slot_mapping)
    _need(slot_mapping.dtype == torch.int32 and slot_mapping.dim() == 1, "slot_mapping must be int32 [T]")
    need = int(lib().pkv_check_slots_workspace_size(int(num_blocks), int(block_size)))
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=slot_mapping.device)
    if report is None:
        report = torch.empty(4, dtype=torch.int32, device=slot_mapping.device)
    _check(lib().pkv_check_slots(_ptr(slot_mapping), slot_mapping.shape[0], int(num_blocks), int(block_size),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(report),
                                 _stream(stream)))
    return report
