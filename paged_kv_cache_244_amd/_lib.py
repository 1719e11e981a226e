"""ctypes binding to libpagedkv.so: argument marshalling only.

Every function here checks shapes and dtypes on the host, passes raw pointers
and the current HIP stream to the C ABI declared in ``include/pagedkv.h``, and
raises on a negative return code.  All computation happens in the library's
HIP kernels (device ops) or its host C++ allocator.  If the library is missing
the first call raises: there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, byref, c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv.so")

PKV_OK = 0
PKV_ERR_INVALID_ARG = -1
PKV_ERR_UNSUPPORTED = -2
PKV_ERR_OUT_OF_BLOCKS = -3
PKV_ERR_BAD_SEQ = -4
PKV_ERR_HIP = -5
PKV_ERR_WORKSPACE = -6
PKV_ERR_SWAPPED = -7
PKV_F32 = 0
PKV_F16 = 1
PKV_POLICY_DEFAULT = 0
PKV_POLICY_VALU = 1

_ERR_NAMES = {
    PKV_ERR_INVALID_ARG: "INVALID_ARG",
    PKV_ERR_UNSUPPORTED: "UNSUPPORTED",
    PKV_ERR_OUT_OF_BLOCKS: "OUT_OF_BLOCKS",
    PKV_ERR_BAD_SEQ: "BAD_SEQ",
    PKV_ERR_HIP: "HIP",
    PKV_ERR_WORKSPACE: "WORKSPACE",
    PKV_ERR_SWAPPED: "SWAPPED",
}


class PagedKVError(RuntimeError):
    def __init__(self, code, message):
        super().__init__(f"pagedkv error {code} ({_ERR_NAMES.get(code, '?')}): {message}")
        self.code = code


class OutOfBlocks(PagedKVError):
    pass


class BadSequence(PagedKVError):
    pass


class Swapped(PagedKVError):
    pass


class DecodePlan(ctypes.Structure):
    _fields_ = [("partition_size", c_int32), ("max_parts", c_int32), ("num_items", c_int32),
                ("waves_per_cu", c_int32), ("workspace_bytes", ctypes.c_uint64),
                ("fuse_groups", c_int32), ("reserved", c_int32)]


class StepLayout(ctypes.Structure):
    _fields_ = [("slots_offset", ctypes.c_uint64), ("pairs_offset", ctypes.c_uint64),
                ("tables_offset", ctypes.c_uint64), ("lens_offset", ctypes.c_uint64),
                ("items_offset", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
                ("num_pairs", c_int32), ("max_blocks", c_int32), ("max_context_len", c_int32),
                ("reserved", c_int32), ("plan", DecodePlan),
                ("groups_offset", ctypes.c_uint64), ("group_items_offset", ctypes.c_uint64),
                ("shared_lens_offset", ctypes.c_uint64),
                ("num_groups", c_int32), ("num_group_items", c_int32)]


class KVStats(ctypes.Structure):
    _fields_ = [("num_blocks", c_int32), ("free_blocks", c_int32), ("used_blocks", c_int32),
                ("shared_blocks", c_int32), ("live_tokens", c_int64), ("sum_refcounts", c_int64),
                ("pending_blocks", c_int32), ("host_blocks", c_int32),
                ("host_free_blocks", c_int32), ("host_used_blocks", c_int32),
                ("host_pending_blocks", c_int32), ("swapped_seqs", c_int32),
                ("swapped_out_blocks", c_int64), ("swapped_in_blocks", c_int64)]


_SIGNATURES = {
    "pkv_last_error": (ctypes.c_char_p, []),
    "kv_cache_write": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int32,
                                 c_int32, c_int32, c_int32, c_void_p]),
    "kv_copy_blocks": (c_int32, [POINTER(c_void_p), POINTER(c_void_p), c_int32, c_void_p, c_int32,
                                 c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "pkv_upload": (c_int32, [c_void_p, c_void_p, ctypes.c_uint64, c_void_p]),
    "pkv_upload_write": (c_int32, [c_void_p, c_void_p, ctypes.c_uint64, c_void_p, c_void_p, c_int32,
                                   c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                   c_void_p]),
    "kv_swap_blocks": (c_int32, [POINTER(c_void_p), POINTER(c_void_p), c_int32, POINTER(c_void_p),
                                 POINTER(c_void_p), c_int32, c_int32, c_void_p, c_int32, c_int32,
                                 c_int32, c_int32, c_void_p]),
    "pkv_time_next_call": (c_int32, [c_void_p, c_void_p]),
    "pkv_event_create": (c_int32, [POINTER(c_void_p)]),
    "pkv_event_destroy": (c_int32, [c_void_p]),
    "pkv_event_elapsed_ms": (c_int32, [c_void_p, c_void_p, POINTER(c_float)]),
    "pkv_read_probe": (c_int32, [c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_void_p]),
    "pkv_wave_timeline_read": (c_int32, [c_int32, c_void_p, c_size_t, c_int32]),
    "pkv_check_tables": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                   c_void_p]),
    "pa_decode_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "pa_decode_set_kernel_policy": (c_int32, [c_int32]),
    "pa_decode_plan": (c_int32, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_void_p, c_int32, POINTER(DecodePlan)]),
    "pa_decode_plan_capacity": (c_int32, [c_int32, c_int32, c_int32]),
    "pa_decode": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p,
                            c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                            c_float, c_int32, c_int32, c_void_p, c_int32, c_int32,
                            c_void_p, c_size_t, c_void_p]),
    "pa_decode_noalloc": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                    c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                                    c_int32, c_int32, c_float, c_int32, c_int32, c_void_p, c_int32,
                                    c_int32, c_void_p]),
    "pa_decode_contiguous": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                       c_void_p, c_int32, c_int32, c_int32, c_int32, c_float,
                                       c_int32, c_int32, c_void_p, c_int32, c_int32, c_void_p,
                                       c_size_t, c_void_p]),
    "pa_prefill": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                             c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                             c_int32, c_float, c_void_p, c_int32, c_void_p]),
    "pa_prefill_queries_per_item": (c_int32, [c_int32, c_int32]),
    "pa_prefill_plan": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p, c_int32,
                                  POINTER(c_int32)]),
    "kv_allocator_create": (c_int32, [c_int32, c_int32, c_void_p, POINTER(c_void_p)]),
    "kv_allocator_destroy": (None, [c_void_p]),
    "kv_seq_create": (c_int32, [c_void_p, POINTER(c_int32)]),
    "kv_seq_fork": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "kv_seq_append": (c_int32, [c_void_p, c_int32, c_int32, c_void_p, c_void_p, POINTER(c_int32)]),
    "kv_batch_append": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, POINTER(c_int32)]),
    "kv_seq_free": (c_int32, [c_void_p, c_int32]),
    "kv_seq_free_deferred": (c_int32, [c_void_p, c_int32, c_int64]),
    "kv_allocator_retire": (c_int32, [c_void_p, c_int64, POINTER(c_int32)]),
    "kv_allocator_add_host_tier": (c_int32, [c_void_p, c_int32, c_void_p]),
    "kv_swap_out": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int64, c_void_p, c_int32,
                              POINTER(c_int32)]),
    "kv_swap_in": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int64, c_void_p, c_int32,
                             POINTER(c_int32)]),
    "kv_seq_is_swapped": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "kv_seq_len": (c_int32, [c_void_p, c_int32, POINTER(c_int32)]),
    "kv_seq_lens": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p]),
    "kv_export_block_tables": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_void_p,
                                         c_void_p]),
    "kv_allocator_stats": (c_int32, [c_void_p, POINTER(KVStats)]),
    "kv_decode_step_host": (c_int32, [c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                      c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                      ctypes.c_uint64, POINTER(StepLayout)]),
    "pa_decode_plan_groups": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                                        c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                        c_int32, POINTER(DecodePlan), c_void_p, c_int32,
                                        POINTER(c_int32), c_void_p, POINTER(c_int32), c_void_p]),
    "pa_decode_grouped": (c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32,
                                    c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                    c_int32, c_float, c_int32, c_int32, c_void_p, c_int32, c_int32,
                                    c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                                    c_void_p, c_size_t, c_void_p]),
}

_lib = None


def lib():
    """Load libpagedkv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m paged_kv_cache_244_amd.build` (no fallback exists)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols():
    return list(_SIGNATURES)


def _check(rc):
    if rc != PKV_OK:
        msg = lib().pkv_last_error().decode(errors="replace")
        cls = {PKV_ERR_OUT_OF_BLOCKS: OutOfBlocks, PKV_ERR_BAD_SEQ: BadSequence,
               PKV_ERR_SWAPPED: Swapped}.get(rc, PagedKVError)
        raise cls(rc, msg)


# --------------------------------------------------------------------------- device ops

def _torch():
    import torch
    return torch


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return c_void_p(t.data_ptr())


def _pool_geometry(k_cache, v_cache):
    if k_cache.shape != v_cache.shape or k_cache.dim() != 4:
        raise ValueError("k_cache and v_cache must both be [num_blocks, kv_heads, block_size, head_dim]")
    return tuple(int(x) for x in k_cache.shape)


def kv_cache_write(k_cache, v_cache, k_new, v_new, slot_mapping, stream=None):
    """Store token j's K/V ([T, Hkv, D] fp16) in slot slot_mapping[j] (int64, <0 skips)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geometry(k_cache, v_cache)
    if k_new.shape != v_new.shape or tuple(k_new.shape[1:]) != (hkv, d):
        raise ValueError(f"k_new/v_new must be [T, {hkv}, {d}]")
    t = int(k_new.shape[0])
    if tuple(slot_mapping.shape) != (t,):
        raise ValueError("slot_mapping must be [T]")
    _check(lib().kv_cache_write(
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"), nb,
        _dev(k_new, torch.float16, "k_new"), _dev(v_new, torch.float16, "v_new"),
        _dev(slot_mapping, torch.int64, "slot_mapping"), t, hkv, d, bs, _stream(stream)))


def kv_copy_blocks(k_caches, v_caches, block_pairs, stream=None):
    """For each (src, dst) row of block_pairs (device int32 [P, 2]) copy every layer's block."""
    torch = _torch()
    if len(k_caches) != len(v_caches) or not k_caches:
        raise ValueError("need the same, non-zero number of K and V pools")
    geo = _pool_geometry(k_caches[0], v_caches[0])
    for k, v in zip(k_caches, v_caches):
        if _pool_geometry(k, v) != geo:
            raise ValueError("all layers' pools must share one geometry")
    nb, hkv, bs, d = geo
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [P, 2]")
    n = len(k_caches)
    kp = (c_void_p * n)(*[_dev(k, torch.float16, "k_cache").value for k in k_caches])
    vp = (c_void_p * n)(*[_dev(v, torch.float16, "v_cache").value for v in v_caches])
    _check(lib().kv_copy_blocks(kp, vp, n, _dev(block_pairs, torch.int32, "block_pairs"),
                                int(block_pairs.shape[0]), nb, hkv, d, bs, _stream(stream)))


def _pool_ptr(t, name):
    """Address of a pool that is a device tensor or a pinned host tensor (the library
    checks which and refuses anything else)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float16 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous fp16 tensor")
    if not (t.is_cuda or t.is_pinned()):
        raise TypeError(f"{name} must be device memory or pinned host memory")
    return t.data_ptr()


def kv_swap_blocks(dst_k, dst_v, src_k, src_v, block_pairs, stream=None):
    """For each (src, dst) row of block_pairs (device int32 [P, 2]) and each layer,
    block dst of the destination pools becomes block src of the source pools.  Pools
    are lists (one per layer) of fp16 [blocks, kv_heads, block_size, head_dim] tensors
    on the device or in pinned host memory."""
    torch = _torch()
    n = len(dst_k)
    if not n or not (len(dst_v) == len(src_k) == len(src_v) == n):
        raise ValueError("need the same, non-zero number of pools on every side")
    dgeo = _pool_geometry(dst_k[0], dst_v[0])
    sgeo = _pool_geometry(src_k[0], src_v[0])
    for a, b in zip(dst_k, dst_v):
        if _pool_geometry(a, b) != dgeo:
            raise ValueError("all destination pools must share one geometry")
    for a, b in zip(src_k, src_v):
        if _pool_geometry(a, b) != sgeo:
            raise ValueError("all source pools must share one geometry")
    if dgeo[1:] != sgeo[1:]:
        raise ValueError("source and destination blocks must have the same geometry")
    if block_pairs.dim() != 2 or block_pairs.shape[1] != 2:
        raise ValueError("block_pairs must be [P, 2]")
    _, hkv, bs, d = dgeo
    arr = [(c_void_p * n)(*[_pool_ptr(t, name) for t in ts])
           for ts, name in ((dst_k, "dst_k"), (dst_v, "dst_v"), (src_k, "src_k"), (src_v, "src_v"))]
    _check(lib().kv_swap_blocks(arr[0], arr[1], dgeo[0], arr[2], arr[3], sgeo[0], n,
                                _dev(block_pairs, torch.int32, "block_pairs"),
                                int(block_pairs.shape[0]), hkv, d, bs, _stream(stream)))


def plan(context_lens, num_q_heads, num_kv_heads, head_dim, block_size, q_dtype=PKV_F16,
         partition_size=-1, num_compute_units=0):
    """Host schedule of one decode launch from host lengths (``pa_decode_plan``).

    Returns (items, plan): items is a host uint32 array of (request << 16 | partition)
    entries, longest piece first; plan a dict with partition_size, max_parts, num_items,
    waves_per_cu and workspace_bytes.  ``partition_size`` < 0 lets the library choose.
    """
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    n = int(lens.shape[0])
    cap = int(lib().pa_decode_plan_capacity(n, int(lens.max()) if n else 0, int(block_size)))
    items = np.empty(max(cap, 1), dtype=np.uint32)
    pl = DecodePlan()
    _check(lib().pa_decode_plan(lens.ctypes.data if n else None, n, int(num_q_heads),
                                int(num_kv_heads), int(head_dim), int(block_size), int(q_dtype),
                                int(partition_size), int(num_compute_units), items.ctypes.data,
                                int(items.shape[0]), byref(pl)))
    info = {name: int(getattr(pl, name)) for name, _ in DecodePlan._fields_}
    return items[: info["num_items"]].copy(), info


GROUP_STRIDE = 17                     # PKV_GROUP_STRIDE: count, then up to 16 members
PKV_STEP_GROUPS = 1


def plan_groups(block_tables, context_lens, num_q_heads, num_kv_heads, head_dim, block_size,
                q_dtype=PKV_F16, partition_size=-1, num_compute_units=0):
    """``pa_decode_plan_groups``: the decode plan with prefix groups, from host tables.

    Returns (items, plan, groups, group_items, shared_lens): the remaining work items,
    the plan dict (its num_items counts them; its workspace_bytes covers the grouped
    launch), groups int32 [num_groups, 17] (count, members), group_items uint32
    (group << 16 | partition) and shared_lens int32 [num_seqs] (a group's shared length
    where it ends inside a partition, else 0).  No worthwhile group: groups is empty and
    the rest equals ``plan``'s result.
    """
    tables = np.ascontiguousarray(block_tables, dtype=np.int32)
    lens = np.ascontiguousarray(context_lens, dtype=np.int32)
    n = int(lens.shape[0])
    if tables.ndim != 2 or tables.shape[0] != n:
        raise ValueError("block_tables must be [num_seqs, max_blocks]")
    cap = int(lib().pa_decode_plan_capacity(n, int(lens.max()) if n else 0, int(block_size)))
    items = np.empty(max(cap, 1), dtype=np.uint32)
    gitems = np.empty(max(cap, 1), dtype=np.uint32)
    gcap = max(1, n // 2)
    groups = np.empty((gcap, GROUP_STRIDE), dtype=np.int32)
    shared = np.zeros(max(n, 1), dtype=np.int32)
    pl, ng, ngi = DecodePlan(), c_int32(0), c_int32(0)
    _check(lib().pa_decode_plan_groups(
        tables.ctypes.data if tables.size else None, int(tables.shape[1]),
        lens.ctypes.data if n else None, n, int(num_q_heads), int(num_kv_heads), int(head_dim),
        int(block_size), int(q_dtype), int(partition_size), int(num_compute_units),
        items.ctypes.data, int(items.shape[0]), byref(pl), groups.ctypes.data, gcap, byref(ng),
        gitems.ctypes.data, byref(ngi), shared.ctypes.data))
    info = {name: int(getattr(pl, name)) for name, _ in DecodePlan._fields_}
    return (items[: info["num_items"]].copy(), info, groups[: ng.value].copy(),
            gitems[: ngi.value].copy(), shared[:n].copy())


def _items(work_items):
    torch = _torch()
    if work_items.dim() != 1:
        raise ValueError("work_items must be 1-D")
    if work_items.dtype not in (torch.int32, torch.uint32):
        raise TypeError("work_items must be int32 or uint32 (request << 16 | partition)")
    return _dev(work_items, work_items.dtype, "work_items"), int(work_items.shape[0])


def set_kernel_policy(policy: int) -> int:
    """PKV_POLICY_DEFAULT (MFMA for fp16 head groups of >= 4) or PKV_POLICY_VALU.
    Returns the previous policy."""
    rc = lib().pa_decode_set_kernel_policy(int(policy))
    if rc < 0:
        _check(rc)
    return rc


def pa_decode_grouped(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size, groups, group_items, workspace=None,
                      stream=None, work_items=None, waves_per_cu=0, shared_lens=None, fuse=1):
    """``pa_decode`` with prefix groups: ``groups`` a device int32 [num_groups, 17] tensor,
    ``group_items`` a device int32/uint32 tensor of (group << 16 | partition) pieces and
    ``shared_lens`` a device int32 [S] tensor (or None), as ``plan_groups`` returns them;
    ``work_items`` the remaining pieces.  The workspace is
    ``pa_decode_workspace_size(S, Hq, D, max_context_len + partition_size, partition_size)``
    bytes (one spare slot per request)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geometry(k_cache, v_cache)
    s, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (s, hq, d):
        raise ValueError("q and out must be [S, Hq, head_dim]")
    if q.dtype != torch.float16:
        raise TypeError("grouped decode needs fp16 q")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(context_lens.shape) != (s,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    if groups.dim() != 2 or groups.shape[1] != GROUP_STRIDE:
        raise ValueError(f"groups must be int32 [num_groups, {GROUP_STRIDE}]")
    g_ptr, n_g = _items(group_items)
    items_ptr, n_items = c_void_p(None), 0
    if work_items is not None:
        # An empty list (every piece grouped) still needs an address: NULL means
        # "every piece" to the library.
        items_ptr, n_items = _items(work_items) if work_items.numel() else (g_ptr, 0)
    ws_ptr, ws_bytes = c_void_p(None), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib().pa_decode_grouped(
        _dev(out, torch.float32, "out"), _dev(q, q.dtype, "q"), PKV_F16,
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"), nb,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(context_lens, torch.int32, "context_lens"), s, hq, hkv, d, bs, float(scale),
        int(max_context_len), int(partition_size), items_ptr, n_items, int(waves_per_cu),
        _dev(groups, torch.int32, "groups"), int(groups.shape[0]), g_ptr, n_g,
        _dev(shared_lens, torch.int32, "shared_lens") if shared_lens is not None else None,
        int(fuse), ws_ptr, ws_bytes, _stream(stream)))


class KernelTimer:
    """A (start, stop) pair of HIP timing events made by the library, recorded by the
    kernels of a call when passed to ``time_next_call``; ``ms()`` waits for the call
    and returns the time from its first kernel's start to its last kernel's end."""

    __slots__ = ("start", "stop")

    def __init__(self):
        self.start, self.stop = c_void_p(), c_void_p()
        _check(lib().pkv_event_create(byref(self.start)))
        _check(lib().pkv_event_create(byref(self.stop)))

    def ms(self) -> float:
        out = c_float()
        _check(lib().pkv_event_elapsed_ms(self.start, self.stop, byref(out)))
        return float(out.value)

    def __del__(self):
        if _lib is not None:
            _lib.pkv_event_destroy(self.start)
            _lib.pkv_event_destroy(self.stop)


def time_next_call(timer=None):
    """Kernel-level timing of the next library device call on this thread: its
    kernels record into ``timer`` (a KernelTimer); None clears."""
    if timer is None:
        lib().pkv_time_next_call(None, None)
    else:
        lib().pkv_time_next_call(timer.start, timer.stop)


def check_tables(block_tables, context_lens, block_size, num_blocks, stream=None):
    """Debug check of device tables (int32 [S, max_blocks]) and lengths (int32 [S]):
    returns {"bad_ids", "bad_lengths", "first_request", "first_entry"} (pkv_check_tables);
    waits for the stream."""
    torch = _torch()
    if block_tables.dim() != 2 or tuple(context_lens.shape) != (block_tables.shape[0],):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    s, mb = (int(x) for x in block_tables.shape)
    result = torch.empty(4, dtype=torch.int32, device=block_tables.device)
    st = _stream(stream)
    _check(lib().pkv_check_tables(_dev(block_tables, torch.int32, "block_tables"), mb,
                                  _dev(context_lens, torch.int32, "context_lens"), s,
                                  int(block_size), int(num_blocks), c_void_p(result.data_ptr()), st))
    (stream if stream is not None else torch.cuda.current_stream()).synchronize()
    r = [int(x) for x in result.cpu()]
    return {"bad_ids": r[0], "bad_lengths": r[1], "first_request": r[2], "first_entry": r[3]}


PKV_TIMELINE_VALU = 0
PKV_TIMELINE_MFMA = 1
PKV_TIMELINE_PREFILL = 2
PKV_TIMELINE_RECORDS = 16384
PKV_TIMELINE_WORDS = 6
TIMELINE_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedkv_timeline.so")


def wave_timeline_read(kernel, clear=True):
    """Per-wave records of the kernel family ``kernel`` (PKV_TIMELINE_VALU,
    PKV_TIMELINE_MFMA or PKV_TIMELINE_PREFILL) as uint64 [PKV_TIMELINE_RECORDS, PKV_TIMELINE_WORDS]
    (pkv_wave_timeline_read; only the instrumented library records any)."""
    import numpy as np
    buf = np.zeros((PKV_TIMELINE_RECORDS, PKV_TIMELINE_WORDS), dtype=np.uint64)
    _check(lib().pkv_wave_timeline_read(int(kernel), c_void_p(buf.ctypes.data), buf.nbytes,
                                        1 if clear else 0))
    return buf


def pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len, partition_size):
    return int(lib().pa_decode_workspace_size(num_seqs, num_q_heads, head_dim, max_context_len,
                                              partition_size))


def pa_decode(out, q, k_cache, v_cache, block_tables, context_lens, scale, max_context_len,
              partition_size=512, workspace=None, stream=None, work_items=None, waves_per_cu=0):
    """Decode attention: out[S, Hq, D] fp32 from q[S, Hq, D] (fp32 or fp16) via the block tables.

    ``workspace`` is a device uint8 tensor of at least ``pa_decode_workspace_size`` bytes
    (needed only when a request may span more than one partition).  ``work_items`` is an
    optional device 1-D int32/uint32 tensor of (request << 16 | partition) pieces in
    dispatch order (``plan``'s list); ``waves_per_cu`` limits residency (0 = none).
    """
    torch = _torch()
    nb, hkv, bs, d = _pool_geometry(k_cache, v_cache)
    s, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (s, hq, d):
        raise ValueError("q and out must be [S, Hq, head_dim]")
    if q.dtype == torch.float32:
        qd = PKV_F32
    elif q.dtype == torch.float16:
        qd = PKV_F16
    else:
        raise TypeError("q must be float32 or float16")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(context_lens.shape) != (s,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    items_ptr, n_items = c_void_p(None), 0
    if work_items is not None:
        items_ptr, n_items = _items(work_items)
    ws_ptr, ws_bytes = c_void_p(None), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib().pa_decode(
        _dev(out, torch.float32, "out"), _dev(q, q.dtype, "q"), qd,
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"), nb,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(context_lens, torch.int32, "context_lens"), s, hq, hkv, d, bs, float(scale),
        int(max_context_len), int(partition_size), items_ptr, n_items, int(waves_per_cu),
        ws_ptr, ws_bytes, _stream(stream)))


PKV_NOALLOC_WORKSPACE_BYTES = 64 << 20     # pagedkv.h


def pa_decode_noalloc(out, q, k_cache, v_cache, block_tables, context_lens, scale,
                      max_context_len, partition_size=512, stream=None, work_items=None,
                      waves_per_cu=0):
    """``pa_decode`` with the split-context partials in the library's fixed per-GPU
    array (``PKV_NOALLOC_WORKSPACE_BYTES``) instead of a caller workspace: the call
    allocates no device memory.  Calls that may overlap on one GPU race on that
    array; issue them on one stream."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geometry(k_cache, v_cache)
    s, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (s, hq, d):
        raise ValueError("q and out must be [S, Hq, head_dim]")
    if q.dtype == torch.float32:
        qd = PKV_F32
    elif q.dtype == torch.float16:
        qd = PKV_F16
    else:
        raise TypeError("q must be float32 or float16")
    if block_tables.dim() != 2 or block_tables.shape[0] != s or tuple(context_lens.shape) != (s,):
        raise ValueError("block_tables must be [S, max_blocks] and context_lens [S]")
    items_ptr, n_items = c_void_p(None), 0
    if work_items is not None:
        items_ptr, n_items = _items(work_items)
    _check(lib().pa_decode_noalloc(
        _dev(out, torch.float32, "out"), _dev(q, q.dtype, "q"), qd,
        _dev(k_cache, torch.float16, "k_cache"), _dev(v_cache, torch.float16, "v_cache"), nb,
        _dev(block_tables, torch.int32, "block_tables"), int(block_tables.shape[1]),
        _dev(context_lens, torch.int32, "context_lens"), s, hq, hkv, d, bs, float(scale),
        int(max_context_len), int(partition_size), items_ptr, n_items, int(waves_per_cu),
        _stream(stream)))


def pa_decode_contiguous(out, q, k_rows, v_rows, context_lens, scale, max_context_len,
                         partition_size=0, workspace=None, stream=None, work_items=None,
                         waves_per_cu=0):
    """Decode attention over the layout without a block table: ``k_rows, v_rows`` are
    device fp16 [S, Hkv, Lmax, D], request i's token t of KV head g at [i, g, t]
    (Lmax a multiple of 16).  Otherwise as ``pa_decode``; the workspace size is
    ``pa_decode_workspace_size`` of the same arguments."""
    torch = _torch()
    if k_rows.shape != v_rows.shape or k_rows.dim() != 4:
        raise ValueError("k_rows and v_rows must both be [S, Hkv, Lmax, D]")
    s, hkv, lmax, d = (int(x) for x in k_rows.shape)
    sq, hq, dq = (int(x) for x in q.shape)
    if sq != s or dq != d or tuple(out.shape) != (s, hq, d):
        raise ValueError("q and out must be [S, Hq, D] matching the rows")
    if q.dtype == torch.float32:
        qd = PKV_F32
    elif q.dtype == torch.float16:
        qd = PKV_F16
    else:
        raise TypeError("q must be float32 or float16")
    if tuple(context_lens.shape) != (s,):
        raise ValueError("context_lens must be [S]")
    items_ptr, n_items = c_void_p(None), 0
    if work_items is not None:
        items_ptr, n_items = _items(work_items)
    ws_ptr, ws_bytes = c_void_p(None), 0
    if workspace is not None:
        ws_ptr = _dev(workspace, torch.uint8, "workspace")
        ws_bytes = workspace.numel()
    _check(lib().pa_decode_contiguous(
        _dev(out, torch.float32, "out"), _dev(q, q.dtype, "q"), qd,
        _dev(k_rows, torch.float16, "k_rows"), _dev(v_rows, torch.float16, "v_rows"), lmax,
        _dev(context_lens, torch.int32, "context_lens"), s, hq, hkv, d, float(scale),
        int(max_context_len), int(partition_size), items_ptr, n_items, int(waves_per_cu),
        ws_ptr, ws_bytes, _stream(stream)))


def prefill_plan(q_lens, context_lens, num_q_heads, num_kv_heads):
    """Work items of a pa_prefill launch (host uint32): requests by their costliest
    block, each request's blocks together, costliest first."""
    ql = np.ascontiguousarray(q_lens, dtype=np.int32)
    cl = np.ascontiguousarray(context_lens, dtype=np.int32)
    if ql.shape != cl.shape or ql.ndim != 1:
        raise ValueError("q_lens and context_lens must be 1-D and of one length")
    n = int(ql.shape[0])
    cap = max(int(np.maximum(ql, 0).sum()), 1)
    items = np.empty(cap, dtype=np.uint32)
    count = c_int32()
    _check(lib().pa_prefill_plan(ql.ctypes.data if n else None, cl.ctypes.data if n else None, n,
                                 int(num_q_heads), int(num_kv_heads), items.ctypes.data, cap,
                                 byref(count)))
    return items[: count.value].copy()


def pa_prefill(out, q, q_starts, k_cache, v_cache, block_tables, context_lens, scale,
               work_items, stream=None):
    """Causal prefill attention: out[T, Hq, D] fp32 from q[T, Hq, D] fp16 (T queries of
    all requests, request i's rows q_starts[i]..q_starts[i+1]) through the block tables;
    ``work_items`` from ``prefill_plan`` (device int32/uint32)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_geometry(k_cache, v_cache)
    t, hq, dq = (int(x) for x in q.shape)
    if dq != d or tuple(out.shape) != (t, hq, d):
        raise ValueError("q and out must be [T, Hq, head_dim]")
    s = int(context_lens.shape[0])
    if tuple(q_starts.shape) != (s + 1,) or block_tables.dim() != 2 or block_tables.shape[0] != s:
        raise ValueError("q_starts must be [S+1], block_tables [S, max_blocks], context_lens [S]")
    items_ptr, n_items = _items(work_items)
    _check(lib().pa_prefill(
        _dev(out, torch.float32, "out"), _dev(q, torch.float16, "q"),
        _dev(q_starts, torch.int32, "q_starts"), t, _dev(k_cache, torch.float16, "k_cache"),
        _dev(v_cache, torch.float16, "v_cache"), nb, _dev(block_tables, torch.int32, "block_tables"),
        int(block_tables.shape[1]), _dev(context_lens, torch.int32, "context_lens"), s, hq, hkv, d,
        bs, float(scale), items_ptr, n_items, _stream(stream)))


# --------------------------------------------------------------------------- host allocator

class BlockAllocator:
    """Owner of one host allocator object (refcounted blocks, tables, copy-on-write)."""

    def __init__(self, num_blocks, block_size, initial_order=None):
        self._h = c_void_p()
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise ValueError("initial_order must have num_blocks entries")
        self._order = order
        _check(lib().kv_allocator_create(num_blocks, block_size,
                                         None if order is None else order.ctypes.data,
                                         byref(self._h)))
        self.num_blocks = num_blocks
        self.block_size = block_size
        self._swap_pairs = np.empty((256, 2), dtype=np.int32)

    def close(self):
        if self._h:
            lib().kv_allocator_destroy(self._h)
            self._h = c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def create(self) -> int:
        out = c_int32()
        _check(lib().kv_seq_create(self._h, byref(out)))
        return out.value

    def fork(self, parent: int) -> int:
        out = c_int32()
        _check(lib().kv_seq_fork(self._h, parent, byref(out)))
        return out.value

    def append(self, seq: int, n: int):
        """Returns (slots int64 [n], cow_pairs list of (src, dst))."""
        slots = np.empty(max(n, 0), dtype=np.int64)
        pair = np.empty(2, dtype=np.int32)
        ncow = c_int32()
        _check(lib().kv_seq_append(self._h, seq, n, slots.ctypes.data, pair.ctypes.data, byref(ncow)))
        return slots, [tuple(int(x) for x in pair)] if ncow.value else []

    def append_batch(self, seqs):
        """One token per listed sequence; returns (slots int64 [n], pairs int32 [P, 2])."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = int(seqs.shape[0])
        slots = np.empty(n, dtype=np.int64)
        pairs = np.empty((max(n, 1), 2), dtype=np.int32)
        ncow = c_int32()
        _check(lib().kv_batch_append(self._h, seqs.ctypes.data, n, slots.ctypes.data,
                                     pairs.ctypes.data, byref(ncow)))
        return slots, pairs[: ncow.value]

    def free(self, seq: int):
        _check(lib().kv_seq_free(self._h, seq))

    def free_deferred(self, seq: int, epoch: int):
        """Free now, but park blocks that reach zero until ``retire(>= epoch)``."""
        _check(lib().kv_seq_free_deferred(self._h, seq, int(epoch)))

    def retire(self, done: int) -> int:
        """Return parked blocks with epoch <= ``done`` to the free list; how many."""
        out = c_int32()
        _check(lib().kv_allocator_retire(self._h, int(done), byref(out)))
        return out.value

    def add_host_tier(self, num_host_blocks, initial_order=None):
        order = None
        if initial_order is not None:
            order = np.ascontiguousarray(initial_order, dtype=np.int32)
            if order.shape != (num_host_blocks,):
                raise ValueError("initial_order must have num_host_blocks entries")
        _check(lib().kv_allocator_add_host_tier(self._h, int(num_host_blocks),
                                                None if order is None else order.ctypes.data))
        self.num_host_blocks = int(num_host_blocks)

    def _swap(self, fn, seqs, deferred, epoch):
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = int(seqs.shape[0])
        pairs = self._swap_pairs
        got = c_int32()
        while True:
            rc = fn(self._h, seqs.ctypes.data, n, int(bool(deferred)), int(epoch),
                    pairs.ctypes.data, int(pairs.shape[0]), byref(got))
            if rc == PKV_ERR_INVALID_ARG and got.value > pairs.shape[0]:
                pairs = self._swap_pairs = np.empty((got.value, 2), dtype=np.int32)
                continue
            _check(rc)
            return pairs[: got.value].copy()

    def swap_out(self, seqs, deferred=False, epoch=0):
        """Move the sequences' blocks to the host tier; int32 [P, 2] (device, host) pairs."""
        return self._swap(lib().kv_swap_out, seqs, deferred, epoch)

    def swap_in(self, seqs, deferred=False, epoch=0):
        """Move swapped-out sequences back; int32 [P, 2] (host, device) pairs."""
        return self._swap(lib().kv_swap_in, seqs, deferred, epoch)

    def is_swapped(self, seq: int) -> bool:
        out = c_int32()
        _check(lib().kv_seq_is_swapped(self._h, seq, byref(out)))
        return bool(out.value)

    def length(self, seq: int) -> int:
        out = c_int32()
        _check(lib().kv_seq_len(self._h, seq, byref(out)))
        return out.value

    def lengths(self, seqs):
        """Lengths of the listed sequences (host int32 array), one library call."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        lens = np.empty(seqs.shape[0], dtype=np.int32)
        _check(lib().kv_seq_lens(self._h, seqs.ctypes.data, int(seqs.shape[0]), lens.ctypes.data))
        return lens

    def export(self, seqs, max_blocks, pad_value=-1, tables_out=None, lens_out=None):
        """Block tables int32 [n, max_blocks] and lengths int32 [n] (host arrays)."""
        seqs = np.ascontiguousarray(seqs, dtype=np.int32)
        n = int(seqs.shape[0])
        tables = tables_out if tables_out is not None else np.empty((n, max_blocks), dtype=np.int32)
        lens = lens_out if lens_out is not None else np.empty(n, dtype=np.int32)
        if tables.shape != (n, max_blocks) or tables.dtype != np.int32 or not tables.flags.c_contiguous:
            raise ValueError("tables_out must be C-contiguous int32 [n, max_blocks]")
        if lens.shape != (n,) or lens.dtype != np.int32:
            raise ValueError("lens_out must be int32 [n]")
        _check(lib().kv_export_block_tables(self._h, seqs.ctypes.data, n, max_blocks, pad_value,
                                            tables.ctypes.data, lens.ctypes.data))
        return tables, lens

    def decode_step_host(self, seqs, max_blocks, pad_value, num_q_heads, num_kv_heads, head_dim,
                         q_dtype, partition_size, buffer_ptr, buffer_bytes, num_compute_units=0,
                         flags=0):
        """One decode step's host work into a caller buffer (``kv_decode_step_host``).

        ``seqs`` must be a C-contiguous int32 array.  Returns the StepLayout, or None when
        the buffer is too small (the allocator is then unchanged and the layout's
        ``total_bytes`` -- see ``needed`` -- says how much is needed)."""
        lay = StepLayout()
        rc = lib().kv_decode_step_host(self._h, seqs.ctypes.data, int(seqs.shape[0]),
                                       int(max_blocks), int(pad_value), int(num_q_heads),
                                       int(num_kv_heads), int(head_dim), int(q_dtype),
                                       int(partition_size), int(num_compute_units), int(flags),
                                       buffer_ptr, int(buffer_bytes), byref(lay))
        if rc == PKV_ERR_INVALID_ARG and lay.total_bytes > buffer_bytes:
            self.needed = int(lay.total_bytes)
            return None
        _check(rc)
        return lay

    def stats(self) -> dict:
        st = KVStats()
        _check(lib().kv_allocator_stats(self._h, byref(st)))
        return {name: getattr(st, name) for name, _ in KVStats._fields_}
