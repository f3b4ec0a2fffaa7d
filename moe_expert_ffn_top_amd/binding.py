"""Thin ctypes binding of libmoe (include/moe.h).

Argument marshalling only: every function forwards to the C entry point of the
same name, passing device pointers (torch tensors or ints) and a HIP stream
handle.  Nothing here computes any part of the MoE layer, and there is no
fallback: if libmoe.so is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libmoe.so is not built at %s; run `python -m moe_expert_ffn_top_amd.build` "
                      "or __graft_entry__.build()" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

MOE_OK = 0
MOE_ERR_ARG = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_NOT_PINNED = -4
MOE_ERR_WORKSPACE = -5
MOE_ERR_HIP = -6
MOE_ERR_STATE = -7
MOE_DEV_BAD_EXPERT_ID = 1
MOE_DEV_NOT_RESIDENT = 2
MOE_DEV_BAD_SLOT = 4
MOE_DEV_TAIL_SKIPPED = 8
MOE_DEV_CACHE_FULL = 16
MOE_DEV_SYNC_TIMEOUT = 32

#: every symbol include/moe.h declares
EXPORTED = ("moe_status_string", "moe_last_error", "moe_version", "moe_blob_layout_init", "moe_workspace_bytes",
            "moe_route", "moe_group", "moe_group_tail_skip", "moe_residency_update", "moe_residency_fill",
            "moe_heat_update", "moe_heat_decay", "moe_swap_plan", "moe_swap_apply",
            "moe_route_group", "moe_route_group_ffn", "moe_route_group_ffn_combine", "moe_expert_ffn",
            "moe_expert_ffn_stages",
            "moe_expert_ffn_combine",
            "moe_expert_ffn_down_combine",
            "moe_blob_layout_init_mx",
            "moe_mx_workspace_bytes", "moe_quantize_mxfp8", "moe_expert_ffn_mx", "moe_expert_ffn_mx_noalloc",
            "moe_route_group_ffn_mx",
            "moe_combine",
            "moe_ring_create", "moe_stage_h2d", "moe_ring_acquire", "moe_ring_release", "moe_ring_slot_ptr",
            "moe_ring_destroy", "moe_probe_hbm_read", "moe_probe_mfma", "moe_probe_scaled_mfma",
            "moe_debug_set_fused_wait")


class Dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("L", ctypes.c_int32)]

    def __init__(self, T, H, I, E, k, L=1):
        super().__init__(T, H, I, E, k, L)


class BlobLayout(ctypes.Structure):
    _fields_ = [("blob_bytes", ctypes.c_uint64), ("slot_stride", ctypes.c_uint64),
                ("off_codes", ctypes.c_uint64 * 3), ("off_scales", ctypes.c_uint64 * 3),
                ("off_globals", ctypes.c_uint64)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__("%s failed: %s (%s)" % (where, _lib.moe_status_string(status).decode(),
                                                 _lib.moe_last_error().decode()))


_vp, _i32, _u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
_DP = ctypes.POINTER(Dims)


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    """Declare the C signatures of include/moe.h on a loaded library."""
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_status_string.argtypes = [ctypes.c_int]
    lib.moe_last_error.restype = ctypes.c_char_p
    lib.moe_version.restype = ctypes.c_char_p
    lib.moe_blob_layout_init.argtypes = [_i32, _i32, ctypes.POINTER(BlobLayout)]
    lib.moe_workspace_bytes.argtypes = [_DP, ctypes.POINTER(_u64)]
    lib.moe_route.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.moe_group.argtypes = [_DP, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _u64, _vp]
    lib.moe_heat_update.argtypes = [_DP, _i32, _vp, _vp, _vp]
    lib.moe_heat_decay.argtypes = [_DP, _vp, ctypes.c_float, _vp]
    lib.moe_swap_plan.argtypes = [_DP, _vp, _vp, ctypes.c_float, _i32, _vp, ctypes.POINTER(_i32)]
    lib.moe_swap_apply.argtypes = [_DP, ctypes.POINTER(BlobLayout), _vp, _vp, _u64, _i32, _vp, _vp, _i32, _vp, _vp,
                                   _vp]
    lib.moe_residency_update.argtypes = [_DP, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
    lib.moe_residency_fill.argtypes = [_DP, ctypes.POINTER(BlobLayout), _vp, _vp, _u64, _i32, _vp, _vp, _vp]
    lib.moe_group_tail_skip.argtypes = [_DP, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _u64,
                                        _vp]
    lib.moe_route_group.argtypes = [_DP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _vp,
                                    _vp, _vp, _u64, _vp]
    lib.moe_route_group_ffn.argtypes = [_DP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                        _vp, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _u64,
                                        _i32, _vp, _vp, _vp]
    lib.moe_route_group_ffn_combine.argtypes = [_DP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp,
                                                _vp, _vp, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp,
                                                _vp, _vp, _u64, _vp, _vp, _vp]
    lib.moe_route_group_ffn_mx.argtypes = [_DP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _vp,
                                           _vp, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _u64,
                                           _vp, _u64, _i32, _vp, _vp, _vp]
    lib.moe_expert_ffn.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _vp, _vp,
                                   _vp, _u64, _vp]
    lib.moe_expert_ffn_stages.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _u64, _i32, _vp, _vp, _vp]
    lib.moe_expert_ffn_combine.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _u64, _vp, _vp, _vp]
    lib.moe_expert_ffn_down_combine.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp, _u64, _vp, _vp, _vp]
    lib.moe_blob_layout_init_mx.argtypes = [_i32, _i32, ctypes.POINTER(BlobLayout)]
    lib.moe_mx_workspace_bytes.argtypes = [_DP, ctypes.POINTER(_u64)]
    lib.moe_quantize_mxfp8.argtypes = [_vp, ctypes.c_int64, _i32, _vp, _vp, _vp]
    lib.moe_expert_ffn_mx.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp, _vp, _vp,
                                      _vp, _u64, _vp, _u64, _i32, _vp, _vp, _vp]
    lib.moe_expert_ffn_mx_noalloc.argtypes = [_DP, _vp, _vp, _u64, ctypes.POINTER(BlobLayout), _vp, _vp, _vp, _vp,
                                              _vp, _vp, _vp, _u64, _i32, _vp]
    lib.moe_combine.argtypes = [_DP, _vp, _vp, _vp, _vp, _vp, _vp]
    lib.moe_ring_create.argtypes = [_vp, _vp, _u64, _vp, ctypes.POINTER(_vp)]
    lib.moe_stage_h2d.argtypes = [_vp, _vp, _u64, ctypes.POINTER(_i32)]
    lib.moe_ring_acquire.argtypes = [_vp, _i32, _vp]
    lib.moe_ring_release.argtypes = [_vp, _i32, _vp]
    lib.moe_ring_slot_ptr.argtypes = [_vp, _i32, ctypes.POINTER(_vp)]
    lib.moe_ring_destroy.argtypes = [_vp]
    lib.moe_probe_hbm_read.argtypes = [_vp, _u64, _i32, _vp, _vp]
    lib.moe_probe_mfma.argtypes = [_i32, _i32, _i32, _vp, _vp]
    lib.moe_probe_scaled_mfma.argtypes = [_vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp]
    lib.moe_debug_set_fused_wait.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.moe_debug_set_fused_wait.restype = None
    return lib


_bind(_lib)


def use_library(path: str) -> None:
    """Route every call of this module to another build of libmoe (e.g. a
    build with different kernel tuning constants)."""
    global _lib
    _lib = _bind(ctypes.CDLL(path))


def _p(t) -> Optional[int]:
    """Device/host address of a torch tensor, an int, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _s(stream) -> Optional[int]:
    """HIP stream handle: None -> torch's current stream; int; torch stream."""
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else 0
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, where)


def moe_version() -> str:
    return _lib.moe_version().decode()


def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_blob_layout_init(H: int, I: int) -> BlobLayout:
    out = BlobLayout()
    _check(_lib.moe_blob_layout_init(H, I, ctypes.byref(out)), "moe_blob_layout_init")
    return out


def moe_workspace_bytes(dims: Dims) -> int:
    out = _u64()
    _check(_lib.moe_workspace_bytes(ctypes.byref(dims), ctypes.byref(out)), "moe_workspace_bytes")
    return out.value


def moe_route(dims, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma,
              stream=None) -> None:
    _check(_lib.moe_route(ctypes.byref(dims), _p(x), _p(w_router), _p(logits_in), _p(w_shared_gate), _p(logits_out),
                          _p(topk_ids), _p(topk_w), _p(shared_sigma), _s(stream)), "moe_route")


def moe_group(dims, layer, topk_ids, slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
              ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_group(ctypes.byref(dims), layer, _p(topk_ids), _p(slot_table), n_slots, _p(offsets), _p(perm),
                          _p(inv_perm), _p(group_slot), _p(dev_status), _p(ws), ws_bytes, _s(stream)), "moe_group")


def moe_residency_update(dims, layer, topk_ids, slot_table, slot_owner, last_use, n_slots, clock, fill_list, n_fill,
                         dev_status, stream=None) -> None:
    _check(_lib.moe_residency_update(ctypes.byref(dims), layer, _p(topk_ids), _p(slot_table), _p(slot_owner),
                                     _p(last_use), n_slots, _p(clock), _p(fill_list), _p(n_fill), _p(dev_status),
                                     _s(stream)), "moe_residency_update")


def moe_residency_fill(dims, layout, host_blobs, pool, pool_bytes, n_slots, fill_list, n_fill, stream=None) -> None:
    """host_blobs: a device-readable address of pinned host memory (an int)."""
    _check(_lib.moe_residency_fill(ctypes.byref(dims), ctypes.byref(layout), _p(host_blobs), _p(pool), pool_bytes,
                                   n_slots, _p(fill_list), _p(n_fill), _s(stream)), "moe_residency_fill")


def moe_heat_update(dims, layer, offsets, heat, stream=None) -> None:
    _check(_lib.moe_heat_update(ctypes.byref(dims), layer, _p(offsets), _p(heat), _s(stream)), "moe_heat_update")


def moe_heat_decay(dims, heat, decay: float = 0.7, stream=None) -> None:
    _check(_lib.moe_heat_decay(ctypes.byref(dims), _p(heat), decay, _s(stream)), "moe_heat_decay")


def moe_swap_plan(dims, heat, slot_table, threshold: float = 1.5, max_swaps: int = 96):
    """Host call on numpy arrays: heat float32 [L][E], slot_table int32 [L][E+1].
    Returns an int32 array [n][3] of (layer, hot, cold)."""
    import numpy as np
    h = np.ascontiguousarray(heat, dtype=np.float32)
    t = np.ascontiguousarray(slot_table, dtype=np.int32)
    plan = np.zeros((max(max_swaps, 1), 3), np.int32)
    n = _i32(0)
    _check(_lib.moe_swap_plan(ctypes.byref(dims), h.ctypes.data, t.ctypes.data, threshold, max_swaps,
                              plan.ctypes.data, ctypes.byref(n)), "moe_swap_plan")
    return plan[:n.value].copy()


def moe_swap_apply(dims, layout, host_blobs, pool, pool_bytes, n_slots, slot_table, plan, n_plan, fill_scratch,
                   n_scratch, stream=None) -> None:
    _check(_lib.moe_swap_apply(ctypes.byref(dims), ctypes.byref(layout), _p(host_blobs), _p(pool), pool_bytes,
                               n_slots, _p(slot_table), _p(plan), n_plan, _p(fill_scratch), _p(n_scratch),
                               _s(stream)), "moe_swap_apply")


def moe_group_tail_skip(dims, layer, topk_ids, slot_table, n_slots, skip_rank, offsets, perm, inv_perm, group_slot,
                        dev_status, n_skipped, ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_group_tail_skip(ctypes.byref(dims), layer, _p(topk_ids), _p(slot_table), n_slots, skip_rank,
                                    _p(offsets), _p(perm), _p(inv_perm), _p(group_slot), _p(dev_status),
                                    _p(n_skipped), _p(ws), ws_bytes, _s(stream)), "moe_group_tail_skip")


def moe_route_group(dims, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w, shared_sigma,
                    slot_table, n_slots, offsets, perm, inv_perm, group_slot, dev_status, ws,
                    ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_route_group(ctypes.byref(dims), layer, _p(x), _p(w_router), _p(logits_in), _p(w_shared_gate),
                                _p(logits_out), _p(topk_ids), _p(topk_w), _p(shared_sigma), _p(slot_table), n_slots,
                                _p(offsets), _p(perm), _p(inv_perm), _p(group_slot), _p(dev_status), _p(ws),
                                ws_bytes, _s(stream)), "moe_route_group")


def moe_route_group_ffn(dims, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                        shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, pool, pool_bytes,
                        layout: BlobLayout, h, y_rows, dev_status, ws, stages: int = 3, ev_start: Optional[int] = None,
                        ev_stop: Optional[int] = None, ws_bytes: Optional[int] = None, stream=None) -> None:
    """moe_route_group, then moe_expert_ffn_stages(stages 1 or 3); ev_start / ev_stop:
    raw hipEvent_t handles (ints) or None."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_route_group_ffn(ctypes.byref(dims), layer, _p(x), _p(w_router), _p(logits_in),
                                    _p(w_shared_gate), _p(logits_out), _p(topk_ids), _p(topk_w), _p(shared_sigma),
                                    _p(slot_table), n_slots, _p(offsets), _p(perm), _p(inv_perm), _p(group_slot),
                                    _p(pool), pool_bytes, ctypes.byref(layout), _p(h), _p(y_rows), _p(dev_status),
                                    _p(ws), ws_bytes, stages, ev_start, ev_stop, _s(stream)), "moe_route_group_ffn")


def moe_route_group_ffn_combine(dims, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                                shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, pool,
                                pool_bytes, layout: BlobLayout, h, y_rows, y, dev_status, ws,
                                ev_start: Optional[int] = None, ev_stop: Optional[int] = None,
                                ws_bytes: Optional[int] = None, stream=None) -> None:
    """moe_route_group_ffn (stages 3), then moe_combine; ev_start / ev_stop:
    raw hipEvent_t handles (ints) or None."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_route_group_ffn_combine(ctypes.byref(dims), layer, _p(x), _p(w_router), _p(logits_in),
                                            _p(w_shared_gate), _p(logits_out), _p(topk_ids), _p(topk_w),
                                            _p(shared_sigma), _p(slot_table), n_slots, _p(offsets), _p(perm),
                                            _p(inv_perm), _p(group_slot), _p(pool), pool_bytes, ctypes.byref(layout),
                                            _p(h), _p(y_rows), _p(y), _p(dev_status), _p(ws), ws_bytes, ev_start,
                                            ev_stop, _s(stream)), "moe_route_group_ffn_combine")


def moe_route_group_ffn_mx(dims, layer, x, w_router, logits_in, w_shared_gate, logits_out, topk_ids, topk_w,
                           shared_sigma, slot_table, n_slots, offsets, perm, inv_perm, group_slot, pool, pool_bytes,
                           layout: BlobLayout, h, y_rows, dev_status, ws, mx_ws, stages: int = 3,
                           ev_start: Optional[int] = None, ev_stop: Optional[int] = None,
                           ws_bytes: Optional[int] = None, mx_ws_bytes: Optional[int] = None, stream=None) -> None:
    """moe_route_group, then moe_expert_ffn_mx(stages 1 or 3); ev_start / ev_stop:
    raw hipEvent_t handles (ints) or None."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    if mx_ws_bytes is None:
        mx_ws_bytes = mx_ws.numel() * mx_ws.element_size()
    _check(_lib.moe_route_group_ffn_mx(ctypes.byref(dims), layer, _p(x), _p(w_router), _p(logits_in),
                                       _p(w_shared_gate), _p(logits_out), _p(topk_ids), _p(topk_w),
                                       _p(shared_sigma), _p(slot_table), n_slots, _p(offsets), _p(perm),
                                       _p(inv_perm), _p(group_slot), _p(pool), pool_bytes, ctypes.byref(layout),
                                       _p(h), _p(y_rows), _p(dev_status), _p(ws), ws_bytes, _p(mx_ws), mx_ws_bytes,
                                       stages, ev_start, ev_stop, _s(stream)), "moe_route_group_ffn_mx")


def moe_expert_ffn(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, h, y_rows, dev_status,
                   ws, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_expert_ffn(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout), _p(offsets),
                               _p(perm), _p(group_slot), _p(h), _p(y_rows), _p(dev_status), _p(ws), ws_bytes,
                               _s(stream)), "moe_expert_ffn")


def moe_expert_ffn_stages(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, h, y_rows,
                          dev_status, ws, stages: int, ev_start: Optional[int] = None, ev_stop: Optional[int] = None,
                          ws_bytes: Optional[int] = None, stream=None) -> None:
    """ev_start / ev_stop: raw hipEvent_t handles (ints) or None."""
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_expert_ffn_stages(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout),
                                      _p(offsets), _p(perm), _p(group_slot), _p(h), _p(y_rows), _p(dev_status),
                                      _p(ws), ws_bytes, stages, ev_start, ev_stop, _s(stream)),
           "moe_expert_ffn_stages")


def moe_expert_ffn_combine(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, inv_perm,
                           topk_w, shared_sigma, h, y_rows, y, dev_status, ws, ev_start: Optional[int] = None,
                           ev_stop: Optional[int] = None, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_expert_ffn_combine(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout),
                                       _p(offsets), _p(perm), _p(group_slot), _p(inv_perm), _p(topk_w),
                                       _p(shared_sigma), _p(h), _p(y_rows), _p(y), _p(dev_status), _p(ws), ws_bytes,
                                       ev_start, ev_stop, _s(stream)), "moe_expert_ffn_combine")


def moe_expert_ffn_down_combine(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, inv_perm,
                                topk_w, shared_sigma, h, y_rows, y, dev_status, ws, ev_start: Optional[int] = None,
                                ev_stop: Optional[int] = None, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_expert_ffn_down_combine(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout),
                                            _p(offsets), _p(perm), _p(group_slot), _p(inv_perm), _p(topk_w),
                                            _p(shared_sigma), _p(h), _p(y_rows), _p(y), _p(dev_status), _p(ws),
                                            ws_bytes, ev_start, ev_stop, _s(stream)), "moe_expert_ffn_down_combine")


def moe_blob_layout_init_mx(H: int, I: int) -> BlobLayout:
    out = BlobLayout()
    _check(_lib.moe_blob_layout_init_mx(H, I, ctypes.byref(out)), "moe_blob_layout_init_mx")
    return out


class MxWorkspace:
    """Section offsets of the MX activation workspace (include/moe.h)."""

    def __init__(self, dims: Dims):
        def a256(v):
            return (v + 255) // 256 * 256
        T, H, I, k = dims.T, dims.H, dims.I, dims.k
        rows_h = T * k + T
        self.xs_stride = (H // 32 + 15) // 16 * 16
        self.hs_stride = (I // 32 + 15) // 16 * 16
        self.gemm = T * k >= 16 * dims.E   # the grouped-GEMM layout; else the bf16 one
        if self.gemm:
            self.off_xq = 0
            self.off_xs = a256(T * H)
            self.off_hq = a256(self.off_xs + T * self.xs_stride)
            self.off_hs = a256(self.off_hq + rows_h * I)
            self.total = a256(self.off_hs + rows_h * self.hs_stride)
            self.off_xb = self.off_hb = self.total
        else:
            self.off_xb = 0
            self.off_hb = a256(T * H * 2)
            self.total = a256(self.off_hb + rows_h * I * 2)
            self.off_xq = self.off_xs = self.off_hq = self.off_hs = self.total


def moe_mx_workspace_bytes(dims: Dims) -> int:
    out = _u64()
    _check(_lib.moe_mx_workspace_bytes(ctypes.byref(dims), ctypes.byref(out)), "moe_mx_workspace_bytes")
    return out.value


def moe_quantize_mxfp8(x, rows: int, K: int, codes, scales, stream=None) -> None:
    _check(_lib.moe_quantize_mxfp8(_p(x), rows, K, _p(codes), _p(scales), _s(stream)), "moe_quantize_mxfp8")


def moe_expert_ffn_mx(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, h, y_rows,
                      dev_status, ws, mx_ws, stages: int = 3, ev_start: Optional[int] = None,
                      ev_stop: Optional[int] = None, ws_bytes: Optional[int] = None,
                      mx_ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    if mx_ws_bytes is None:
        mx_ws_bytes = mx_ws.numel() * mx_ws.element_size()
    _check(_lib.moe_expert_ffn_mx(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout),
                                  _p(offsets), _p(perm), _p(group_slot), _p(h), _p(y_rows), _p(dev_status), _p(ws),
                                  ws_bytes, _p(mx_ws), mx_ws_bytes, stages, ev_start, ev_stop, _s(stream)),
           "moe_expert_ffn_mx")


def moe_expert_ffn_mx_noalloc(dims, x, pool, pool_bytes, layout: BlobLayout, offsets, perm, group_slot, h, y_rows,
                              dev_status, ws, stages: int = 3, ws_bytes: Optional[int] = None, stream=None) -> None:
    if ws_bytes is None:
        ws_bytes = ws.numel() * ws.element_size()
    _check(_lib.moe_expert_ffn_mx_noalloc(ctypes.byref(dims), _p(x), _p(pool), pool_bytes, ctypes.byref(layout),
                                          _p(offsets), _p(perm), _p(group_slot), _p(h), _p(y_rows), _p(dev_status),
                                          _p(ws), ws_bytes, stages, _s(stream)), "moe_expert_ffn_mx_noalloc")


def moe_combine(dims, y_rows, inv_perm, topk_w, shared_sigma, y, stream=None) -> None:
    _check(_lib.moe_combine(ctypes.byref(dims), _p(y_rows), _p(inv_perm), _p(topk_w), _p(shared_sigma), _p(y),
                            _s(stream)), "moe_combine")


def moe_ring_create(slot0, slot1, slot_bytes: int, copy_stream) -> int:
    out = _vp()
    _check(_lib.moe_ring_create(_p(slot0), _p(slot1), slot_bytes, _s(copy_stream), ctypes.byref(out)),
           "moe_ring_create")
    return out.value


def moe_stage_h2d(ring: int, pinned_host_src, nbytes: int) -> int:
    slot = _i32()
    _check(_lib.moe_stage_h2d(ring, _p(pinned_host_src), nbytes, ctypes.byref(slot)), "moe_stage_h2d")
    return slot.value


def moe_ring_acquire(ring: int, slot: int, compute_stream=None) -> None:
    _check(_lib.moe_ring_acquire(ring, slot, _s(compute_stream)), "moe_ring_acquire")


def moe_ring_release(ring: int, slot: int, compute_stream=None) -> None:
    _check(_lib.moe_ring_release(ring, slot, _s(compute_stream)), "moe_ring_release")


def moe_ring_slot_ptr(ring: int, slot: int) -> int:
    out = _vp()
    _check(_lib.moe_ring_slot_ptr(ring, slot, ctypes.byref(out)), "moe_ring_slot_ptr")
    return out.value


def moe_ring_destroy(ring: int) -> None:
    _check(_lib.moe_ring_destroy(ring), "moe_ring_destroy")


def moe_probe_hbm_read(buf, nbytes: int, grid: int, sink, stream=None) -> None:
    _check(_lib.moe_probe_hbm_read(_p(buf), nbytes, grid, _p(sink), _s(stream)), "moe_probe_hbm_read")


def moe_probe_mfma(kind: int, grid: int, iters: int, sink, stream=None) -> None:
    _check(_lib.moe_probe_mfma(kind, grid, iters, _p(sink), _s(stream)), "moe_probe_mfma")


def moe_probe_scaled_mfma(a, b, sa, sb, n: int, split: int, d, stream=None) -> None:
    _check(_lib.moe_probe_scaled_mfma(_p(a), _p(b), _p(sa), _p(sb), n, split, _p(d), _s(stream)),
           "moe_probe_scaled_mfma")


def raw_status(fn_name: str, *args) -> int:
    """Call a C entry point and return its status without raising (for tests of
    the argument validation)."""
    return getattr(_lib, fn_name)(*args)
