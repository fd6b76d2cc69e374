"""Python binding of libcolimoe.so, the MI355X (gfx950) int4 routed-expert MoE layer.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels.  The functions carry the C ABI's names (``include/colimoe.h``) and
take plain integers for device pointers (e.g. ``tensor.data_ptr()``); PyTorch
is only a source of device memory and streams.  There is no fallback: if the
library is missing or a call fails, an exception says so.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcolimoe.so")

COLIMOE_OK = 0
COLIMOE_E_ARG = -1
COLIMOE_E_SHAPE = -2
COLIMOE_E_NOT_LOADED = -3
COLIMOE_E_WORKSPACE = -4
COLIMOE_E_HIP = -5
COLIMOE_E_STATE = -6

COLIMOE_FWD_AUTO = 0
COLIMOE_FWD_FP32 = 1
COLIMOE_FWD_BF16_MFMA = 2
COLIMOE_FWD_FXP = 3
COLIMOE_CFG_INT8 = 1
COLIMOE_STATIC_SCRATCH_BYTES = 32 << 20

EXPORTED = [
    "colimoe_create", "colimoe_destroy", "colimoe_set_stream", "colimoe_expert_bytes", "colimoe_layer_bytes",
    "colimoe_workspace_bytes", "colimoe_set_workspace", "colimoe_load_experts", "colimoe_route",
    "colimoe_union_build", "colimoe_forward", "colimoe_route_forward", "colimoe_rmsnorm_route_forward", "colimoe_rmsnorm", "colimoe_debug_expert", "colimoe_sync", "colimoe_status_str",
    "colimoe_timing_enable", "colimoe_timing_read", "colimoe_set_expert_top_p", "colimoe_expert_cache_bytes",
    "colimoe_host_layer_bytes", "colimoe_set_expert_cache", "colimoe_load_experts_host", "colimoe_cache_stats",
    "colimoe_cache_repin", "colimoe_route_forward_static", "colimoe_cache_set_prefetch", "colimoe_cache_set_autorepin",
    "colimoe_cache_usage", "colimoe_cache_usage_save", "colimoe_cache_usage_load", "colimoe_cache_get_info",
]


class colimoe_config(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("group_size", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class colimoe_layer_src(ctypes.Structure):
    _fields_ = [("router", ctypes.c_void_p), ("bias", ctypes.c_void_p), ("experts", ctypes.c_void_p),
                ("shared", ctypes.c_void_p)]


class colimoe_union(ctypes.Structure):
    _fields_ = [("n_unique", ctypes.c_void_p), ("ids", ctypes.c_void_p), ("offsets", ctypes.c_void_p),
                ("pair_token", ctypes.c_void_p), ("pair_slot", ctypes.c_void_p), ("pair_of", ctypes.c_void_p)]


class colimoe_cache_info(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64), ("predicted", ctypes.c_int64),
                ("predicted_hits", ctypes.c_int64), ("prefetched", ctypes.c_int64), ("prefetched_used", ctypes.c_int64),
                ("slots", ctypes.c_int32), ("slots_per_layer", ctypes.c_int32), ("pinned", ctypes.c_int32)]


class ColimoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %d (%s)" % (fn, status, status_str(status)))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libcolimoe.so not built: run python -m int4_routed_expert_fp32_amd._build; "
                              "there is no CPU fallback")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_size_t
        cfgp = ctypes.POINTER(colimoe_config)
        L.colimoe_create.argtypes = [cfgp, vp, ctypes.POINTER(vp)]
        L.colimoe_create.restype = ctypes.c_int
        L.colimoe_set_expert_top_p.argtypes = [vp, ctypes.c_float]
        L.colimoe_set_expert_top_p.restype = ctypes.c_int
        L.colimoe_destroy.argtypes = [vp]
        L.colimoe_destroy.restype = None
        L.colimoe_set_stream.argtypes = [vp, vp]
        L.colimoe_set_stream.restype = ctypes.c_int
        for fn in ("colimoe_expert_bytes", "colimoe_layer_bytes", "colimoe_workspace_bytes"):
            getattr(L, fn).argtypes = [cfgp]
            getattr(L, fn).restype = sz
        L.colimoe_set_workspace.argtypes = [vp, vp, sz]
        L.colimoe_set_workspace.restype = ctypes.c_int
        L.colimoe_load_experts.argtypes = [vp, i32, ctypes.POINTER(colimoe_layer_src), vp, sz]
        L.colimoe_load_experts.restype = ctypes.c_int
        L.colimoe_load_experts_host.argtypes = [vp, i32, ctypes.POINTER(colimoe_layer_src), vp, sz]
        L.colimoe_load_experts_host.restype = ctypes.c_int
        L.colimoe_expert_cache_bytes.argtypes = [cfgp, i32]
        L.colimoe_expert_cache_bytes.restype = sz
        L.colimoe_host_layer_bytes.argtypes = [cfgp]
        L.colimoe_host_layer_bytes.restype = sz
        L.colimoe_set_expert_cache.argtypes = [vp, vp, sz]
        L.colimoe_set_expert_cache.restype = ctypes.c_int
        L.colimoe_cache_stats.argtypes = [vp, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                                          ctypes.POINTER(i32)]
        L.colimoe_cache_stats.restype = ctypes.c_int
        L.colimoe_cache_repin.argtypes = [vp, i32]
        L.colimoe_cache_repin.restype = ctypes.c_int
        L.colimoe_cache_set_prefetch.argtypes = [vp, i32]
        L.colimoe_cache_set_prefetch.restype = ctypes.c_int
        L.colimoe_cache_set_autorepin.argtypes = [vp, i32, i32]
        L.colimoe_cache_set_autorepin.restype = ctypes.c_int
        L.colimoe_cache_usage.argtypes = [vp, i32, vp]
        L.colimoe_cache_usage.restype = ctypes.c_int
        L.colimoe_cache_usage_save.argtypes = [vp, ctypes.c_char_p]
        L.colimoe_cache_usage_save.restype = ctypes.c_int
        L.colimoe_cache_usage_load.argtypes = [vp, ctypes.c_char_p]
        L.colimoe_cache_usage_load.restype = ctypes.c_int
        L.colimoe_cache_get_info.argtypes = [vp, ctypes.POINTER(colimoe_cache_info)]
        L.colimoe_cache_get_info.restype = ctypes.c_int
        L.colimoe_route.argtypes = [vp, i32, vp, i32, vp, vp, ctypes.POINTER(colimoe_union), vp]
        L.colimoe_route.restype = ctypes.c_int
        L.colimoe_union_build.argtypes = [vp, vp, i32, ctypes.POINTER(colimoe_union)]
        L.colimoe_union_build.restype = ctypes.c_int
        L.colimoe_forward.argtypes = [vp, i32, vp, i32, vp, vp, ctypes.POINTER(colimoe_union), vp, u32]
        L.colimoe_forward.restype = ctypes.c_int
        L.colimoe_route_forward.argtypes = [vp, i32, vp, i32, vp, vp, ctypes.POINTER(colimoe_union), vp, u32]
        L.colimoe_route_forward.restype = ctypes.c_int
        L.colimoe_route_forward_static.argtypes = [vp, i32, vp, i32, vp, vp, ctypes.POINTER(colimoe_union), vp, u32]
        L.colimoe_route_forward_static.restype = ctypes.c_int
        L.colimoe_rmsnorm_route_forward.argtypes = [vp, i32, vp, i32, ctypes.c_float, vp, vp, vp,
                                                    ctypes.POINTER(colimoe_union), u32]
        L.colimoe_rmsnorm_route_forward.restype = ctypes.c_int
        L.colimoe_rmsnorm.argtypes = [vp, vp, i32, ctypes.c_float, vp]
        L.colimoe_rmsnorm.restype = ctypes.c_int
        L.colimoe_debug_expert.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
        L.colimoe_debug_expert.restype = ctypes.c_int
        L.colimoe_timing_enable.argtypes = [vp, ctypes.c_int]
        L.colimoe_timing_enable.restype = ctypes.c_int
        L.colimoe_timing_read.argtypes = [vp, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                          ctypes.POINTER(ctypes.c_int64), ctypes.c_int]
        L.colimoe_timing_read.restype = ctypes.c_int
        L.colimoe_sync.argtypes = [vp]
        L.colimoe_sync.restype = ctypes.c_int
        L.colimoe_status_str.argtypes = [ctypes.c_int]
        L.colimoe_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().colimoe_status_str(status).decode()


def _check(fn: str, status: int) -> int:
    if status != COLIMOE_OK:
        raise ColimoeError(fn, status)
    return status


def make_config(d: int, f: int, n_experts: int, top_k: int, n_layers: int = 1, n_shared: int = 0,
                max_tokens: int = 1, group_size: int = 64, flags: int = 0) -> colimoe_config:
    return colimoe_config(d, f, n_experts, top_k, n_layers, n_shared, group_size, max_tokens, flags)


def colimoe_expert_bytes(cfg: colimoe_config) -> int:
    return int(lib().colimoe_expert_bytes(ctypes.byref(cfg)))


def colimoe_layer_bytes(cfg: colimoe_config) -> int:
    return int(lib().colimoe_layer_bytes(ctypes.byref(cfg)))


def colimoe_workspace_bytes(cfg: colimoe_config) -> int:
    return int(lib().colimoe_workspace_bytes(ctypes.byref(cfg)))


def colimoe_create(cfg: colimoe_config, stream: Optional[int] = None, check: bool = True):
    """Returns (status, ctx handle)."""
    h = ctypes.c_void_p()
    rc = lib().colimoe_create(ctypes.byref(cfg), stream or None, ctypes.byref(h))
    if check:
        _check("colimoe_create", rc)
    return rc, h.value


def colimoe_destroy(ctx) -> None:
    if ctx:
        lib().colimoe_destroy(ctx)


def colimoe_set_stream(ctx, stream: Optional[int]) -> int:
    return _check("colimoe_set_stream", lib().colimoe_set_stream(ctx, stream or None))


def colimoe_set_expert_top_p(ctx, p: float, check: bool = True) -> int:
    rc = lib().colimoe_set_expert_top_p(ctx, p)
    return _check("colimoe_set_expert_top_p", rc) if check else rc


def colimoe_set_workspace(ctx, dev_ptr: int, nbytes: int, check: bool = True) -> int:
    rc = lib().colimoe_set_workspace(ctx, dev_ptr, nbytes)
    return _check("colimoe_set_workspace", rc) if check else rc


def colimoe_load_experts(ctx, layer: int, router_host: int, bias_host: Optional[int], experts_host: int,
                         shared_host: Optional[int], dev_dst: int, dev_bytes: int, check: bool = True) -> int:
    src = colimoe_layer_src(router_host, bias_host or None, experts_host, shared_host or None)
    rc = lib().colimoe_load_experts(ctx, layer, ctypes.byref(src), dev_dst, dev_bytes)
    return _check("colimoe_load_experts", rc) if check else rc


def colimoe_load_experts_host(ctx, layer: int, router_host: int, bias_host: Optional[int], experts_host: int,
                              shared_host: Optional[int], dev_dst: int, dev_bytes: int, check: bool = True) -> int:
    src = colimoe_layer_src(router_host, bias_host or None, experts_host, shared_host or None)
    rc = lib().colimoe_load_experts_host(ctx, layer, ctypes.byref(src), dev_dst, dev_bytes)
    return _check("colimoe_load_experts_host", rc) if check else rc


def colimoe_expert_cache_bytes(cfg: colimoe_config, n_slots: int) -> int:
    return int(lib().colimoe_expert_cache_bytes(ctypes.byref(cfg), n_slots))


def colimoe_host_layer_bytes(cfg: colimoe_config) -> int:
    return int(lib().colimoe_host_layer_bytes(ctypes.byref(cfg)))


def colimoe_set_expert_cache(ctx, dev_ptr: int, nbytes: int, check: bool = True) -> int:
    rc = lib().colimoe_set_expert_cache(ctx, dev_ptr, nbytes)
    return _check("colimoe_set_expert_cache", rc) if check else rc


def colimoe_cache_repin(ctx, n: int, check: bool = True) -> int:
    rc = lib().colimoe_cache_repin(ctx, n)
    return _check("colimoe_cache_repin", rc) if check else rc


def colimoe_cache_set_prefetch(ctx, depth: int, check: bool = True) -> int:
    rc = lib().colimoe_cache_set_prefetch(ctx, int(depth))
    return _check("colimoe_cache_set_prefetch", rc) if check else rc


def colimoe_cache_set_autorepin(ctx, every_tokens: int, n: int, check: bool = True) -> int:
    rc = lib().colimoe_cache_set_autorepin(ctx, every_tokens, n)
    return _check("colimoe_cache_set_autorepin", rc) if check else rc


def colimoe_cache_usage(ctx, layer: int, counts_ptr: int, check: bool = True) -> int:
    """Writes the layer's E usage counts (uint32) to host memory at counts_ptr."""
    rc = lib().colimoe_cache_usage(ctx, layer, counts_ptr)
    return _check("colimoe_cache_usage", rc) if check else rc


def colimoe_cache_usage_save(ctx, path: str, check: bool = True) -> int:
    rc = lib().colimoe_cache_usage_save(ctx, path.encode())
    return _check("colimoe_cache_usage_save", rc) if check else rc


def colimoe_cache_usage_load(ctx, path: str, check: bool = True) -> int:
    rc = lib().colimoe_cache_usage_load(ctx, path.encode())
    return _check("colimoe_cache_usage_load", rc) if check else rc


def colimoe_cache_get_info(ctx) -> colimoe_cache_info:
    info = colimoe_cache_info()
    _check("colimoe_cache_get_info", lib().colimoe_cache_get_info(ctx, ctypes.byref(info)))
    return info


def colimoe_cache_stats(ctx):
    """(hits, misses, slots) of the expert cache."""
    h, m, n = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check("colimoe_cache_stats", lib().colimoe_cache_stats(ctx, ctypes.byref(h), ctypes.byref(m), ctypes.byref(n)))
    return int(h.value), int(m.value), int(n.value)


def make_union(n_unique: int, ids: int, offsets: int, pair_token: int, pair_slot: int,
               pair_of: int) -> colimoe_union:
    return colimoe_union(n_unique, ids, offsets, pair_token, pair_slot, pair_of)


def colimoe_route(ctx, layer: int, x: int, T: int, idx: int, w: int, union: Optional[colimoe_union] = None,
                  logits: Optional[int] = None, check: bool = True) -> int:
    rc = lib().colimoe_route(ctx, layer, x, T, idx, w, ctypes.byref(union) if union is not None else None,
                             logits or None)
    return _check("colimoe_route", rc) if check else rc


def colimoe_union_build(ctx, idx: int, T: int, union: colimoe_union, check: bool = True) -> int:
    rc = lib().colimoe_union_build(ctx, idx, T, ctypes.byref(union))
    return _check("colimoe_union_build", rc) if check else rc


def colimoe_forward(ctx, layer: int, x: int, T: int, idx: int, w: int, union: Optional[colimoe_union],
                    residual: int, flags: int = COLIMOE_FWD_AUTO, check: bool = True) -> int:
    rc = lib().colimoe_forward(ctx, layer, x, T, idx, w, ctypes.byref(union) if union is not None else None,
                               residual, flags)
    return _check("colimoe_forward", rc) if check else rc


def colimoe_route_forward(ctx, layer: int, x: int, T: int, idx: int, w: int, union: Optional[colimoe_union],
                          residual: int, flags: int = COLIMOE_FWD_AUTO, check: bool = True) -> int:
    rc = lib().colimoe_route_forward(ctx, layer, x, T, idx, w, ctypes.byref(union) if union is not None else None,
                                     residual, flags)
    return _check("colimoe_route_forward", rc) if check else rc


def colimoe_route_forward_static(ctx, layer: int, x: int, T: int, idx: int, w: int, union: Optional[colimoe_union],
                                 residual: int, flags: int = COLIMOE_FWD_AUTO, check: bool = True) -> int:
    rc = lib().colimoe_route_forward_static(ctx, layer, x, T, idx, w,
                                            ctypes.byref(union) if union is not None else None, residual, flags)
    return _check("colimoe_route_forward_static", rc) if check else rc


def colimoe_rmsnorm_route_forward(ctx, layer: int, r: int, T: int, eps: float, x_out: int, idx: int, w: int,
                                  union: Optional[colimoe_union], flags: int = 0, check: bool = True) -> int:
    rc = lib().colimoe_rmsnorm_route_forward(ctx, layer, r, T, eps, x_out, idx, w,
                                             ctypes.byref(union) if union is not None else None, flags)
    return _check("colimoe_rmsnorm_route_forward", rc) if check else rc


def colimoe_rmsnorm(ctx, r: int, T: int, eps: float, x_out: int, check: bool = True) -> int:
    rc = lib().colimoe_rmsnorm(ctx, r, T, eps, x_out)
    return _check("colimoe_rmsnorm", rc) if check else rc


def colimoe_debug_expert(ctx, layer: int, e: int, x: int, g: Optional[int], u: Optional[int], h: Optional[int],
                         y: int, check: bool = True) -> int:
    rc = lib().colimoe_debug_expert(ctx, layer, e, x, g or None, u or None, h or None, y)
    return _check("colimoe_debug_expert", rc) if check else rc


def colimoe_sync(ctx, check: bool = True) -> int:
    rc = lib().colimoe_sync(ctx)
    return _check("colimoe_sync", rc) if check else rc


def colimoe_timing_enable(ctx, enable: bool) -> int:
    return _check("colimoe_timing_enable", lib().colimoe_timing_enable(ctx, 1 if enable else 0))


def colimoe_timing_read(ctx, name: str, reset: bool = False):
    """(total_ms, launches) of one kernel since the last reset."""
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check("colimoe_timing_read", lib().colimoe_timing_read(ctx, name.encode(), ctypes.byref(ms), ctypes.byref(n),
                                                            1 if reset else 0))
    return ms.value, n.value


def colimoe_status_str(status: int) -> str:
    return status_str(status)
