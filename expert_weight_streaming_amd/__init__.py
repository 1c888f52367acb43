"""Python binding of libmoe (argument marshalling only).

Every function here forwards to the C entry point of the same name in
libmoe.so (include/moe.h); all arithmetic runs in the library's HIP kernels.
Tensors are torch tensors on the GPU (PyTorch supplies device memory and
streams).  There is no fallback: the first call raises ImportError when
libmoe.so is missing.
"""
from __future__ import annotations

import ctypes
import os

from ._build import SO as _SO, build  # noqa: F401

MOE_OK = 0
MOE_EINVAL = -1
MOE_EUNSUPPORTED = -2
MOE_EHIP = -3
MOE_ESTATE = -4
MOE_DEVERR_EXPERT_RANGE = 1


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class LayerDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("inter", ctypes.c_int32), ("n_shared", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("group", ctypes.c_int32), ("rms_eps", ctypes.c_float), ("router_w", ctypes.c_void_p),
                ("gamma", ctypes.c_void_p), ("experts", ctypes.c_void_p), ("shared", ctypes.c_void_p),
                ("slab", ctypes.c_void_p), ("blob_bytes", ctypes.c_uint64), ("expert_addr", ctypes.c_void_p)]


class ExpertCache(ctypes.Structure):
    _fields_ = [("slots", ctypes.c_void_p), ("n_slots", ctypes.c_int32), ("meta", ctypes.c_void_p),
                ("hits", ctypes.c_uint64), ("misses", ctypes.c_uint64), ("speculate", ctypes.c_int32),
                ("spec_fills", ctypes.c_uint64)]


class Streamer(ctypes.Structure):
    _fields_ = [("host_arena", ctypes.c_void_p), ("host_shared", ctypes.c_void_p), ("blob_bytes", ctypes.c_uint64),
                ("n_experts", ctypes.c_int32), ("n_layers", ctypes.c_int32), ("arena_blobs", ctypes.c_int64),
                ("shared_blobs", ctypes.c_int64), ("slab", ctypes.c_void_p * 2), ("slab_blobs", ctypes.c_int32),
                ("cache", ctypes.POINTER(ExpertCache))]


EXPORTS = ["moe_blob_bytes", "moe_workspace_bytes", "moe_workspace_state_bytes", "moe_strerror", "moe_last_error", "moe_route",
           "moe_expert_forward", "moe_layer_step", "moe_stack_step", "moe_stack_step_noalloc", "moe_layer_plan", "moe_expert_gemv", "moe_workspace_grouping", "moe_stream_prefetch", "moe_stream_token",
           "moe_host_alloc", "moe_host_free", "moe_expert_cache_meta_bytes", "moe_expert_cache_reset"]

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            raise ImportError(f"libmoe.so is not built ({_SO}); run __graft_entry__.build()")
        L = ctypes.CDLL(_SO)
        i32, u64, sz, vp, cp = ctypes.c_int32, ctypes.c_uint64, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p
        L.moe_blob_bytes.restype = sz
        L.moe_blob_bytes.argtypes = [i32, i32, i32, i32]
        L.moe_workspace_bytes.restype = sz
        L.moe_workspace_bytes.argtypes = [ctypes.POINTER(LayerDesc), i32]
        L.moe_workspace_state_bytes.restype = sz
        L.moe_workspace_state_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
        L.moe_strerror.restype = cp
        L.moe_strerror.argtypes = [ctypes.c_int]
        L.moe_last_error.restype = cp
        L.moe_last_error.argtypes = []
        L.moe_route.restype = ctypes.c_int
        L.moe_route.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_expert_forward.restype = ctypes.c_int
        L.moe_expert_forward.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, vp, vp, vp, vp, sz, vp]
        L.moe_layer_step.restype = ctypes.c_int
        L.moe_layer_step.argtypes = [ctypes.POINTER(LayerDesc), vp, vp, i32, vp, vp, vp, sz, vp]
        L.moe_stack_step.restype = ctypes.c_int
        L.moe_stack_step.argtypes = [ctypes.POINTER(LayerDesc), i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.moe_expert_gemv.restype = ctypes.c_int
        L.moe_expert_gemv.argtypes = [ctypes.POINTER(LayerDesc), vp, i32, i32, vp, vp, vp]
        L.moe_stack_step_noalloc.restype = ctypes.c_int
        L.moe_stack_step_noalloc.argtypes = [ctypes.POINTER(LayerDesc), i32, vp, vp, vp, vp, vp, vp, vp]
        L.moe_layer_plan.restype = ctypes.c_int
        L.moe_layer_plan.argtypes = [ctypes.POINTER(LayerDesc), i32, vp]
        L.moe_workspace_grouping.restype = ctypes.c_int
        L.moe_workspace_grouping.argtypes = [ctypes.POINTER(LayerDesc), i32, vp]
        L.moe_stream_prefetch.restype = ctypes.c_int
        L.moe_stream_prefetch.argtypes = [ctypes.POINTER(Streamer), i32, vp, i32, i32, i32, vp, vp]
        L.moe_stream_token.restype = ctypes.c_int
        L.moe_stream_token.argtypes = [ctypes.POINTER(LayerDesc), i32, ctypes.POINTER(Streamer), vp, vp, vp, vp, vp, vp,
                                       vp, sz, vp, vp, vp]
        L.moe_host_alloc.restype = ctypes.c_int
        L.moe_host_alloc.argtypes = [sz, ctypes.POINTER(ctypes.c_void_p)]
        L.moe_host_free.restype = ctypes.c_int
        L.moe_host_free.argtypes = [vp]
        L.moe_expert_cache_meta_bytes.restype = sz
        L.moe_expert_cache_meta_bytes.argtypes = [i32, i32, i32]
        L.moe_expert_cache_reset.restype = ctypes.c_int
        L.moe_expert_cache_reset.argtypes = [ctypes.POINTER(ExpertCache), i32, i32]
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(rc, lib().moe_last_error().decode())


def make_desc(*, hidden, n_experts, top_k, inter, n_shared, bits, group=64, rms_eps=1e-6, router_w, gamma,
              experts=None, shared=None, slab=None, blob_bytes=None, expert_addr=None) -> LayerDesc:
    bb = blob_bytes if blob_bytes is not None else moe_blob_bytes(hidden, inter, bits, group)
    return LayerDesc(hidden, n_experts, top_k, inter, n_shared, bits, group, rms_eps, _ptr(router_w), _ptr(gamma),
                     _ptr(experts), _ptr(shared), _ptr(slab), bb, _ptr(expert_addr))


def moe_blob_bytes(hidden: int, inter: int, bits: int, group: int = 64) -> int:
    return int(lib().moe_blob_bytes(hidden, inter, bits, group))


def moe_workspace_bytes(desc: LayerDesc, n_tokens: int) -> int:
    return int(lib().moe_workspace_bytes(ctypes.byref(desc), n_tokens))


def moe_workspace_state_bytes(desc: LayerDesc) -> int:
    return int(lib().moe_workspace_state_bytes(ctypes.byref(desc)))


def moe_strerror(status: int) -> str:
    return lib().moe_strerror(status).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_route(desc, x, n_tokens, topk_idx, topk_w, logits, workspace, stream=None, ws_bytes=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_route(ctypes.byref(desc), _ptr(x), n_tokens, _ptr(topk_idx), _ptr(topk_w), _ptr(logits),
                           _ptr(workspace), ws_bytes, _stream(stream)))


def moe_expert_forward(desc, x, n_tokens, topk_idx, topk_w, y, workspace, stream=None, ws_bytes=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_expert_forward(ctypes.byref(desc), _ptr(x), n_tokens, _ptr(topk_idx), _ptr(topk_w), _ptr(y),
                                    _ptr(workspace), ws_bytes, _stream(stream)))


def moe_layer_step(desc, resid, x, n_tokens, topk_idx, topk_w, workspace, stream=None, ws_bytes=None) -> None:
    ws_bytes = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_layer_step(ctypes.byref(desc), _ptr(resid), _ptr(x), n_tokens, _ptr(topk_idx), _ptr(topk_w),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def moe_stack_step(descs, resid, x, topk_idx, topk_w, workspace, record=None, stream=None, ws_bytes=None) -> None:
    """descs: a ctypes array of LayerDesc."""
    ws_bytes = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    _check(lib().moe_stack_step(descs, len(descs), _ptr(resid), _ptr(x), _ptr(topk_idx), _ptr(topk_w), _ptr(record),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def moe_expert_gemv(desc, x, first: int, count: int, h, y, stream=None) -> None:
    _check(lib().moe_expert_gemv(ctypes.byref(desc), _ptr(x), first, count, _ptr(h), _ptr(y), _stream(stream)))


def moe_stack_step_noalloc(descs, resid, x, topk_idx, topk_w, record=None, flags=None, stream=None) -> None:
    """moe_stack_step on the library's own scratch (no workspace); descs: a
    ctypes array of LayerDesc; flags: None or a device int32/uint32 tensor of
    one element receiving the device error bits."""
    _check(lib().moe_stack_step_noalloc(descs, len(descs), _ptr(resid), _ptr(x), _ptr(topk_idx), _ptr(topk_w),
                                        _ptr(record), _ptr(flags), _stream(stream)))


def moe_layer_plan(desc, n_tokens: int = 1) -> dict:
    out = (ctypes.c_int32 * 7)()
    _check(lib().moe_layer_plan(ctypes.byref(desc), n_tokens, ctypes.cast(out, ctypes.c_void_p)))
    keys = ("fused", "grid", "block", "per_cu", "n_cu", "vgprs", "scratch")
    return dict(zip(keys, (int(v) for v in out)))


def moe_workspace_grouping(desc, n_tokens: int) -> dict:
    out = (ctypes.c_size_t * 6)()
    _check(lib().moe_workspace_grouping(ctypes.byref(desc), n_tokens, ctypes.cast(out, ctypes.c_void_p)))
    keys = ("count", "offset", "perm", "pos", "act", "n_act")
    return dict(zip(keys, (int(v) for v in out)))


def moe_stream_prefetch(streamer: Streamer, layer: int, expert_ids, slot: int, with_shared: bool, copy_stream,
                        done_event=None) -> None:
    ids = (ctypes.c_int32 * len(expert_ids))(*[int(e) for e in expert_ids])
    ev = None if done_event is None else (done_event if isinstance(done_event, int) else done_event.cuda_event)
    if done_event is not None and not ev:
        raise ValueError("done_event has no HIP event yet: record it once before handing it over")
    _check(lib().moe_stream_prefetch(ctypes.byref(streamer), layer, ctypes.cast(ids, ctypes.c_void_p),
                                     len(expert_ids), slot, 1 if with_shared else 0, _stream(copy_stream), ev))


def moe_stream_token(descs, streamer: Streamer, resid, x, topk_idx, topk_w, host_ids, workspace, compute_stream,
                     copy_stream, events, ws_bytes=None, record=None) -> None:
    """descs: a ctypes array of LayerDesc (streamed form); host_ids: pinned
    int32 tensor of K; events: five torch.cuda.Event; record: None or a
    device tensor [layers + 1][2][D]."""
    ws_bytes = workspace.numel() * workspace.element_size() if ws_bytes is None else ws_bytes
    if any(not e.cuda_event for e in events):
        raise ValueError("every event must have been recorded once (its HIP event is created lazily)")
    ev = (ctypes.c_void_p * 5)(*[e.cuda_event for e in events])
    _check(lib().moe_stream_token(descs, len(descs), ctypes.byref(streamer), _ptr(resid), _ptr(x), _ptr(topk_idx),
                                  _ptr(topk_w), _ptr(record), _ptr(host_ids), _ptr(workspace), ws_bytes,
                                  _stream(compute_stream),
                                  _stream(copy_stream), ctypes.cast(ev, ctypes.c_void_p)))


def moe_expert_cache_meta_bytes(n_slots: int, n_layers: int, n_experts: int) -> int:
    return int(lib().moe_expert_cache_meta_bytes(n_slots, n_layers, n_experts))


def moe_expert_cache_reset(cache: ExpertCache, n_layers: int, n_experts: int) -> None:
    _check(lib().moe_expert_cache_reset(ctypes.byref(cache), n_layers, n_experts))


class HostArena:
    """Pinned host memory from moe_host_alloc, exposed as a CPU uint8 tensor
    (`.tensor`) for filling and checking; freed when the object goes."""

    def __init__(self, nbytes: int):
        import numpy as np
        import torch
        p = ctypes.c_void_p()
        _check(lib().moe_host_alloc(nbytes, ctypes.byref(p)))
        self.ptr, self.nbytes = int(p.value), int(nbytes)
        arr = np.ctypeslib.as_array((ctypes.c_uint8 * self.nbytes).from_address(self.ptr))
        self.tensor = torch.from_numpy(arr)

    def data_ptr(self) -> int:
        return self.ptr

    def __del__(self):
        if getattr(self, "ptr", None):
            self.tensor = None
            lib().moe_host_free(self.ptr)
            self.ptr = None
