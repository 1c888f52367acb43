"""Python face of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
benchmark's cpu_baseline leg may import this package.  It is a plain fp64
evaluation of the MoE block on the canonical expert blobs and shares no code
with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")


def build(force: bool = False) -> None:
    if force or not os.path.exists(_SO):
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off", "-std=c99",
             os.path.join(_HERE, "oracle.c"), "-o", _SO + ".tmp", "-lm"])
        os.replace(_SO + ".tmp", _SO)


class _Args(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("E", ctypes.c_int32), ("K", ctypes.c_int32), ("I", ctypes.c_int32),
                ("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("eps", ctypes.c_double),
                ("router", ctypes.c_void_p), ("gamma", ctypes.c_void_p), ("blobs", ctypes.c_void_p),
                ("shared", ctypes.c_void_p)]


_L = None


def load(path: str | None = None):
    """Load the oracle library (or a variant built at `path`)."""
    global _L
    if path is None and _L is not None:
        return _L
    if path is None and not os.path.exists(_SO):
        build()
    L = ctypes.CDLL(path or _SO)
    i32, u64, dbl, vp = ctypes.c_int32, ctypes.c_uint64, ctypes.c_double, ctypes.c_void_p
    L.orc_set_threads.argtypes = [ctypes.c_int]
    L.orc_get_threads.restype = ctypes.c_int
    L.orc_blob_bytes.restype = u64
    L.orc_blob_bytes.argtypes = [ctypes.c_int] * 4
    L.orc_q.restype = ctypes.c_int
    L.orc_q.argtypes = [vp] + [ctypes.c_int] * 6
    L.orc_sb.argtypes = [vp] + [ctypes.c_int] * 7 + [vp, vp]
    L.orc_w.restype = dbl
    L.orc_w.argtypes = [vp] + [ctypes.c_int] * 7
    L.orc_row_dot.restype = dbl
    L.orc_row_dot.argtypes = [vp] + [ctypes.c_int] * 6 + [vp, ctypes.c_int]
    L.orc_router.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
    L.orc_topk.restype = ctypes.c_int
    L.orc_topk.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp, vp]
    L.orc_route_weights.argtypes = [vp, vp, ctypes.c_int, vp]
    L.orc_expert.argtypes = [vp] + [ctypes.c_int] * 4 + [vp, vp, vp]
    L.orc_resnorm.argtypes = [vp, vp, vp, ctypes.c_int, dbl, vp, vp]
    L.orc_layer.restype = ctypes.c_int
    L.orc_layer.argtypes = [ctypes.POINTER(_Args)] + [vp] * 10
    L.orc_group.argtypes = [vp, ctypes.c_int, ctypes.c_int, ctypes.c_int, vp, vp, vp]
    if path is None:
        _L = L
    return L


def _p(a: np.ndarray) -> int:
    return a.ctypes.data


def set_threads(n: int) -> None:
    load().orc_set_threads(int(n))


def get_threads() -> int:
    return int(load().orc_get_threads())


def blob_bytes(D, I, bits, group, L=None) -> int:
    return int((L or load()).orc_blob_bytes(D, I, bits, group))


def q(blob, D, I, bits, mat, row, col, L=None) -> int:
    return int((L or load()).orc_q(_p(blob), D, I, bits, mat, row, col))


def sb(blob, D, I, bits, group, mat, row, col, L=None):
    s, b = ctypes.c_double(), ctypes.c_double()
    (L or load()).orc_sb(_p(blob), D, I, bits, group, mat, row, col, ctypes.byref(s), ctypes.byref(b))
    return s.value, b.value


def w(blob, D, I, bits, group, mat, row, col, L=None) -> float:
    return float((L or load()).orc_w(_p(blob), D, I, bits, group, mat, row, col))


def row_dot(blob, D, I, bits, group, mat, row, x, form, L=None) -> float:
    x = np.ascontiguousarray(x, dtype=np.float64)
    return float((L or load()).orc_row_dot(_p(blob), D, I, bits, group, mat, row, _p(x), form))


def router(Wr, x, L=None) -> np.ndarray:
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    E, D = Wr.shape
    x = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(E, dtype=np.float64)
    (L or load()).orc_router(_p(Wr), E, D, _p(x), _p(out))
    return out


def topk(logits, K, L=None):
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    sel = np.empty(K, dtype=np.int32)
    gap = ctypes.c_double()
    rc = (L or load()).orc_topk(_p(logits), logits.size, K, _p(sel), ctypes.byref(gap))
    if rc:
        raise ValueError("orc_topk: bad K")
    return sel, gap.value


def route_weights(logits, sel, L=None) -> np.ndarray:
    logits = np.ascontiguousarray(logits, dtype=np.float64)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    out = np.empty(sel.size, dtype=np.float64)
    (L or load()).orc_route_weights(_p(logits), _p(sel), sel.size, _p(out))
    return out


def expert(blob, D, I, bits, group, x, L=None):
    x = np.ascontiguousarray(x, dtype=np.float64)
    h = np.empty(I, dtype=np.float64)
    y = np.empty(D, dtype=np.float64)
    (L or load()).orc_expert(_p(blob), D, I, bits, group, _p(x), _p(h), _p(y))
    return h, y


def resnorm(r, c, gamma, eps, L=None):
    r = np.ascontiguousarray(r, dtype=np.float64)
    c = np.ascontiguousarray(c, dtype=np.float64)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    ro = np.empty_like(r)
    xo = np.empty_like(r)
    (L or load()).orc_resnorm(_p(r), _p(c), _p(gamma), r.size, eps, _p(ro), _p(xo))
    return ro, xo


def group(topk_idx, E, L=None):
    idx = np.ascontiguousarray(topk_idx, dtype=np.int32)
    T, K = idx.shape
    count = np.empty(E, dtype=np.int32)
    offset = np.empty(E + 1, dtype=np.int32)
    perm = np.empty(T * K, dtype=np.int32)
    (L or load()).orc_group(_p(idx), T, K, E, _p(count), _p(offset), _p(perm))
    return count, offset, perm


def layer(D, E, K, I, bits, group_size, eps, Wr, gamma, blob_of, shared_blob, r, x, forced_sel=None, L=None):
    """One MoE layer for one token (oracle.c: orc_layer).

    blob_of(e) returns expert e's canonical blob (uint8); only the selected
    experts are requested.  The routing is the oracle's own top-K unless
    forced_sel (a valid selection, e.g. the other side's choice at a near tie)
    is given.  Returns a dict of fp64 arrays plus sel (int32) and gap.
    """
    L = L or load()
    Wr = np.ascontiguousarray(Wr, dtype=np.float32)
    gamma = np.ascontiguousarray(gamma, dtype=np.float32)
    r32 = np.ascontiguousarray(r, dtype=np.float32)
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    logits0 = router(Wr, x32.astype(np.float64), L=L)
    sel0, gap = topk(logits0, K, L=L)
    sel = sel0 if forced_sel is None else np.ascontiguousarray(forced_sel, dtype=np.int32)
    keep = {int(e): np.ascontiguousarray(blob_of(int(e)), dtype=np.uint8) for e in sel}
    table = (ctypes.c_void_p * E)()
    for e, b in keep.items():
        table[e] = b.ctypes.data
    args = _Args(D, E, K, I, bits, group_size, eps, Wr.ctypes.data, gamma.ctypes.data,
                 ctypes.cast(table, ctypes.c_void_p).value,
                 None if shared_blob is None else np.ascontiguousarray(shared_blob).ctypes.data)
    logits = np.empty(E, np.float64)
    sel_out = np.empty(K, np.int32)
    wts = np.empty(K, np.float64)
    gapc = ctypes.c_double()
    c = np.empty(D, np.float64)
    ro = np.empty(D, np.float64)
    xo = np.empty(D, np.float64)
    rc = L.orc_layer(ctypes.byref(args), _p(r32), _p(x32), _p(sel), _p(logits), _p(sel_out), _p(wts),
                     ctypes.byref(gapc), _p(c), _p(ro), _p(xo))
    if rc:
        raise ValueError("orc_layer: bad arguments")
    return {"logits": logits, "sel": sel_out, "w": wts, "gap": gap, "c": c, "r": ro, "x": xo,
            "oracle_sel": sel0}
