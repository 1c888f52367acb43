"""The C ABI: libmoe.so loads, exports every symbol include/moe.h declares,
and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

import expert_weight_streaming_amd as ews

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(moe_\w+)\s*\(", src, re.M)))


def test_header_matches_binding():
    assert _declared() == sorted(ews.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(ews._SO)
    for name in _declared():
        assert hasattr(L, name), name


def test_blob_bytes():
    assert ews.moe_blob_bytes(4096, 1024, 4, 64) == 7077888
    assert ews.moe_blob_bytes(4096, 1024, 2, 64) == 3932160
    assert ews.moe_blob_bytes(256, 128, 4, 64) == 55296
    assert ews.moe_blob_bytes(4096, 1024, 3, 64) == 0
    assert ews.moe_blob_bytes(4096, 1000, 4, 64) == 0
    assert ews.moe_blob_bytes(4096, 1024, 4, 32) == 0


def _desc(**kw):
    base = dict(hidden=256, n_experts=16, top_k=2, inter=128, n_shared=1, bits=4, router_w=4096, gamma=8192,
                experts=16384, shared=32768)
    base.update(kw)
    return ews.make_desc(**base)


def test_workspace_state_is_independent_of_token_count():
    """The state a call hands to the next (flags, counters, the fused step's
    epochs and exchange words) leads the workspace at fixed offsets; every
    per-call region of any token count lies after it."""
    for shape in (dict(), dict(hidden=4096, n_experts=512, top_k=4, inter=1024), dict(bits=2, top_k=8, n_experts=64),
                  dict(n_shared=0, hidden=448, inter=320)):
        d = _desc(**shape)
        d.blob_bytes = ews.moe_blob_bytes(d.hidden, d.inter, d.bits, 64)
        state = ews.moe_workspace_state_bytes(d)
        assert state > 0 and state % 256 == 0
        S = d.top_k + d.n_shared
        # epochs of up to 1024 workgroups and the tagged logits, h, residual rows and sums of squares
        assert state >= 1024 * 64 + 8 * (1024 + d.n_experts + S * d.inter + d.hidden)
        prev = 0
        for T in range(1, 65):
            total = ews.moe_workspace_bytes(d, T)
            assert total > state and total >= prev
            prev = total
            if T >= 2:
                assert min(ews.moe_workspace_grouping(d, T).values()) >= state
    assert ews.moe_workspace_state_bytes(_desc(bits=3)) == 0


def test_workspace_bytes():
    d = _desc()
    n = ews.moe_workspace_bytes(d, 1)
    assert n > 0 and n % 256 == 0
    assert ews.moe_workspace_bytes(_desc(bits=3), 1) == 0
    assert ews.moe_workspace_bytes(_desc(top_k=17), 1) == 0
    assert ews.moe_workspace_bytes(_desc(top_k=9, n_experts=32), 1) == 0
    assert ews.moe_workspace_bytes(d, 0) == 0


@pytest.mark.parametrize("bad", [dict(bits=3), dict(group=32), dict(hidden=100), dict(inter=0), dict(top_k=0),
                                 dict(top_k=17), dict(n_shared=2), dict(router_w=4097), dict(gamma=None),
                                 dict(experts=16385), dict(shared=None), dict(blob_bytes=12345),
                                 dict(experts=None, slab=None), dict(n_experts=5000)])
def test_bad_descriptor_rejected(bad):
    d = _desc(**bad)
    L = ews.lib()
    rc = L.moe_route(ctypes.byref(d), 65536, 1, 65536, 65536, None, 65536 * 4, 1 << 20, None)
    assert rc == ews.MOE_EINVAL, (bad, rc, ews.moe_last_error())
    assert ews.moe_last_error()


def test_bad_buffers_rejected():
    d = _desc()
    L = ews.lib()
    ws = ews.moe_workspace_bytes(d, 1)
    assert L.moe_route(ctypes.byref(d), None, 1, 65536, 65536, None, 1 << 20, ws, None) == ews.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 65540, 1, 65536, 65536, None, 1 << 20, ws, None) == ews.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 65536, 1, 65536, 65536, None, (1 << 20) + 16, ws, None) == ews.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 65536, 1, 65536, 65536, None, 1 << 20, ws - 1, None) == ews.MOE_EINVAL
    assert L.moe_route(ctypes.byref(d), 65536, 0, 65536, 65536, None, 1 << 20, ws, None) == ews.MOE_EINVAL
    assert L.moe_expert_forward(ctypes.byref(d), 65536, 1, 65536, 65536, None, 1 << 20, ws, None) == ews.MOE_EINVAL
    # resid and x overlapping
    assert L.moe_layer_step(ctypes.byref(d), 65536, 65536 + 512, 1, 4096, 4096, 1 << 20, ws, None) == ews.MOE_EINVAL
    assert L.moe_layer_step(None, 65536, 1 << 19, 1, 4096, 4096, 1 << 20, ws, None) == ews.MOE_EINVAL


def test_streamer_misuse_rejected():
    st = ews.Streamer()
    L = ews.lib()
    ids = (ctypes.c_int32 * 4)(0, 1, 2, 3)
    ip = ctypes.cast(ids, ctypes.c_void_p)
    assert L.moe_stream_prefetch(ctypes.byref(st), 0, ip, 4, 0, 1, None, None) == ews.MOE_ESTATE  # no arena
    st.host_arena, st.host_shared, st.blob_bytes = 4096, 8192, 7077888
    st.n_experts, st.n_layers, st.arena_blobs, st.shared_blobs, st.slab_blobs = 512, 60, 30720, 60, 5
    st.slab[0], st.slab[1] = 1 << 20, 1 << 21
    assert L.moe_stream_prefetch(ctypes.byref(st), 0, ip, 4, 2, 1, None, None) == ews.MOE_ESTATE  # slot
    assert L.moe_stream_prefetch(ctypes.byref(st), 60, ip, 4, 0, 1, None, None) == ews.MOE_ESTATE  # layer
    assert L.moe_stream_prefetch(ctypes.byref(st), 0, ip, 5, 0, 1, None, None) == ews.MOE_ESTATE   # too many
    bad = (ctypes.c_int32 * 4)(0, 1, 512, 3)
    assert L.moe_stream_prefetch(ctypes.byref(st), 0, ctypes.cast(bad, ctypes.c_void_p), 4, 0, 1, None,
                                 None) == ews.MOE_ESTATE
    assert L.moe_stream_prefetch(None, 0, ip, 4, 0, 1, None, None) == ews.MOE_ESTATE


def test_strerror():
    for s in (0, -1, -2, -3, -4):
        assert ews.moe_strerror(s)


def test_stream_token_misuse_rejected():
    """moe_stream_token validates everything before enqueueing anything."""
    L = ews.lib()
    D, E, K, I = 256, 16, 2, 128
    bb = ews.moe_blob_bytes(D, I, 4, 64)
    st = ews.Streamer()
    st.host_arena, st.host_shared, st.blob_bytes = 4096, 8192, bb
    st.n_experts, st.n_layers, st.arena_blobs, st.shared_blobs, st.slab_blobs = E, 2, 2 * E, 2, K + 1
    st.slab[0], st.slab[1] = 1 << 20, 1 << 21
    mk = lambda **kw: ews.make_desc(**{**dict(hidden=D, n_experts=E, top_k=K, inter=I, n_shared=1, bits=4,
                                               router_w=1 << 12, gamma=1 << 13, slab=1 << 20), **kw})
    descs = (ews.LayerDesc * 2)(mk(), mk())
    ev = (ctypes.c_void_p * 5)(*([1 << 4] * 5))
    evp = ctypes.cast(ev, ctypes.c_void_p)
    ws = 1 << 16
    args = lambda d, n, s, e, rec=None: (d, n, s, 1 << 8, 1 << 9, 1 << 10, 1 << 11, rec, 1 << 14, ws, 1 << 30, None,
                                         None, e)
    assert L.moe_stream_token(*args(descs, 0, ctypes.byref(st), evp)) == ews.MOE_EINVAL       # no layers
    assert L.moe_stream_token(*args(descs, 3, ctypes.byref(st), evp)) == ews.MOE_ESTATE       # > streamer layers
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), None)) == ews.MOE_EINVAL      # events
    bad_ev = (ctypes.c_void_p * 5)(1, 1, None, 1, 1)
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), ctypes.cast(bad_ev, ctypes.c_void_p))) \
        == ews.MOE_EINVAL
    resident = (ews.LayerDesc * 2)(mk(), mk(experts=1 << 20))
    assert L.moe_stream_token(*args(resident, 2, ctypes.byref(st), evp)) == ews.MOE_EINVAL    # resident, no shared
    other_k = (ews.LayerDesc * 2)(mk(), mk(top_k=3))
    assert L.moe_stream_token(*args(other_k, 2, ctypes.byref(st), evp)) == ews.MOE_EINVAL
    st.slab_blobs = K
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), evp)) == ews.MOE_ESTATE       # slab size
    st.slab_blobs = K + 1
    small_ws = args(descs, 2, ctypes.byref(st), evp)
    small_ws = small_ws[:10] + (256,) + small_ws[11:]
    assert L.moe_stream_token(*small_ws) == ews.MOE_EINVAL                                    # workspace
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), evp, (1 << 20) + 8)) == ews.MOE_EINVAL  # record
    # an expert cache that was not reset for this streamer
    meta = (ctypes.c_uint64 * 64)()
    cache = ews.ExpertCache(1 << 22, 4, ctypes.addressof(meta), 0, 0)
    st.cache = ctypes.pointer(cache)
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), evp)) == ews.MOE_ESTATE
    ews.moe_expert_cache_reset(cache, 1, E)                                                  # another layer count
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), evp)) == ews.MOE_ESTATE
    cache.slots = None
    assert L.moe_stream_token(*args(descs, 2, ctypes.byref(st), evp)) == ews.MOE_ESTATE


def test_address_table_mode_validation():
    """Address-table descriptors: only with experts and slab NULL, one
    token, and not for moe_expert_forward (nothing is enqueued)."""
    L = ews.lib()
    D, E, K, I = 256, 16, 2, 128
    mk = lambda **kw: ews.make_desc(**{**dict(hidden=D, n_experts=E, top_k=K, inter=I, n_shared=1, bits=4,
                                               router_w=1 << 12, gamma=1 << 13, shared=1 << 14,
                                               expert_addr=1 << 15), **kw})
    ws = ews.moe_workspace_bytes(mk(), 1)
    assert ws > 0 and ews.moe_workspace_bytes(mk(), 2) == 0           # one token only
    assert ews.moe_workspace_bytes(mk(experts=1 << 16), 1) == 0        # excludes experts
    assert ews.moe_workspace_bytes(mk(slab=1 << 16), 1) == 0           # and slab
    assert ews.moe_workspace_bytes(mk(shared=None), 1) == 0            # shared blob needed
    assert ews.moe_workspace_bytes(mk(expert_addr=(1 << 15) + 8), 1) == 0  # alignment
    d = mk()
    rc = L.moe_expert_forward(ctypes.byref(d), 1 << 20, 1, 1 << 21, 1 << 22, 1 << 23, 1 << 24, ws, None)
    assert rc == ews.MOE_EUNSUPPORTED


def test_expert_cache_meta_and_reset():
    L = ews.lib()
    assert ews.moe_expert_cache_meta_bytes(0, 2, 16) == 0
    assert ews.moe_expert_cache_meta_bytes(4, 0, 16) == 0
    n1 = ews.moe_expert_cache_meta_bytes(4, 2, 16)
    # grows by 4 bytes per indexed blob (a layer's 16 routed experts and its
    # shared one) and per remembered selection (8 per layer), 16 per slot
    assert ews.moe_expert_cache_meta_bytes(4, 3, 16) - n1 == (17 + 8) * 4
    assert ews.moe_expert_cache_meta_bytes(5, 2, 16) - n1 == 16
    meta = (ctypes.c_uint64 * (n1 // 8 + 1))()
    c = ews.ExpertCache(1 << 22, 4, ctypes.addressof(meta), 7, 9, 1, 5)
    ews.moe_expert_cache_reset(c, 2, 16)
    assert (c.hits, c.misses, c.spec_fills, c.speculate) == (0, 0, 0, 1)
    assert L.moe_expert_cache_reset(None, 2, 16) == ews.MOE_EINVAL
    for bad in (ews.ExpertCache(None, 4, ctypes.addressof(meta), 0, 0), ews.ExpertCache(1 << 22, 4, None, 0, 0),
                ews.ExpertCache(1 << 22, 0, ctypes.addressof(meta), 0, 0)):
        assert L.moe_expert_cache_reset(ctypes.byref(bad), 2, 16) == ews.MOE_EINVAL
    assert L.moe_expert_cache_reset(ctypes.byref(c), 0, 16) == ews.MOE_EINVAL
    odd = ews.ExpertCache(1 << 22, 4, ctypes.addressof(meta) + 4, 0, 0)
    assert L.moe_expert_cache_reset(ctypes.byref(odd), 2, 16) == ews.MOE_EINVAL


def test_host_alloc_rejects_bad_arguments():
    L = ews.lib()
    p = ctypes.c_void_p()
    assert L.moe_host_alloc(0, ctypes.byref(p)) == ews.MOE_EINVAL
    assert L.moe_host_alloc(16, None) == ews.MOE_EINVAL
    assert L.moe_host_free(None) == ews.MOE_OK


def test_expert_gemv_validation():
    """moe_expert_gemv checks its range, its layer mode and its buffers before
    enqueueing anything."""
    L = ews.lib()
    d = _desc()
    ok = dict(x=1 << 20, h=1 << 21, y=1 << 22)
    call = lambda desc, first, count, x=ok["x"], h=ok["h"], y=ok["y"]: L.moe_expert_gemv(
        ctypes.byref(desc), x, first, count, h, y, None)
    assert call(d, -1, 2) == ews.MOE_EINVAL
    assert call(d, 0, 0) == ews.MOE_EINVAL
    assert call(d, 10, 7) == ews.MOE_EINVAL
    assert call(d, 0, 2, x=None) == ews.MOE_EINVAL
    assert call(d, 0, 2, h=(1 << 21) + 4) == ews.MOE_EINVAL
    assert call(_desc(experts=None, slab=1 << 23), 0, 2) == ews.MOE_EINVAL
    assert call(_desc(bits=3), 0, 2) == ews.MOE_EINVAL


def test_noalloc_scratch_holds_every_one_token_shape():
    """The library's scratch (1 MiB per device) holds the one-token workspace
    of the largest valid shape; bad arguments are refused before any device
    work."""
    d = _desc(hidden=8192, n_experts=4096, top_k=8, inter=4096)
    d.blob_bytes = ews.moe_blob_bytes(8192, 4096, 4, 64)
    assert 0 < ews.moe_workspace_bytes(d, 1) <= 1 << 20
    L = ews.lib()
    descs = (ews.LayerDesc * 1)(_desc())
    assert L.moe_stack_step_noalloc(None, 1, 1 << 20, 1 << 21, 1 << 22, 1 << 23, None, None, None) == ews.MOE_EINVAL
    assert L.moe_stack_step_noalloc(descs, 0, 1 << 20, 1 << 21, 1 << 22, 1 << 23, None, None, None) == ews.MOE_EINVAL
    assert L.moe_stack_step_noalloc(descs, 1, 1 << 20, 1 << 20, 1 << 22, 1 << 23, None, None, None) == ews.MOE_EINVAL
    assert L.moe_stack_step_noalloc(descs, 1, 1 << 20, 1 << 21, 1 << 22, 1 << 23, None, (1 << 24) + 2,
                                    None) == ews.MOE_EINVAL

