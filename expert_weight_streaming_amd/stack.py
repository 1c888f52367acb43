"""Expert stacks on one GPU: device buffers and the per-token layer loop.

A ResidentStack keeps every layer's routed experts (canonical blobs), shared
expert, router and gamma in HBM and runs the layers with moe_layer_step; the
loop over layers can be captured once into a HIP graph and replayed per token
(the pages' deferred submission: the expert work is enqueued without the host
waiting, hakusoku.com, "主要技術").  Between layers the residual stream and
the normalised activation are handed on unchanged (attention is identity in
these workloads).
"""
from __future__ import annotations

import ctypes

import torch

from . import (HostArena, LayerDesc, make_desc, moe_blob_bytes, moe_layer_step, moe_stack_step, moe_workspace_bytes)


class ResidentStack:
    def __init__(self, *, hidden, n_experts, top_k, inter, bits, layers, n_shared=1, group=64, eps=1e-6,
                 n_tokens=1, device="cuda"):
        self.D, self.E, self.K, self.I = hidden, n_experts, top_k, inter
        self.bits, self.group, self.layers, self.n_shared, self.eps = bits, group, layers, n_shared, eps
        self.T = n_tokens
        self.bb = moe_blob_bytes(hidden, inter, bits, group)
        dev = torch.device(device)
        self.arena = torch.empty(layers * n_experts * self.bb, dtype=torch.uint8, device=dev)
        self.shared = torch.empty(max(1, layers * n_shared) * self.bb, dtype=torch.uint8, device=dev)
        self.router = torch.empty(layers, n_experts, hidden, dtype=torch.float32, device=dev)
        self.gamma = torch.ones(layers, hidden, dtype=torch.float32, device=dev)
        self.descs = [self._desc(l) for l in range(layers)]
        self.desc_array = (LayerDesc * layers)(*self.descs)
        self.ws_bytes = moe_workspace_bytes(self.descs[0], n_tokens)
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.topk_idx = torch.zeros(layers, n_tokens, top_k, dtype=torch.int32, device=dev)
        self.topk_w = torch.zeros(layers, n_tokens, top_k, dtype=torch.float32, device=dev)
        self.graph = None

    def _desc(self, l):
        return make_desc(hidden=self.D, n_experts=self.E, top_k=self.K, inter=self.I, n_shared=self.n_shared,
                         bits=self.bits, group=self.group, rms_eps=self.eps, router_w=self.router[l], gamma=self.gamma[l],
                         experts=self.arena.data_ptr() + l * self.E * self.bb,
                         shared=(self.shared.data_ptr() + l * self.bb) if self.n_shared else None,
                         blob_bytes=self.bb)

    def expert_ptr(self, l: int, e: int) -> int:
        return self.arena.data_ptr() + (l * self.E + e) * self.bb

    def shared_ptr(self, l: int) -> int:
        return self.shared.data_ptr() + l * self.bb

    def layer_step(self, l, resid, x, stream=None):
        moe_layer_step(self.descs[l], resid, x, self.T, self.topk_idx[l], self.topk_w[l], self.workspace, stream)

    def step(self, resid, x, record=None, stream=None):
        """All layers for one batch; record (optional) [layers+1][2][T][D]
        receives every layer's (resid, x) input and the final output.  One
        token runs as moe_stack_step (one persistent launch); a batch runs
        layer by layer."""
        if self.T == 1:
            moe_stack_step(self.desc_array, resid, x, self.topk_idx, self.topk_w, self.workspace, record, stream)
            return
        for l in range(self.layers):
            if record is not None:
                record[l, 0].copy_(resid)
                record[l, 1].copy_(x)
            self.layer_step(l, resid, x, stream)
        if record is not None:
            record[self.layers, 0].copy_(resid)
            record[self.layers, 1].copy_(x)

    def step_layers(self, resid, x, record=None, stream=None):
        """The same as step, one moe_layer_step call per layer."""
        for l in range(self.layers):
            if record is not None:
                record[l, 0].copy_(resid)
                record[l, 1].copy_(x)
            self.layer_step(l, resid, x, stream)
        if record is not None:
            record[self.layers, 0].copy_(resid)
            record[self.layers, 1].copy_(x)

    def capture(self, resid, x):
        """Capture step(resid, x) into a HIP graph (static buffers)."""
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                self.step(resid, x, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        self.graph = g
        return g


class StreamedStack:
    """Expert stack whose expert weights live in pinned host memory.

    Routers and gammas stay in HBM; per token and layer the K selected
    experts and the shared expert are copied host->device into one of two
    slab slots (moe_stream_token, hakusoku.com, "パイプライン概要": routing,
    then the experts' reads, then the forward).  arena_blobs < layers *
    n_experts aliases expert (l, e) onto host blob (l * E + e) mod
    arena_blobs: the bytes moved per token are unchanged, only the host
    footprint shrinks.
    """

    def __init__(self, *, hidden, n_experts, top_k, inter, bits, layers, n_shared=1, group=64, eps=1e-6,
                 arena_blobs=None, device="cuda"):
        from . import LayerDesc, Streamer
        self.D, self.E, self.K, self.I = hidden, n_experts, top_k, inter
        self.bits, self.group, self.layers, self.n_shared, self.eps = bits, group, layers, n_shared, eps
        self.bb = moe_blob_bytes(hidden, inter, bits, group)
        self.P = layers * n_experts if arena_blobs is None else int(arena_blobs)
        if not 0 < self.P <= layers * n_experts:
            raise ValueError(f"arena_blobs {self.P} outside 1..{layers * n_experts}")
        dev = torch.device(device)
        # moe_host_alloc, not torch's pinned allocator (which rounds every
        # request up to a power of two)
        self._arena = HostArena(self.P * self.bb)
        self._shared = HostArena(max(1, layers * n_shared) * self.bb)
        self.host_arena, self.host_shared = self._arena.tensor, self._shared.tensor
        self.router = torch.empty(layers, n_experts, hidden, dtype=torch.float32, device=dev)
        self.gamma = torch.ones(layers, hidden, dtype=torch.float32, device=dev)
        self.slab_blobs = top_k + n_shared
        self.slab = torch.empty(2, self.slab_blobs * self.bb, dtype=torch.uint8, device=dev)
        st = Streamer()
        st.host_arena, st.host_shared = self._arena.ptr, self._shared.ptr
        st.blob_bytes, st.n_experts, st.n_layers = self.bb, n_experts, layers
        st.arena_blobs, st.shared_blobs = self.P, max(1, layers * n_shared) if n_shared else 0
        st.slab[0], st.slab[1] = self.slab[0].data_ptr(), self.slab[1].data_ptr()
        st.slab_blobs = self.slab_blobs
        self.streamer = st
        descs = [make_desc(hidden=hidden, n_experts=n_experts, top_k=top_k, inter=inter, n_shared=n_shared, bits=bits,
                           group=group, rms_eps=eps, router_w=self.router[l], gamma=self.gamma[l], experts=None,
                           shared=None, slab=self.slab[0], blob_bytes=self.bb) for l in range(layers)]
        self.descs = (LayerDesc * layers)(*descs)
        self.ws_bytes = moe_workspace_bytes(descs[0], 1)
        self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=dev)
        self.topk_idx = torch.zeros(layers, 1, top_k, dtype=torch.int32, device=dev)
        self.topk_w = torch.zeros(layers, 1, top_k, dtype=torch.float32, device=dev)
        self.host_ids = torch.zeros(top_k, dtype=torch.int32, pin_memory=True)
        self.copy_stream = torch.cuda.Stream(device=dev)
        # events are created on their first record
        self.events = [torch.cuda.Event() for _ in range(5)]
        for e in self.events:
            e.record(self.copy_stream)
        self.copy_stream.synchronize()

    def host_blob(self, l: int, e: int) -> torch.Tensor:
        """The host bytes that expert (l, e) streams from."""
        p = (l * self.E + e) % self.P
        return self.host_arena[p * self.bb:(p + 1) * self.bb]

    def host_shared_blob(self, l: int) -> torch.Tensor:
        return self.host_shared[l * self.bb:(l + 1) * self.bb]

    def set_resident(self, l: int, experts, shared=None):
        """Hybrid residency: layer l's E expert blobs at `experts` in HBM (a
        device tensor or address, E * blob_bytes bytes in expert order) and
        its shared blob at `shared`; the token pipeline then runs the layer
        without copies or a host wait.  The bytes should equal what the layer
        streams (host_blob(l, e), host_shared_blob(l)) for the output to equal
        the streamed one.  experts=None makes the layer streamed again."""
        from . import make_desc
        resident = experts is not None
        self.descs[l] = make_desc(hidden=self.D, n_experts=self.E, top_k=self.K, inter=self.I, n_shared=self.n_shared,
                                  bits=self.bits, group=self.group, rms_eps=self.eps, router_w=self.router[l],
                                  gamma=self.gamma[l], experts=experts if resident else None,
                                  shared=shared if resident and self.n_shared else None,
                                  slab=None if resident else self.slab[0], blob_bytes=self.bb)

    def enable_cache(self, n_slots: int, speculate: bool = False):
        """An HBM cache of n_slots expert blobs for the streamed layers
        (moe_expert_cache): moe_stream_token copies cached experts device to
        device and fills the least recently used slot on a miss; with
        speculate, it also copies the previous token's selection of the next
        streamed layer into the cache ahead of that layer's routing.
        enable_cache(0) removes it.  Returns the cache (hits, misses,
        spec_fills)."""
        import numpy as np
        from . import ExpertCache, moe_expert_cache_meta_bytes, moe_expert_cache_reset
        if n_slots <= 0:
            self.streamer.cache = None
            self._cache = self._cache_slots = self._cache_meta = None
            return None
        self._cache_slots = torch.empty(n_slots * self.bb, dtype=torch.uint8, device=self.slab.device)
        # 8-byte aligned host block of the metadata's size
        self._cache_meta = np.zeros((moe_expert_cache_meta_bytes(n_slots, self.layers, self.E) + 7) // 8,
                                    dtype=np.uint64)
        c = ExpertCache()
        c.slots, c.n_slots, c.meta = self._cache_slots.data_ptr(), n_slots, self._cache_meta.ctypes.data
        c.speculate = 1 if speculate else 0
        moe_expert_cache_reset(c, self.layers, self.E)
        self._cache = c
        self.streamer.cache = ctypes.pointer(c)
        return c

    @property
    def cache(self):
        return getattr(self, "_cache", None)

    def zero_copy_descs(self):
        """Descriptors whose experts and shared expert are the pinned host
        arenas themselves: the kernels' own loads fetch each selected expert
        over the link (GPU-initiated streaming), so a token needs no copies
        and no host round trip and runs as one persistent moe_stack_step
        launch.  Layer l's E blobs must be contiguous in the arena, which
        holds when arena_blobs is a multiple of n_experts."""
        from . import make_desc
        if self.P % self.E:
            raise ValueError(f"arena_blobs {self.P} is not a multiple of n_experts {self.E}")
        descs = [make_desc(hidden=self.D, n_experts=self.E, top_k=self.K, inter=self.I, n_shared=self.n_shared,
                           bits=self.bits, group=self.group, rms_eps=self.eps, router_w=self.router[l],
                           gamma=self.gamma[l], experts=self._arena.ptr + (l * self.E) % self.P * self.bb,
                           shared=(self._shared.ptr + l * self.bb) if self.n_shared else None, blob_bytes=self.bb)
                 for l in range(self.layers)]
        return (LayerDesc * self.layers)(*descs)

    def zero_copy_hybrid_descs(self, n_resident, experts_of, shared_of):
        """zero_copy_descs with layers 0..n_resident-1 reading HBM instead:
        experts_of(l) / shared_of(l) give their device addresses (the same
        bytes as the host arena's for that layer).  One launch per token
        still, no copies."""
        from . import make_desc
        zc = self.zero_copy_descs()
        for l in range(n_resident):
            zc[l] = make_desc(hidden=self.D, n_experts=self.E, top_k=self.K, inter=self.I, n_shared=self.n_shared,
                              bits=self.bits, group=self.group, rms_eps=self.eps, router_w=self.router[l],
                              gamma=self.gamma[l], experts=experts_of(l),
                              shared=shared_of(l) if self.n_shared else None, blob_bytes=self.bb)
        return zc

    def step_zero_copy(self, resid, x, stream=None, descs=None, record=None):
        """One token through every layer reading the experts from host
        memory in the kernel (zero_copy_descs): one launch, no host wait."""
        if descs is None:
            if getattr(self, "_zc", None) is None:
                self._zc = self.zero_copy_descs()
            descs = self._zc
        moe_stack_step(descs, resid, x, self.topk_idx, self.topk_w, self.workspace, record, stream)

    # ---- per-expert residency through device address tables (one launch per token)
    def host_addr(self, l: int, e: int) -> int:
        return self._arena.ptr + ((l * self.E + e) % self.P) * self.bb

    def place_experts(self, n_slots: int, hot, shared_in_hbm: bool = True):
        """Per-expert residency: the (layer, expert) pairs in `hot` (most
        wanted first; at most n_slots of them) get a copy in an HBM pool of
        n_slots blobs, every other expert is read from the pinned host arena
        by the kernel itself.  Each layer's descriptor carries a device table
        of its experts' blob addresses (address-table mode), so a token is
        still one moe_stack_step launch with no copies and no host wait.
        With shared_in_hbm the layers' shared experts are copied to HBM too.
        Returns the set of (layer, expert) pairs placed in HBM."""
        import numpy as np
        from . import make_desc
        dev = self.slab.device
        if getattr(self, "_pool", None) is None or self._pool.numel() < n_slots * self.bb:
            self._pool = torch.empty(max(1, n_slots) * self.bb, dtype=torch.uint8, device=dev)
        if shared_in_hbm and self.n_shared and getattr(self, "_shared_hbm", None) is None:
            self._shared_hbm = torch.empty(self.layers * self.bb, dtype=torch.uint8, device=dev)
            self._shared_hbm.copy_(self.host_shared[:self.layers * self.bb])
        addr = np.empty((self.layers, self.E), dtype=np.uint64)
        for l in range(self.layers):
            for e in range(self.E):
                addr[l, e] = self.host_addr(l, e)
        placed = []
        for slot, (l, e) in enumerate(list(hot)[:n_slots]):
            self._pool[slot * self.bb:(slot + 1) * self.bb].copy_(self.host_blob(l, e))
            addr[l, e] = self._pool.data_ptr() + slot * self.bb
            placed.append((l, e))
        self._tables = torch.from_numpy(addr.view(np.int64)).to(dev)
        sh = self._shared_hbm if shared_in_hbm and self.n_shared else None
        descs = []
        for l in range(self.layers):
            shared = (sh.data_ptr() + l * self.bb) if sh is not None else (
                (self._shared.ptr + l * self.bb) if self.n_shared else None)
            descs.append(make_desc(hidden=self.D, n_experts=self.E, top_k=self.K, inter=self.I,
                                   n_shared=self.n_shared, bits=self.bits, group=self.group, rms_eps=self.eps,
                                   router_w=self.router[l], gamma=self.gamma[l], shared=shared,
                                   expert_addr=self._tables[l], blob_bytes=self.bb))
        self._table_descs = (LayerDesc * self.layers)(*descs)
        torch.cuda.synchronize()
        return set(placed)

    def step_placed(self, resid, x, stream=None, record=None):
        """One token through every layer in address-table mode (after
        place_experts): one launch, HBM or host per expert."""
        moe_stack_step(self._table_descs, resid, x, self.topk_idx, self.topk_w, self.workspace, record, stream)

    def resident_layers(self) -> list[int]:
        return [l for l in range(self.layers) if self.descs[l].experts]

    def step(self, resid, x, stream=None, record=None):
        """One token (resid, x: [1][D] device) through every layer; returns
        when the last layer is enqueued on `stream`.  record (optional)
        [layers+1][2][1][D] receives every layer's (resid, x) input and the
        output."""
        from . import moe_stream_token
        cs = torch.cuda.current_stream() if stream is None else stream
        moe_stream_token(self.descs, self.streamer, resid, x, self.topk_idx, self.topk_w, self.host_ids,
                         self.workspace, cs, self.copy_stream, self.events, record=record)
