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

import torch

from . import (make_desc, moe_blob_bytes, moe_layer_step, moe_workspace_bytes)


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
        receives every layer's (resid, x) input and the final output."""
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
