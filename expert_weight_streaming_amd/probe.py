"""Per-layer timeline of the persistent stack kernel.

The timeline build of libmoe (moe_stack.hip compiled with
-DMOE_STACK_PROBE, linked as libmoe_probe.so next to the package's objects)
stores the device's constant-rate clock (s_memrealtime, 100 MHz) at fixed
points of every layer, per workgroup and wave.  This tool runs a stack of a
seeded workload through that build and prints, per point, the time from the
layer's start (the earliest workgroup's first stamp of the layer) as medians
over workgroups and layers.  The stamps perturb the kernel a little (one
scalar clock read and one store per point and wave); the figures locate the
time, the untouched library's timing is the one to quote.

    python -m expert_weight_streaming_amd.probe --config stack4 --tokens 8
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys

import numpy as np

from . import _build

PROBE_SO = os.path.join(_build.HERE, "libmoe_probe.so")
POINTS = 16
TICK_NS = 10.0  # s_memrealtime: 100 MHz

LABELS = {
    1: "previous layer's residual rows and sums of squares all arrived",
    2: "x and its digit table built",
    3: "router rows done",
    4: "logits stored",
    5: "top-K done (wave 0) / shared gate/up rows done (other waves)",
    6: "routed gate/up unit stored",
    7: "down rows requested",
    8: "h of every slot arrived, digit tables built",
    9: "after the block barrier (all h tables complete)",
    10: "down rows combined",
    11: "residual rows and sum of squares stored (wave 0)",
}


def build(force: bool = False) -> str:
    os.makedirs(os.path.dirname(PROBE_SO), exist_ok=True)
    return _build.build(force=force, extra=["-DMOE_STACK_PROBE"], out=PROBE_SO)


def run(config: str, tokens: int, layers: int | None = None, lib: str | None = None):
    """lib: a timeline build of the library to load instead of the package's
    own (libmoe_probe.so)."""
    import torch
    import expert_weight_streaming_amd as ews
    so = os.path.abspath(lib) if lib else build()
    if ews._lib is not None and ews._SO != so:
        raise RuntimeError("the library is loaded already; run the timeline in a fresh process")
    ews._SO = so  # this process runs the timeline build
    L = ews.lib()
    L.moe_probe_set.restype = ctypes.c_int
    L.moe_probe_set.argtypes = [ctypes.c_void_p]
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    sys.path.insert(0, root)
    import seedgen
    from .stack import ResidentStack
    cfg = seedgen.CONFIGS[config]
    n = layers or cfg.layers
    st = ResidentStack(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits, layers=n,
                       n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps)
    s = torch.cuda.current_stream().cuda_stream
    for l in range(n):
        seedgen.dev_blobs(cfg, l, 0, cfg.E, st.expert_ptr(l, 0), s)
        seedgen.dev_blobs(cfg, l, seedgen.SHARED_ID, 1, st.shared_ptr(l), s)
        st.router[l].copy_(torch.from_numpy(seedgen.router(cfg, l)))
    plan = ews.moe_layer_plan(st.descs[0])
    grid = plan["grid"]
    probe = torch.zeros(n, grid, 8, POINTS, dtype=torch.int64, device="cuda")
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    r, x = v.clone(), v.clone()
    stamps, ms = [], []
    for t in range(tokens):
        probe.zero_()
        L.moe_probe_set(probe.data_ptr() if t >= 2 else None)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r.copy_(x)
        e0.record()
        st.step(r, x)
        e1.record()
        torch.cuda.synchronize()
        if t >= 2:
            stamps.append(probe.cpu().numpy())
            ms.append(e0.elapsed_time(e1))
    L.moe_probe_set(None)
    return cfg, plan, np.stack(stamps), ms


def summarize(cfg, plan, stamps, ms, skip=2):
    """stamps [tokens][layers][grid][8][POINTS] -> markdown lines."""
    T, n = stamps.shape[0], stamps.shape[1]
    rel = []
    for t in range(T):
        for l in range(skip, n):
            s = stamps[t, l].astype(np.int64)
            t0 = s[:, :, 0].min()
            rel.append((s - t0) * TICK_NS / 1e3)  # us from the layer's start
    rel = np.stack(rel)  # [samples][grid][8][POINTS]
    layer_us = []
    for t in range(T):
        starts = stamps[t, :, :, :, 0].min(axis=(1, 2))
        layer_us.append(np.diff(starts[skip:]) * TICK_NS / 1e3)
    layer_us = np.concatenate(layer_us)
    lines = [f"workload {cfg.name}: {n} layers, grid {plan['grid']} x {plan['block']} threads, "
             f"{np.mean(ms) * 1e3:.1f} us per token launch (events) = {np.mean(ms) * 1e3 / n:.2f} us per layer; "
             f"layer starts {np.median(layer_us):.2f} us apart (median of {layer_us.size})",
             "",
             "| point | us from layer start: wave 0 | waves 1-7 (median of waves) | slowest wave of a block: median / max over blocks |",
             "|---|---:|---:|---:|"]
    for p, label in LABELS.items():
        w0 = np.median(rel[:, :, 0, p])
        wo = np.median(rel[:, :, 1:, p])
        bmax = rel[:, :, :, p].max(axis=2)
        lines.append(f"| {p}. {label} | {w0:.2f} | {wo:.2f} | {np.median(bmax):.2f} / {np.median(bmax.max(axis=1)):.2f} |")
    # which workgroups are late: per point, each block's slowest wave against
    # the median block of the same layer, averaged over layers; by
    # workgroup id modulo 8 (the dispatcher's round-robin over the XCDs) and
    # the agreement of the per-block means between two halves of the samples
    G = rel.shape[1]
    lines += ["", "Late workgroups: per point, a block's slowest wave minus the median block of the same layer "
              "(us, mean over layers), by workgroup id mod 8; r: correlation of the per-block means between "
              "two halves of the layers (near 1: the same blocks are late every layer).", "",
              "| point | slowest block, median over layers | " + " | ".join(f"id%8={x}" for x in range(8)) + " | r |",
              "|---|---:|" + "---:|" * 8 + "---:|"]
    for p in LABELS:
        bmax = rel[:, :, :, p].max(axis=2)
        late = bmax - np.median(bmax, axis=1, keepdims=True)
        mean_late = late.mean(axis=0)
        by = [mean_late[np.arange(G) % 8 == x].mean() for x in range(8)]
        r = np.corrcoef(late[::2].mean(axis=0), late[1::2].mean(axis=0))[0, 1]
        lines.append(f"| {p} | {np.median(late.max(axis=1)):.2f} | " + " | ".join(f"{v:+.2f}" for v in by) + f" | {r:.2f} |")
    return lines


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--config", default="stack4")
    ap.add_argument("--tokens", type=int, default=6)
    ap.add_argument("--layers", type=int, default=None)
    ap.add_argument("--build-only", action="store_true")
    ap.add_argument("--lib", default=None, help="another timeline build of the library to run")
    args = ap.parse_args()
    if args.build_only:
        print(build(force=True))
        return
    cfg, plan, stamps, ms = run(args.config, args.tokens, args.layers, args.lib)
    print("\n".join(summarize(cfg, plan, stamps, ms)), flush=True)


if __name__ == "__main__":
    main()
