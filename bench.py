#!/usr/bin/env python3
"""MoE expert-stack decode benchmark on one MI355X.

Workload (default): the 60-layer, hidden-4096, 512-expert (K=4 + shared),
4-bit stack with every expert blob resident in HBM (about 217 GB), batch 1,
each token's output fed back as the next token's input.  Inputs are seeded
synthetic data (seedgen); weights are random, not trained.

A step is one decode token: one persistent launch running all 60 layers
(routing, expert forward, combine, residual, RMSNorm), replayed as a HIP
graph.

Printed: one JSON line with tokens/s, the roofline of the stack kernel
(HBM bytes per launch / average launch time from HIP events on the launch
stream), the oracle's CPU baseline on a bounded sample, and a parity check of
sampled layers of the first token against the oracle.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
# the sources of the stack kernel; the committed traffic counters apply only
# while these hash the same
KERNEL_SOURCES = ("moe_stack.hip", "moe_device.h", "moe_internal.h")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def algorithmic_bytes(cfg):
    """HBM bytes one layer must read per token: the fp32 router plus the K
    selected blobs and the shared blob."""
    return cfg.E * cfg.D * 4 + (cfg.K + cfg.n_shared) * cfg.blob_bytes


def counted_traffic(cfg):
    """HBM bytes per k_stack launch from the committed counter summary, or
    None when that summary is for other kernel sources or another workload."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"k_stack_{cfg.name}_counters.md")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if ":" in line and not line.startswith(("|", "#", "`")):
            k, _, v = line.partition(":")
            vals[k.strip()] = v.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "expert_weight_streaming_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    if vals.get("kernel_source_sha256_16") != h.hexdigest()[:16]:
        log("counter summary is for other kernel sources: traffic unknown")
        return None
    return int(vals["traffic_bytes_per_launch"])


def build(cfg):
    import torch
    import seedgen
    from expert_weight_streaming_amd.stack import ResidentStack
    free, total = torch.cuda.mem_get_info()
    need = cfg.layers * (cfg.E + cfg.n_shared) * cfg.blob_bytes + cfg.layers * cfg.E * cfg.D * 4
    log(f"HBM free {free / 1e9:.1f} GB of {total / 1e9:.1f} GB; workload needs {need / 1e9:.1f} GB")
    if need > free:
        raise SystemExit(f"workload needs {need / 1e9:.1f} GB of HBM, {free / 1e9:.1f} GB free")
    t0 = time.time()
    st = ResidentStack(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits, layers=cfg.layers,
                       n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps)
    s = torch.cuda.current_stream().cuda_stream
    for l in range(cfg.layers):
        seedgen.dev_blobs(cfg, l, 0, cfg.E, st.expert_ptr(l, 0), s)
        if cfg.n_shared:
            seedgen.dev_blobs(cfg, l, seedgen.SHARED_ID, 1, st.shared_ptr(l), s)
        st.router[l].copy_(torch.from_numpy(seedgen.router(cfg, l)), non_blocking=False)
    torch.cuda.synchronize()
    log(f"built {cfg.layers} layers in {time.time() - t0:.1f} s")
    return st


def kernel_timing(st, r, x, tokens):
    """Average duration of a one-layer launch (moe_layer_step), from HIP
    events recorded around every launch on the launch stream (eager)."""
    import torch
    stream = torch.cuda.current_stream()
    evs = []
    for _ in range(tokens):
        r.copy_(x)
        for l in range(st.layers):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st.layer_step(l, r, x, stream)
            e1.record(stream)
            evs.append((e0, e1))
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in evs]
    return sum(ms) / len(ms), len(ms)


def cpu_baseline(cfg, v0, seconds, check_rows):
    """The oracle (fp64, all host cores) on the first layers of token 0,
    extrapolated to the full stack; also returns its per-layer outputs for
    the parity check."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads as W
    cores = os.cpu_count() or 1
    oracle.set_threads(cores)
    r, x = v0.copy(), v0.copy()
    times, outs = [], []
    t_start = time.time()
    for l in range(cfg.layers):
        ref = W.LayerRef(cfg, l)
        for e in oracle.topk(oracle.router(ref.Wr, x.astype(np.float64)), cfg.K)[0]:
            ref.blob(int(e))  # generate the selected blobs outside the timed call
        t0 = time.time()
        res = ref.run(r, x)
        times.append(time.time() - t0)
        outs.append(res)
        r, x = res["r"].astype(np.float32), res["x"].astype(np.float32)
        if time.time() - t_start > seconds and l + 1 >= check_rows:
            break
    per_layer = sum(times) / len(times)
    all_cores = oracle.get_threads()
    # the same oracle on one core, over the first layers of the same token
    oracle.set_threads(1)
    r, x = v0.copy(), v0.copy()
    t1 = []
    for l in range(min(3, cfg.layers)):
        ref = W.LayerRef(cfg, l)
        for e in oracle.topk(oracle.router(ref.Wr, x.astype(np.float64)), cfg.K)[0]:
            ref.blob(int(e))
        t0 = time.time()
        res = ref.run(r, x)
        t1.append(time.time() - t0)
        r, x = res["r"].astype(np.float32), res["x"].astype(np.float32)
    oracle.set_threads(cores)
    one = sum(t1) / len(t1)
    return {"value": 1.0 / (per_layer * cfg.layers), "unit": "tokens/s", "cores": all_cores,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"token 0, layers 0..{len(times) - 1} of {cfg.layers} (fp64 oracle, blob generation excluded), "
                      f"{per_layer * 1e3:.1f} ms per layer, extrapolated to the full stack",
            "single_core": {"value": 1.0 / (one * cfg.layers), "cores": 1,
                            "sample": f"token 0, layers 0..{len(t1) - 1}, {one * 1e3:.1f} ms per layer, extrapolated"}}, outs


def cpu_model():
    """The host CPU's model name with its family and model numbers (which
    name the generation where the model name is generic) and the count of
    logical CPUs the kernel reports."""
    fields = {}
    n = 0
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k = k.strip()
                if k == "processor":
                    n += 1
                elif k in ("model name", "cpu family", "model") and k not in fields:
                    fields[k] = v.strip()
    except OSError:
        return "unknown"
    name = fields.get("model name", "unknown")
    return f"{name} (family {fields.get('cpu family', '?')}, model {fields.get('model', '?')}, {n} logical CPUs)"


def mem_available():
    try:
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemAvailable:"):
                    return int(line.split()[1]) * 1024
    except OSError:
        pass
    return 0


def streamed_bench(cfg, resident, out0, v0, tokens, warmup, arena_gb):
    """The host-streamed stack: every expert blob in pinned host memory,
    K + shared blobs per layer and token copied into the double-buffered
    slab on a side stream (moe_stream_token).  The host arena is filled from
    the resident stack's HBM arena; the streamed output must equal, bit for
    bit, that of the resident stack holding the same bytes.  This rewrites
    the resident arena when the host arena is aliased: run it last."""
    import torch
    import seedgen
    import expert_weight_streaming_amd as ews
    from expert_weight_streaming_amd.stack import StreamedStack
    bb, L, E = cfg.blob_bytes, cfg.layers, cfg.E
    full = L * E
    # the driver pins at most ~65 GiB in all on the machines measured so far,
    # so the default arena is at most 56 GiB (rounded down to whole layers), aliased
    want = (56 << 30) if arena_gb is None else int(arena_gb * 2**30)
    room = mem_available() - 32 * 2**30
    # whole layers' worth of blobs, so that the zero-copy descriptors (each
    # layer's experts contiguous in the arena) apply too
    P = int(min(full, max(E, min(want, room) // bb))) // E * E
    st = None
    while st is None:
        log(f"streamed: pinning a {P * bb / 2**30:.1f} GiB host arena ({P} of {full} blobs; host MemAvailable "
            f"{mem_available() / 2**30:.1f} GiB)")
        t0 = time.time()
        try:
            st = StreamedStack(hidden=cfg.D, n_experts=E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits, layers=L,
                               n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps, arena_blobs=P)
        except ews.MoeError as err:
            if P <= E:
                raise
            log(f"streamed: {err}; halving the arena")
            P = max(E, P // 2 // E * E)
    log(f"streamed: pinned in {time.time() - t0:.1f} s")
    t0 = time.time()
    chunk = max(1, (2 << 30) // bb)
    for p0 in range(0, P, chunk):
        n = min(chunk, P - p0)
        st.host_arena[p0 * bb:(p0 + n) * bb].copy_(resident.arena[p0 * bb:(p0 + n) * bb])
    if cfg.n_shared:
        st.host_shared.copy_(resident.shared[:st.host_shared.numel()])
    st.router.copy_(resident.router)
    st.gamma.copy_(resident.gamma)
    torch.cuda.synchronize()
    log(f"streamed: arena filled in {time.time() - t0:.1f} s")

    # the link: one large copy, and the streamer's own pattern without compute
    dev = torch.empty(min(P * bb, 4 << 30), dtype=torch.uint8, device="cuda")
    cs = st.copy_stream
    big = []
    for _ in range(3):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(cs):
            dev.copy_(st.host_arena[:dev.numel()], non_blocking=True)
        cs.synchronize()
        big.append(dev.numel() / (time.perf_counter() - t0) / 1e9)
    del dev
    # the streamer's own copy pattern without compute: four passes over all
    # layers (K + shared blobs each), timed by wall clock around each pass
    ids = list(range(cfg.K))
    pats = []
    for rep in range(4):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for l in range(L):
            ews.moe_stream_prefetch(st.streamer, l, [(i * 97 + l * 31 + rep) % E for i in ids], l & 1,
                                    cfg.n_shared > 0, cs)
        cs.synchronize()
        pats.append(L * st.slab_blobs * bb / (time.perf_counter() - t0) / 1e9)
    pattern = max(pats)
    link = max(big)
    log(f"streamed: H2D one large copy {max(big):.1f} GB/s, streamer pattern {pattern:.1f} GB/s")

    # bitwise check of one token against the resident stack holding the same
    # bytes: with an aliased arena, resident blob q becomes a copy of blob
    # q mod P (the first P blobs are the ones the host arena was filled from)
    D = cfg.D
    for q0 in range(P, full, P):
        n = min(P, full - q0)
        resident.arena[q0 * bb:(q0 + n) * bb].copy_(resident.arena[:n * bb])
    r = torch.from_numpy(v0.copy()).cuda().view(1, D)
    want = r.clone()
    resident.step(r, want)
    torch.cuda.synchronize()
    if P == full:
        assert torch.equal(want, out0)
    r = torch.from_numpy(v0.copy()).cuda().view(1, D)
    x = r.clone()
    st.step(r, x)
    torch.cuda.synchronize()
    identical = bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
    if not identical:
        raise SystemExit("streamed output differs from the resident stack holding the same bytes")

    xin = torch.from_numpy(seedgen.activations(cfg, 0, tokens + warmup)).cuda()
    for t in range(warmup):
        r.copy_(xin[t:t + 1])
        x.copy_(xin[t:t + 1])
        st.step(r, x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(tokens):
        r.copy_(xin[warmup + t:warmup + t + 1])
        x.copy_(xin[warmup + t:warmup + t + 1])
        st.step(r, x)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    flags = int(st.workspace[:4].view(torch.int32).item())
    tps = tokens / wall
    per_token = L * st.slab_blobs * bb
    gbs = per_token * tps / 1e9
    log(f"streamed: {tokens} tokens in {wall:.3f} s = {tps:.2f} tok/s, {gbs:.1f} GB/s over the link, flags {flags}")

    # GPU-initiated streaming: the stack kernel reads the selected experts
    # from the pinned arena itself (one launch per token, no copies, no host
    # round trip per layer)
    r.copy_(torch.from_numpy(v0.copy()).cuda().view(1, D))
    x.copy_(r)
    st.step_zero_copy(r, x)
    torch.cuda.synchronize()
    zc_same = bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
    if not zc_same:
        raise SystemExit("zero-copy output differs from the resident stack holding the same bytes")
    for t in range(warmup):
        r.copy_(xin[t:t + 1])
        x.copy_(xin[t:t + 1])
        st.step_zero_copy(r, x)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(tokens):
        r.copy_(xin[warmup + t:warmup + t + 1])
        x.copy_(xin[warmup + t:warmup + t + 1])
        st.step_zero_copy(r, x)
    torch.cuda.synchronize()
    zw = time.perf_counter() - t0
    zflags = int(st.workspace[:4].view(torch.int32).item())
    z_tps = tokens / zw
    log(f"streamed: zero-copy (kernel loads from pinned host memory): {z_tps:.2f} tok/s, "
        f"{per_token * z_tps / 1e9:.1f} GB/s over the link, flags {zflags}")
    # zero-copy with the first half of the layers in HBM (per-layer residency, still one launch per token)
    n_res = L // 2
    zh = st.zero_copy_hybrid_descs(n_res, lambda l: resident.arena.data_ptr() + l * E * bb,
                                   lambda l: resident.shared.data_ptr() + l * bb)
    r.copy_(torch.from_numpy(v0.copy()).cuda().view(1, D))
    x.copy_(r)
    st.step_zero_copy(r, x, descs=zh)
    torch.cuda.synchronize()
    zh_same = bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
    if not zh_same:
        raise SystemExit("zero-copy hybrid output differs from the resident stack")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(tokens):
        r.copy_(xin[warmup + t:warmup + t + 1])
        x.copy_(xin[warmup + t:warmup + t + 1])
        st.step_zero_copy(r, x, descs=zh)
    torch.cuda.synchronize()
    zhw = time.perf_counter() - t0
    zflags |= int(st.workspace[:4].view(torch.int32).item())
    zh_bytes = (L - n_res) * st.slab_blobs * bb
    log(f"streamed: zero-copy with {n_res} of {L} layers in HBM: {tokens / zhw:.2f} tok/s, "
        f"{zh_bytes * tokens / zhw / 1e9:.1f} GB/s over the link")
    zero_copy = {"tokens_per_s": round(z_tps, 3), "ms_per_token": round(zw / tokens * 1e3, 3),
                 "pcie_gbs": round(per_token * z_tps / 1e9, 2), "bitwise_equal_resident": zc_same,
                 "hybrid": {"resident_layers": n_res, "tokens_per_s": round(tokens / zhw, 3),
                            "pcie_bytes_per_token": zh_bytes, "pcie_gbs": round(zh_bytes * tokens / zhw / 1e9, 2),
                            "bitwise_equal_resident": zh_same},
                 "device_flags": zflags}

    # per-expert residency through address tables: the experts routed most
    # often over a few zero-copy warm-up tokens get a copy in an HBM pool
    # (32 GiB), the rest are read from host memory by the kernel; one launch
    # per token, no copies, no host round trip
    free_b, _ = torch.cuda.mem_get_info()
    n_pool = int(min(32 << 30, max(0, free_b - (8 << 30))) // bb) - L * cfg.n_shared
    placed_out = None
    if n_pool >= L * cfg.K:
        counts = {}
        n_warm = 64
        # warm-up inputs disjoint from the timed ones (tokens 100000.. of the seeded sequence)
        xw = torch.from_numpy(seedgen.activations(cfg, 100000, n_warm)).cuda()
        for t in range(n_warm):
            r.copy_(xw[t:t + 1])
            x.copy_(xw[t:t + 1])
            st.step_zero_copy(r, x)
            for l, row in enumerate(st.topk_idx[:, 0].cpu().tolist()):
                for e in row:
                    counts[(l, e)] = counts.get((l, e), 0) + 1
        hot = sorted(counts, key=lambda k: (-counts[k], k))
        placed = st.place_experts(n_pool, hot)
        r.copy_(torch.from_numpy(v0.copy()).cuda().view(1, D))
        x.copy_(r)
        st.step_placed(r, x)
        torch.cuda.synchronize()
        pl_same = bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
        if not pl_same:
            raise SystemExit("address-table output differs from the resident stack")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(tokens):
            r.copy_(xin[warmup + t:warmup + t + 1])
            x.copy_(xin[warmup + t:warmup + t + 1])
            st.step_placed(r, x)
        torch.cuda.synchronize()
        pw = time.perf_counter() - t0
        pflags = int(st.workspace[:4].view(torch.int32).item())
        # the share of the timed tokens' selections that the pool served (same inputs, untimed)
        in_pool = total = 0
        for t in range(tokens):
            r.copy_(xin[warmup + t:warmup + t + 1])
            x.copy_(xin[warmup + t:warmup + t + 1])
            st.step_placed(r, x)
            for l, row in enumerate(st.topk_idx[:, 0].cpu().tolist()):
                in_pool += sum((l, e) in placed for e in row)
                total += len(row)
        frac = in_pool / max(1, total)
        link_bytes = (total - in_pool) / tokens * bb
        log(f"streamed: address tables, {len(placed)} experts + {L * cfg.n_shared} shared in HBM "
            f"({(len(placed) + L * cfg.n_shared) * bb / 2**30:.1f} GiB, ranked over {n_warm} warm-up tokens): "
            f"{tokens / pw:.2f} tok/s, {frac:.1%} of selections from HBM, flags {pflags}")
        placed_out = {"hbm_experts": len(placed), "hbm_shared": L * cfg.n_shared, "warmup_tokens": n_warm,
                      "policy": "most often routed over the warm-up tokens (inputs disjoint from the timed ones), "
                                "fixed while timed",
                      "tokens_per_s": round(tokens / pw, 3), "ms_per_token": round(pw / tokens * 1e3, 3),
                      "selections_from_hbm": round(frac, 4), "pcie_bytes_per_token": int(link_bytes),
                      "bitwise_equal_resident": pl_same, "device_flags": pflags}
        st._pool = st._shared_hbm = st._tables = st._table_descs = None
        torch.cuda.empty_cache()

    # hybrid residency: the first n layers keep their experts in HBM (the
    # resident arena, which now holds the same bytes), the rest stream
    hybrid = []
    for n_res in (L // 2, 3 * L // 4):
        for l in range(L):
            st.set_resident(l, resident.arena.data_ptr() + l * E * bb if l < n_res else None,
                            resident.shared.data_ptr() + l * bb if l < n_res and cfg.n_shared else None)
        r.copy_(torch.from_numpy(v0.copy()).cuda().view(1, D))
        x.copy_(r)
        st.step(r, x)
        torch.cuda.synchronize()
        same = bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
        if not same:
            raise SystemExit(f"hybrid ({n_res} resident layers) output differs from the resident stack")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for t in range(tokens):
            r.copy_(xin[warmup + t:warmup + t + 1])
            x.copy_(xin[warmup + t:warmup + t + 1])
            st.step(r, x)
        torch.cuda.synchronize()
        hw = time.perf_counter() - t0
        hflags = int(st.workspace[:4].view(torch.int32).item())
        h_tps = tokens / hw
        h_bytes = (L - n_res) * st.slab_blobs * bb
        log(f"streamed: hybrid, {n_res} of {L} layers resident: {h_tps:.2f} tok/s, "
            f"{h_bytes * h_tps / 1e9:.1f} GB/s over the link, flags {hflags}")
        hybrid.append({"resident_layers": n_res, "tokens_per_s": round(h_tps, 3),
                       "ms_per_token": round(hw / tokens * 1e3, 3), "pcie_bytes_per_token": h_bytes,
                       "pcie_gbs": round(h_bytes * h_tps / 1e9, 2), "bitwise_equal_resident": same,
                       "device_flags": hflags})
    for l in range(L):
        st.set_resident(l, None)

    # HBM expert cache over the streamed layers (up to 32 GiB of HBM)
    import expert_weight_streaming_amd as ews_
    free_b, _ = torch.cuda.mem_get_info()
    n_slots = int(min(32 << 30, max(0, free_b - (8 << 30))) // bb)
    cache_out = None
    if n_slots >= L * cfg.K:
        c = st.enable_cache(n_slots)
        v0t = torch.from_numpy(v0.copy()).cuda().view(1, D)
        same = True
        for _ in range(2):  # cold, then served from the cache
            r.copy_(v0t)
            x.copy_(v0t)
            st.step(r, x)
            torch.cuda.synchronize()
            same = same and bool(torch.equal(x, want)) and bool(torch.equal(st.topk_idx, resident.topk_idx))
        if not same:
            raise SystemExit("streamed output through the expert cache differs from the resident stack")

        def timed(inputs):
            ews_.moe_expert_cache_reset(c, L, E)
            for t in range(warmup):
                r.copy_(inputs(t))
                x.copy_(r)
                st.step(r, x)
            torch.cuda.synchronize()
            h0, m0, f0 = c.hits, c.misses, c.spec_fills
            t0 = time.perf_counter()
            for t in range(tokens):
                r.copy_(inputs(warmup + t))
                x.copy_(r)
                st.step(r, x)
            torch.cuda.synchronize()
            w_ = time.perf_counter() - t0
            h, m, f = c.hits - h0, c.misses - m0, c.spec_fills - f0
            return {"tokens_per_s": round(tokens / w_, 3), "ms_per_token": round(w_ / tokens * 1e3, 3),
                    "hit_rate": round(h / max(1, h + m), 4), "pcie_bytes_per_token": int((m + f) / tokens * bb),
                    "speculative_fills_per_token": round(f / tokens, 2)}
        fresh = timed(lambda t: xin[t:t + 1])
        repeat = timed(lambda t: v0t)
        # the same fresh inputs with the temporal guess of the next layer's experts
        c.speculate = 1
        spec = timed(lambda t: xin[t:t + 1])
        c.speculate = 0
        cflags = int(st.workspace[:4].view(torch.int32).item())
        # a cache smaller than one token's blobs (half of L * (K + 1)): LRU
        # alone keeps little, the guess fetches the next layer's likely
        # experts while the current layer runs
        small = {}
        st.enable_cache(0)
        c = st.enable_cache(L * (cfg.K + cfg.n_shared) // 2)
        small["slots"] = c.n_slots
        small["fresh_inputs"] = timed(lambda t: xin[t:t + 1])
        c.speculate = 1
        small["fresh_inputs_speculative"] = timed(lambda t: xin[t:t + 1])
        cflags |= int(st.workspace[:4].view(torch.int32).item())
        log(f"streamed: expert cache of {c.n_slots} blobs: fresh inputs {small['fresh_inputs']['tokens_per_s']:.2f} "
            f"tok/s at {small['fresh_inputs']['hit_rate']:.1%} hits; with the next-layer guess "
            f"{small['fresh_inputs_speculative']['tokens_per_s']:.2f} tok/s at "
            f"{small['fresh_inputs_speculative']['hit_rate']:.1%} hits, "
            f"{small['fresh_inputs_speculative']['speculative_fills_per_token']:.1f} guessed blobs per token")
        log(f"streamed: expert cache of {n_slots} blobs ({n_slots * bb / 2**30:.1f} GiB HBM): fresh inputs "
            f"{fresh['tokens_per_s']:.2f} tok/s at {fresh['hit_rate']:.1%} hits; one input repeated "
            f"{repeat['tokens_per_s']:.2f} tok/s at {repeat['hit_rate']:.1%} hits; fresh inputs with the "
            f"next-layer guess {spec['tokens_per_s']:.2f} tok/s at {spec['hit_rate']:.1%} hits, "
            f"{spec['speculative_fills_per_token']:.1f} guessed blobs per token, flags {cflags}")
        cache_out = {"slots": n_slots, "hbm_bytes": n_slots * bb, "policy": "LRU over (layer, expert)",
                     "fresh_inputs": fresh, "repeated_input": repeat, "fresh_inputs_speculative": spec,
                     "small_cache": small, "bitwise_equal_resident": same,
                     "device_flags": cflags}
        st.enable_cache(0)
    return {"workload": f"{L}-layer {cfg.bits}-bit stack, experts in pinned host RAM, K={cfg.K} + {cfg.n_shared} "
                        f"shared blobs per layer copied host->HBM per token, fresh N(0,1) input per token",
            "tokens": tokens, "tokens_per_s": round(tps, 3), "ms_per_token": round(wall / tokens * 1e3, 3),
            "pcie_bytes_per_token": per_token, "pcie_gbs": round(gbs, 2),
            "pcie_peak_measured_gbs": round(link, 2), "pcie_peak_source": "one 4 GiB pinned hipMemcpyAsync, best of 3",
            "pcie_frac_measured": round(gbs / link, 4),
            "h2d_copy_pattern_no_compute_gbs": round(pattern, 2),
            "arena_blobs": P, "arena_aliased": P != full, "bitwise_equal_resident": identical,
            "device_flags": flags, "zero_copy": zero_copy, "address_tables": placed_out, "hybrid": hybrid,
            "expert_cache": cache_out}


def gemv_bench(st, cfg, calls=20, warmup=10):
    """moe_expert_gemv over all E experts of one layer per call: one launch,
    each workgroup streaming whole experts (gate/up, SwiGLU, then down from h
    kept on chip), so every byte of the layer's E blobs (3.6 GB at 4-bit) is
    read once per call; the calls cycle through the stack's layers, far more
    bytes than the 256 MB last-level cache holds.  Timed with HIP events on
    the launch stream; three experts of the last call checked against the
    oracle."""
    import numpy as np
    import torch
    import oracle
    import seedgen
    import expert_weight_streaming_amd as ews
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads as W
    E, D, I, L = cfg.E, cfg.D, cfg.I, st.layers
    x = torch.from_numpy(seedgen.activation(cfg, 7)).cuda()
    h = torch.empty(E, I, dtype=torch.float32, device="cuda")
    y = torch.empty(E, D, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    for c in range(warmup):
        ews.moe_expert_gemv(st.descs[c % L], x, 0, E, h, y, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for c in range(calls):
        ews.moe_expert_gemv(st.descs[(warmup + c) % L], x, 0, E, h, y, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    blob_bytes = E * cfg.blob_bytes
    alg = blob_bytes + D * 4 + E * (I + D) * 4  # the blobs, x, and h and y written
    gbs = alg / (us * 1e-6) / 1e9
    last = (warmup + calls - 1) % L
    xv = seedgen.activation(cfg, 7).astype(np.float64)
    hn, yn = h.cpu().numpy(), y.cpu().numpy()
    worst = 0.0
    for e in (0, E // 2, E - 1):
        oh, oy = oracle.expert(seedgen.blob(cfg, last, e), D, I, cfg.bits, cfg.group, xv)
        worst = max(worst, W.assert_close(hn[e], oh, f"gemv h {e}"), W.assert_close(yn[e], oy, f"gemv y {e}"))
    log(f"gemv {cfg.bits}-bit: {E} experts per launch, {us:.1f} us, {gbs:.0f} GB/s = {gbs / HBM_PEAK_GBS:.1%} of HBM peak")
    return {"workload": f"moe_expert_gemv: all {E} experts of a hidden-{D}, inter-{I}, {cfg.bits}-bit layer per launch "
                        f"(gate/up + SwiGLU + down, one vector), layers cycled", "bits": cfg.bits,
            "launches_timed": calls, "avg_launch_us": round(us, 2), "bytes_per_launch": alg,
            "blob_bytes_per_launch": blob_bytes, "achieved_gbs": round(gbs, 1), "peak_gbs": HBM_PEAK_GBS,
            "frac": round(gbs / HBM_PEAK_GBS, 4), "experts_checked_vs_oracle": 3, "worst_rel_l2": worst}


def sampled_parity(cfg, rec, sel, w, tokens=(0, 1, 63, 127), n_random=64, seed=12345):
    """Every layer of the listed tokens plus n_random random (token, layer)
    pairs of the recorded decode, each layer against the oracle on the
    (resid, x) the GPU recorded entering it.  rec [T][L+1][2][1][D], sel/w
    [T][L][1][K] (numpy)."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import workloads as W
    T, L = rec.shape[0], cfg.layers
    pairs = {(t, l) for t in tokens if t < T for l in range(L)}
    rng = np.random.default_rng(seed)
    while len(pairs) < len({(t, l) for t in tokens if t < T for l in range(L)}) + n_random:
        pairs.add((int(rng.integers(0, T)), int(rng.integers(0, L))))
    oracle.set_threads(os.cpu_count() or 1)
    worst, near = 0.0, 0
    t0 = time.time()
    for l in range(L):
        ts = sorted(t for (t, ll) in pairs if ll == l)
        if not ts:
            continue
        ref = W.LayerRef(cfg, l)
        for t in ts:
            st = {}
            res = W.check_layer(ref, rec[t, l, 0, 0], rec[t, l, 1, 0], sel[t, l, 0], w[t, l, 0], rec[t, l + 1, 0, 0],
                                rec[t, l + 1, 1, 0], st)
            near += st.get("near_ties", 0)
            worst = max(worst, W.rel_l2(rec[t, l + 1, 0, 0], res["r"]), W.rel_l2(rec[t, l + 1, 1, 0], res["x"]))
    log(f"parity: {len(pairs)} (token, layer) pairs against the oracle in {time.time() - t0:.1f} s, worst rel-L2 "
        f"{worst:.2e}, near ties {near}")
    return {"pairs_vs_oracle": len(pairs), "tokens_all_layers": [t for t in tokens if t < T],
            "random_pairs": n_random, "worst_rel_l2": worst, "near_ties": near,
            "rule": "per layer on the GPU-recorded (resid, x) input: top-K set equal (or oracle gap < 1e-5), "
                    "rel-L2 <= 1e-4 and max-abs <= 1e-3 max|ref| on resid and x"}


def ne_histogram(sel, E):
    """Tokens per active expert, per layer, as a histogram (mean count of
    experts per bin and layer)."""
    import numpy as np
    bins = [(1, 1), (2, 2), (3, 3), (4, 7), (8, 15), (16, 10 ** 9)]
    out = {f"{a}" if a == b else (f"{a}+" if b > 10 ** 8 else f"{a}-{b}"): 0.0 for a, b in bins}
    for l in range(sel.shape[0]):
        c = np.bincount(sel[l].reshape(-1), minlength=E)
        for (a, b), k in zip(bins, out):
            out[k] += float(((c >= a) & (c <= b)).sum())
    return {k: round(v / sel.shape[0], 2) for k, v in out.items()}


def resident_extra(cfg, steps, warmup):
    """Another resident workload of the same family, timed like the headline
    (graph replays, output fed back): the 2-bit stack at batch 1, or at a
    batch of cfg.tokens tokens through the grouped path.  Reported next to
    the headline, not instead of it."""
    import numpy as np
    import torch
    import seedgen
    from expert_weight_streaming_amd.stack import ResidentStack
    T = cfg.tokens
    st = ResidentStack(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits, layers=cfg.layers,
                       n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps, n_tokens=T)
    s = torch.cuda.current_stream().cuda_stream
    for l in range(cfg.layers):
        seedgen.dev_blobs(cfg, l, 0, cfg.E, st.expert_ptr(l, 0), s)
        if cfg.n_shared:
            seedgen.dev_blobs(cfg, l, seedgen.SHARED_ID, 1, st.shared_ptr(l), s)
        st.router[l].copy_(torch.from_numpy(seedgen.router(cfg, l)))
    torch.cuda.synchronize()
    x = torch.from_numpy(seedgen.activations(cfg, 0, T)).cuda()
    x_in = x.clone()
    r = x.clone()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cs):
        with torch.cuda.graph(graph, stream=cs):
            r.copy_(x)
            st.step(r, x, stream=cs)
    torch.cuda.current_stream().wait_stream(cs)
    def timed(inputs):
        """Time `steps` graph replays of the step with x first set to
        `inputs` (then fed back); bytes per step from the selections of a
        replay of the same first step."""
        x.copy_(inputs)
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        flags = int(st.workspace[:4].view(torch.int32).item())
        sel = st.topk_idx.cpu().numpy()  # [L][T][K] of the last step
        distinct = [len(np.unique(sel[l])) for l in range(cfg.layers)]
        step_bytes = sum(cfg.E * cfg.D * 4 + (d + cfg.n_shared) * cfg.blob_bytes for d in distinct)
        gbs = step_bytes / (ms * 1e-3) / 1e9
        o = {"ms_per_step": round(ms, 4), "tokens_per_s": round(T * 1e3 / ms, 2), "hbm_bytes_per_step": step_bytes,
             "hbm_gbs": round(gbs, 1), "frac_of_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "device_flags": flags}
        if T > 1:
            o["distinct_experts_per_layer"] = round(float(np.mean(distinct)), 2)
            o["tokens_per_active_expert_histogram"] = ne_histogram(sel, cfg.E)
        return o

    out = {"workload": f"{cfg.layers}-layer {cfg.bits}-bit stack resident in HBM, batch {T}, output fed back",
           "tokens_per_step": T, "steps": steps}
    out.update(timed(x_in))
    log(f"{cfg.name}: {out['tokens_per_s']} tok/s, {out['ms_per_step']:.3f} ms per step, {out['hbm_gbs']:.0f} GB/s, "
        f"flags {out['device_flags']}")
    if T > 1:
        # a skewed input set: every token near one shared base, so experts
        # receive many tokens each
        base = seedgen.activation(cfg, 5000)
        skew = (base[None, :] + 0.1 * seedgen.activations(cfg, 5001, T)).astype(np.float32)
        out["skewed"] = timed(torch.from_numpy(skew).cuda())
        out["skewed"]["inputs"] = "tokens = one N(0,1) base + 0.1 N(0,1) noise each"
        log(f"{cfg.name} skewed: {out['skewed']['tokens_per_s']} tok/s, {out['skewed']['hbm_gbs']:.0f} GB/s, "
            f"{out['skewed']['distinct_experts_per_layer']} distinct experts per layer")
    else:
        out["gemv"] = gemv_bench(st, cfg)
    del st, graph
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=128, help="timed decode tokens")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--config", default="stack4")
    ap.add_argument("--kernel-tokens", type=int, default=4,
                    help="tokens of the one-layer-per-launch event timing pass (0: skip)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle baseline and parity check")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-stream", action="store_true", help="skip the host-streamed stack")
    ap.add_argument("--no-extra", action="store_true", help="skip the 2-bit stacks (batch 1 and batch 32)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run one plain elementwise copy of 1 GiB (reads 1 GiB, writes 1 GiB), the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--stream-tokens", type=int, default=64)
    ap.add_argument("--stream-arena-gb", type=float, default=None,
                    help="host arena size (default: the whole stack when host RAM allows, else aliased)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (see DESIGN.md on sharding)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import seedgen

    cfg = seedgen.CONFIGS[args.config]
    if args.copy_probe:
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.neg(a, out=b)
        torch.cuda.synchronize()
        del a, b
    st = build(cfg)
    D = cfg.D
    v0 = seedgen.activation(cfg, 0)
    r = torch.zeros(1, D, dtype=torch.float32, device="cuda")
    x = torch.from_numpy(v0.copy()).cuda().view(1, D)

    # token 0 eagerly, recording every layer's output for the parity check
    rec = torch.zeros(cfg.layers + 1, 2, 1, D, dtype=torch.float32, device="cuda")
    r.copy_(x)
    st.step(r, x, record=rec)
    torch.cuda.synchronize()
    out0 = x.clone()

    # the per-token graph: r <- x (the fed-back input), then all layers
    x.copy_(torch.from_numpy(v0).view(1, D))
    graph = None
    if not args.no_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                r.copy_(x)
                st.step(r, x, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        x.copy_(torch.from_numpy(v0).view(1, D))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(x, out0), "graph replay differs from eager execution"

    def token():
        if graph is not None:
            graph.replay()
        else:
            r.copy_(x)
            st.step(r, x)

    for _ in range(args.warmup):
        token()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        token()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dev_ms = e0.elapsed_time(e1)
    ms_per_step = max(wall * 1e3, dev_ms) / args.steps
    value = 1e3 / ms_per_step
    flags = int(st.workspace[:4].view(torch.int32).item())
    log(f"{args.steps} tokens: wall {wall * 1e3:.2f} ms, events {dev_ms:.2f} ms, flags {flags}")

    # the stack kernel's average duration: HIP events around the timed region
    # on the launch stream, over its `steps` launches (one per token, all
    # layers; the 16 KB r <- x copy node of each replay is included)
    k_ms = dev_ms / args.steps
    n_launch = args.steps
    k_ms_layer, n_eager = kernel_timing(st, r, x, args.kernel_tokens) if args.kernel_tokens > 0 else (float("nan"), 0)
    bytes_per_launch = algorithmic_bytes(cfg) * cfg.layers
    achieved = bytes_per_launch / (k_ms * 1e-3) / 1e9
    log(f"stack kernel: {k_ms * 1e3:.2f} us per token launch ({k_ms * 1e3 / cfg.layers:.2f} us per layer, "
        f"{achieved:.0f} GB/s); one layer per launch: {k_ms_layer * 1e3:.2f} us between events over {n_eager} "
        f"eager launches")
    traffic = counted_traffic(cfg)
    out = {
        "metric": "MoE expert-stack tokens/s (batch 1, 4-bit); dequant-GEMV HBM GB/s vs peak",
        "value": round(value, 2), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"u{cfg.bits} codes x 23-bit fixed-point activations (one step per 16-byte code chunk, "
                 f"exact i32 digit-plane dot products), bf16 scale/bias, f32 elsewhere",
        "data": "synthetic (seeded, random weights)",
        "config": {"workload": f"{cfg.layers}-layer MoE expert stack, hidden {cfg.D}, {cfg.E} experts, top-{cfg.K} "
                               f"+ {cfg.n_shared} shared, inter {cfg.I}, {cfg.bits}-bit group-{cfg.group} "
                               f"experts resident in HBM, batch {cfg.tokens}, output fed back",
                   "global_batch": cfg.tokens, "layers": cfg.layers, "graph": graph is not None,
                   "expert_bytes_resident": cfg.layers * (cfg.E + cfg.n_shared) * cfg.blob_bytes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                     "kernel": f"k_stack (persistent, {cfg.layers} layers per launch)",
                     "bytes_per_launch": bytes_per_launch, "avg_launch_us": round(k_ms * 1e3, 3),
                     "launches_timed": n_launch, "us_per_layer": round(k_ms * 1e3 / cfg.layers, 3),
                     "one_layer_launch_us_eager_events": round(k_ms_layer * 1e3, 3) if n_eager else None},
        "stack_gbs": round(bytes_per_launch / (ms_per_step * 1e-3) / 1e9, 1),
        "device_flags": flags,
    }
    # the dequant GEMV kernel alone at a large shape (all experts of a layer per launch)
    out["gemv"] = {"bits4": gemv_bench(st, cfg)}
    # the decode sequence again, eagerly, recording every layer's input and
    # output of every token for the oracle's sampled check (before the
    # streamed leg, which may rewrite the resident arena)
    n_rec = min(args.steps, 128)
    rec_all = torch.zeros(n_rec, cfg.layers + 1, 2, 1, D, dtype=torch.float32, device="cuda")
    sel_all = torch.zeros(n_rec, cfg.layers, 1, cfg.K, dtype=torch.int32, device="cuda")
    w_all = torch.zeros(n_rec, cfg.layers, 1, cfg.K, dtype=torch.float32, device="cuda")
    x.copy_(torch.from_numpy(v0).view(1, D))
    for t in range(n_rec):
        r.copy_(x)
        st.step(r, x, record=rec_all[t])
        sel_all[t].copy_(st.topk_idx)
        w_all[t].copy_(st.topk_w)
    torch.cuda.synchronize()
    assert torch.equal(rec_all[0], rec), "recorded token 0 differs from the first eager run"
    rec_np, sel_np, w_np = rec_all.cpu().numpy(), sel_all.cpu().numpy(), w_all.cpu().numpy()
    del rec_all, sel_all, w_all
    if not args.no_stream:
        out["streamed"] = streamed_bench(cfg, st, out0, v0, args.stream_tokens, 2, args.stream_arena_gb)
    if not args.no_extra:
        # free the 4-bit stack (and the graph holding its buffers) first
        del st, graph
        torch.cuda.empty_cache()
        out["stack2"] = resident_extra(seedgen.CONFIGS["stack2"], 128, 8)
        out["gemv"]["bits2"] = out["stack2"].pop("gemv")
        out["stack2_b32"] = resident_extra(seedgen.CONFIGS["stack2_b32"], 8, 2)
    if not args.no_cpu:
        sys.path.insert(0, os.path.join(ROOT, "tests"))
        import workloads as W
        base, outs = cpu_baseline(cfg, v0, args.cpu_seconds, check_rows=2)
        out["cpu_baseline"] = base
        # parity: every layer of tokens 0, 1, 63, 127 and 64 random (token,
        # layer) pairs, each on the GPU-recorded input of that layer
        out["check"] = sampled_parity(cfg, rec_np, sel_np, w_np)
        # and the oracle's own chain over token 0 (as far as no near tie
        # lets the two chains part)
        checked, worst = 0, 0.0
        for l, res in enumerate(outs):
            gsel = sorted(int(e) for e in sel_np[0, l, 0])
            if gsel != sorted(int(e) for e in res["sel"]):
                if res["gap"] >= W.NEAR_TIE:
                    raise SystemExit(f"layer {l}: top-K differs from the oracle")
                break
            e1_ = W.assert_close(rec_np[0, l + 1, 0, 0], res["r"], f"layer {l} residual")
            e2_ = W.assert_close(rec_np[0, l + 1, 1, 0], res["x"], f"layer {l} output")
            worst = max(worst, e1_, e2_)
            checked += 1
        out["check"]["token0_oracle_chain"] = {"layers": checked, "worst_rel_l2": worst}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
