"""GPU tests of the host-streamed path: the slab receives exactly the host
bytes of the selected experts, and a streamed stack gives bit-identical
outputs and selections to a resident stack holding the same bytes (same
kernels, same inputs), including an aliased host arena, a stack without
a shared expert, and stacks where some layers stay resident (hybrid
residency).  Every mode's recorded layers are also checked against the
oracle, each on the (resid, x) the GPU recorded entering it, with a
distinct non-unit RMSNorm weight per layer and a non-default epsilon."""
import numpy as np
import pytest

import seedgen
import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def test_prefetch_copies_selected_blobs():
    import expert_weight_streaming_amd as ews
    cfg = seedgen.CONFIGS["tiny"].replace(layers=3, seed=0x5EED0E01)
    print("[gpu case] prefetch bytes", flush=True)
    st = W.build_streamed(cfg, layers=3, arena_blobs=37)
    cs = st.copy_stream
    ids = [5, 0, 15][:cfg.K]
    ev = torch.cuda.Event()
    ev.record(cs)  # creates the HIP event
    for l, slot in ((0, 0), (2, 1), (1, 0)):
        st.slab.fill_(0xAB)
        cs.wait_stream(torch.cuda.current_stream())  # the fill before the copies
        ews.moe_stream_prefetch(st.streamer, l, ids, slot, True, cs, ev)
        ev.synchronize()
        got = st.slab[slot].cpu()
        for j, e in enumerate(ids):
            assert torch.equal(got[j * st.bb:(j + 1) * st.bb], st.host_blob(l, e)), (l, j, e)
        assert torch.equal(got[(st.slab_blobs - 1) * st.bb:], st.host_shared_blob(l)), l
        # the other slot is untouched
        assert bool((st.slab[1 - slot].cpu() == 0xAB).all())
    with pytest.raises(ValueError):
        ews.moe_stream_prefetch(st.streamer, 0, [0], 0, False, cs, torch.cuda.Event())  # never recorded
    with pytest.raises(ews.MoeError):
        ews.moe_stream_prefetch(st.streamer, 0, [cfg.E], 0, False, cs)
    with pytest.raises(ews.MoeError):
        ews.moe_stream_prefetch(st.streamer, 3, [0], 0, False, cs)


def _g(cfg):
    """The config with a distinct non-unit RMSNorm weight per layer and a
    non-default epsilon."""
    return cfg.replace(gamma_sigma=0.25, eps=3e-4)


def _refs(cfg, st):
    return [W.LayerRef(cfg, l, arena_blobs=st.P) for l in range(st.layers)]


def _rec(st):
    return torch.zeros(st.layers + 1, 2, 1, st.D, dtype=torch.float32, device="cuda")


def _check(refs, st, rec, stats):
    W.check_record(refs, rec.cpu().numpy(), st.topk_idx.cpu().numpy(), st.topk_w.cpu().numpy(), stats)


def run_pair(cfg, layers, tokens, arena_blobs=None):
    st = W.build_streamed(cfg, layers=layers, arena_blobs=arena_blobs)
    rs = W.resident_twin(st)
    refs = _refs(cfg, st)
    rec_s, rec_r = _rec(st), _rec(st)
    stats = {}
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    xs, xr = v.clone(), v.clone()
    for t in range(tokens):
        r_s, r_r = xs.clone(), xr.clone()
        st.step(r_s, xs, record=rec_s)
        rs.step(r_r, xr, record=rec_r)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0, "device error flags (streamed)"
        assert torch.equal(st.topk_idx, rs.topk_idx), t
        assert torch.equal(st.topk_w, rs.topk_w), t
        assert torch.equal(r_s, r_r) and torch.equal(xs, xr), t
        assert torch.equal(rec_s, rec_r), t
        assert bool(torch.isfinite(xs).all())
        _check(refs, st, rec_s, stats)
    assert stats["layers"] == layers * tokens
    return st, rs


@pytest.mark.parametrize("name,bits", [("tiny", 4), ("tiny", 2)])
def test_streamed_equals_resident_tiny(name, bits):
    cfg = _g(seedgen.CONFIGS[name].replace(bits=bits, layers=6, seed=0x5EED0E10 + bits))
    print(f"[gpu case] streamed tiny bits={bits}", flush=True)
    run_pair(cfg, 6, 4)


def test_streamed_equals_resident_hidden4096():
    cfg = _g(seedgen.CONFIGS["layer"].replace(E=24, layers=5, seed=0x5EED0E20))
    print("[gpu case] streamed hidden-4096", flush=True)
    st, _ = run_pair(cfg, 5, 3)
    # the selections really vary across layers, so the slots are exercised
    sel = st.topk_idx.cpu().numpy()
    assert len({tuple(sorted(s[0])) for s in sel}) > 1


def test_streamed_aliased_arena():
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=5, seed=0x5EED0E30))
    print("[gpu case] streamed aliased arena", flush=True)
    run_pair(cfg, 5, 3, arena_blobs=23)


def test_streamed_no_shared():
    cfg = _g(seedgen.CONFIGS["tiny"].replace(n_shared=0, layers=4, seed=0x5EED0E40))
    print("[gpu case] streamed without shared expert", flush=True)
    run_pair(cfg, 4, 3)


def test_streamed_matches_oracle_first_layer():
    """Layer 0 of the streamed stack against the oracle (the later layers
    are covered by bitwise equality with the resident stack, whose
    per-layer outputs the resident stack tests check)."""
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=1, seed=0x5EED0E50))
    print("[gpu case] streamed layer 0 vs oracle", flush=True)
    st = W.build_streamed(cfg, layers=1)
    x0 = seedgen.activation(cfg, 0)
    r, x = torch.from_numpy(x0).cuda().view(1, -1), torch.from_numpy(x0).cuda().view(1, -1)
    st.step(r, x)
    torch.cuda.synchronize()
    ref = W.LayerRef(cfg, 0)
    W.check_layer(ref, x0, x0, st.topk_idx[0, 0].cpu().numpy(), st.topk_w[0, 0].cpu().numpy(),
                  r[0].cpu().numpy(), x[0].cpu().numpy(), {})


@pytest.mark.parametrize("pattern", ["RSRRSS", "SRRSRS", "RRRRRR", "SSSSSR"])
def test_hybrid_residency_equals_resident(pattern):
    """Per-layer hybrid residency: layers marked R keep their experts in HBM
    (pointing into the resident twin's arena, the same bytes), the others
    stream.  Output, selections and weights equal the resident stack's bit
    for bit, whichever layers stream (first streamed layer after resident
    ones, resident runs in the middle and at the end, none streamed)."""
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=len(pattern), seed=0x5EED0E60))
    print(f"[gpu case] hybrid residency {pattern}", flush=True)
    st = W.build_streamed(cfg, layers=len(pattern), arena_blobs=29)
    rs = W.resident_twin(st)
    refs, rec, stats = _refs(cfg, st), _rec(st), {}
    for l, c in enumerate(pattern):
        if c == "R":
            st.set_resident(l, rs.arena.data_ptr() + l * st.E * st.bb, rs.shared.data_ptr() + l * st.bb)
    assert st.resident_layers() == [l for l, c in enumerate(pattern) if c == "R"]
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    xs, xr = v.clone(), v.clone()
    for t in range(3):
        r_s, r_r = xs.clone(), xr.clone()
        st.step(r_s, xs, record=rec)
        rs.step(r_r, xr)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        assert torch.equal(st.topk_idx, rs.topk_idx), t
        assert torch.equal(st.topk_w, rs.topk_w), t
        assert torch.equal(r_s, r_r) and torch.equal(xs, xr), t
        _check(refs, st, rec, stats)
    assert stats["layers"] == 3 * len(pattern)
    # and back to fully streamed
    for l in range(len(pattern)):
        st.set_resident(l, None)
    assert st.resident_layers() == []
    r_s, r_r = xs.clone(), xr.clone()
    st.step(r_s, xs)
    rs.step(r_r, xr)
    torch.cuda.synchronize()
    assert torch.equal(xs, xr)


def _lru(events, n_slots):
    """Hits, misses and speculative fills of an LRU cache of n_slots over a
    sequence of ("get", key) requests and ("fill", key) guesses (a guess
    fills an uncached key and leaves a cached one alone)."""
    from collections import OrderedDict
    od, hits, misses, fills = OrderedDict(), 0, 0, 0
    for kind, k in events:
        if k in od:
            if kind == "get":
                hits += 1
                od.move_to_end(k)
            continue
        if kind == "get":
            misses += 1
        else:
            fills += 1
        if len(od) >= n_slots:
            od.popitem(last=False)
        od[k] = True
    return hits, misses, fills


@pytest.mark.parametrize("n_slots,pattern,speculate,bits", [(5, "SSSS", False, 4), (64, "SSSS", False, 4),
                                                            (3, "SRSS", False, 4), (6, "SSSS", True, 4),
                                                            (64, "SRSS", True, 4), (9, "SSSS", True, 2)])
def test_expert_cache_equals_resident(n_slots, pattern, speculate, bits):
    """The HBM expert cache: outputs equal the resident stack's bit for bit
    (cached blobs come from HBM, missed ones over the link), and the hit and
    miss counts equal an LRU of n_slots over the streamed blobs in the order
    the token pipeline requests them: a streamed layer's selections (the
    first streamed layer's shared blob right after them), then the next
    streamed layer's shared blob, then (speculate) the previous token's
    selection of that layer as guesses.  Tokens repeat, so a cache that
    holds every blob serves the repeats entirely from HBM."""
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=len(pattern), bits=bits, seed=0x5EED0E70 + bits))
    print(f"[gpu case] expert cache slots={n_slots} {pattern} speculate={speculate} bits={bits}", flush=True)
    st = W.build_streamed(cfg, layers=len(pattern), arena_blobs=31)
    rs = W.resident_twin(st)
    refs, rec, stats = _refs(cfg, st), _rec(st), {}
    for l, c in enumerate(pattern):
        if c == "R":
            st.set_resident(l, rs.arena.data_ptr() + l * st.E * st.bb, rs.shared.data_ptr() + l * st.bb)
    cache = st.enable_cache(n_slots, speculate=speculate)
    events, pred = [], {}
    inputs = [seedgen.activation(cfg, t) for t in (0, 1, 0, 0, 1)]
    for t, v0 in enumerate(inputs):
        v = torch.from_numpy(v0).cuda().view(1, -1)
        r_s, x_s, r_r, x_r = v.clone(), v.clone(), v.clone(), v.clone()
        st.step(r_s, x_s, record=rec)
        rs.step(r_r, x_r)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        assert torch.equal(st.topk_idx, rs.topk_idx), t
        assert torch.equal(r_s, r_r) and torch.equal(x_s, x_r), t
        _check(refs, st, rec, stats)
        sel = st.topk_idx.cpu().numpy()
        streamed = [l for l, c in enumerate(pattern) if c == "S"]
        LE = len(pattern) * cfg.E
        for j, l in enumerate(streamed):
            events += [("get", l * cfg.E + int(e)) for e in sel[l, 0]]
            if j == 0:
                events.append(("get", LE + l))                  # its own shared blob
            pred[l] = [int(e) for e in sel[l, 0]]
            if j + 1 < len(streamed):
                ln = streamed[j + 1]
                events.append(("get", LE + ln))                 # the next streamed layer's shared blob
                if speculate and ln in pred:
                    events += [("fill", ln * cfg.E + e) for e in pred[ln]]
    assert (cache.hits, cache.misses, cache.spec_fills) == _lru(events, n_slots)
    keys = {k for kind, k in events if kind == "get"}
    if n_slots >= len(keys):
        assert cache.misses == len(keys)  # every repeat served from HBM
    st.enable_cache(0)
    assert st.streamer.cache is None or not st.streamer.cache


@pytest.mark.parametrize("arena_blobs,bits", [(None, 4), (32, 4), (32, 2)])
def test_zero_copy_equals_resident(arena_blobs, bits):
    """GPU-initiated streaming: the stack kernel reads the selected experts
    straight from the pinned host arena (one launch per token, no copies, no
    host wait).  Outputs and selections equal the resident stack's holding
    the same bytes, bit for bit, with a full and an aliased arena (32 blobs =
    two layers' experts)."""
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=5, bits=bits, seed=0x5EED0E80 + bits))
    print(f"[gpu case] zero-copy arena_blobs={arena_blobs} bits={bits}", flush=True)
    st = W.build_streamed(cfg, layers=5, arena_blobs=arena_blobs)
    rs = W.resident_twin(st)
    refs, rec, stats = _refs(cfg, st), _rec(st), {}
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    xz, xr = v.clone(), v.clone()
    for t in range(3):
        r_z, r_r = xz.clone(), xr.clone()
        st.step_zero_copy(r_z, xz, record=rec)
        rs.step(r_r, xr)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        assert torch.equal(st.topk_idx, rs.topk_idx), t
        assert torch.equal(st.topk_w, rs.topk_w), t
        assert torch.equal(r_z, r_r) and torch.equal(xz, xr), t
        _check(refs, st, rec, stats)
    # layers 0 and 1 from HBM (the twin's arena), the rest from host memory, one launch
    zh = st.zero_copy_hybrid_descs(2, lambda l: rs.arena.data_ptr() + l * st.E * st.bb,
                                   lambda l: rs.shared.data_ptr() + l * st.bb)
    r_z, r_r = xz.clone(), xr.clone()
    st.step_zero_copy(r_z, xz, descs=zh)
    rs.step(r_r, xr)
    torch.cuda.synchronize()
    assert torch.equal(st.topk_idx, rs.topk_idx)
    assert torch.equal(r_z, r_r) and torch.equal(xz, xr)


def test_zero_copy_needs_whole_layers():
    cfg = seedgen.CONFIGS["tiny"].replace(layers=3, seed=0x5EED0E81)
    st = W.build_streamed(cfg, layers=3, arena_blobs=cfg.E + 3)
    with pytest.raises(ValueError):
        st.zero_copy_descs()


@pytest.mark.parametrize("arena_blobs,n_slots,bits", [(None, 40, 4), (32, 7, 4), (None, 20, 2)])
def test_address_tables_equal_resident(arena_blobs, n_slots, bits):
    """Per-expert residency: each layer's descriptor carries a device table of
    blob addresses, the placed experts in an HBM pool, the others in the
    pinned host arena, read by the stack kernel itself (one launch per
    token).  Outputs equal the resident stack's bit for bit; one layer
    through moe_layer_step in the same mode does too."""
    import expert_weight_streaming_amd as ews
    cfg = _g(seedgen.CONFIGS["tiny"].replace(layers=4, bits=bits, seed=0x5EED0E90 + bits))
    print(f"[gpu case] address tables arena={arena_blobs} slots={n_slots} bits={bits}", flush=True)
    st = W.build_streamed(cfg, layers=4, arena_blobs=arena_blobs)
    rs = W.resident_twin(st)
    refs, rec, stats = _refs(cfg, st), _rec(st), {}
    hot = [(l, e) for l in range(4) for e in range(cfg.E) if (l + e) % 3 == 0]
    placed = st.place_experts(n_slots, hot)
    assert len(placed) == min(n_slots, len(hot))
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    xp, xr = v.clone(), v.clone()
    for t in range(3):
        r_p, r_r = xp.clone(), xr.clone()
        st.step_placed(r_p, xp, record=rec)
        rs.step(r_r, xr)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        assert torch.equal(st.topk_idx, rs.topk_idx), t
        assert torch.equal(r_p, r_r) and torch.equal(xp, xr), t
        _check(refs, st, rec, stats)
    r_p, r_r, x_p, x_r = v.clone(), v.clone(), v.clone(), v.clone()
    ews.moe_layer_step(st._table_descs[0], r_p, x_p, 1, st.topk_idx[0], st.topk_w[0], st.workspace)
    rs.layer_step(0, r_r, x_r)
    torch.cuda.synchronize()
    assert torch.equal(r_p, r_r) and torch.equal(x_p, x_r)


def test_zero_copy_and_tables_hidden4096():
    """The hidden-4096 shape (the 60-layer stack's kernel instantiation):
    zero-copy and address-table tokens equal the resident stack bit for
    bit."""
    cfg = _g(seedgen.CONFIGS["layer"].replace(E=24, layers=3, seed=0x5EED0EA0))
    print("[gpu case] zero-copy and tables hidden-4096", flush=True)
    st = W.build_streamed(cfg, layers=3)
    rs = W.resident_twin(st)
    refs, rec, stats = _refs(cfg, st), _rec(st), {}
    st.place_experts(20, [(l, e) for l in range(3) for e in range(0, cfg.E, 3)])
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    for step in (st.step_zero_copy, st.step_placed):
        xs, xr = v.clone(), v.clone()
        for t in range(2):
            r_s, r_r = xs.clone(), xr.clone()
            step(r_s, xs, record=rec)
            rs.step(r_r, xr)
            torch.cuda.synchronize()
            assert int(st.workspace[:4].view(torch.int32).item()) == 0
            assert torch.equal(st.topk_idx, rs.topk_idx), (step.__name__, t)
            assert torch.equal(r_s, r_r) and torch.equal(xs, xr), (step.__name__, t)
            _check(refs, st, rec, stats)
