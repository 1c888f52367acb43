"""GPU parity of multi-layer stacks: every layer of every token is compared
with the oracle's own chained evaluation (the oracle feeds itself its own
previous outputs; only a near-tie routing choice is taken from the GPU, as a
valid alternative).  Also: HIP-graph replay equals eager execution bitwise.
"""
import numpy as np
import pytest

import oracle
import seedgen
import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def run_and_check(cfg, layers, tokens, feedback=True, stats=None):
    st = W.build_stack(cfg, layers=layers)
    refs = [W.LayerRef(cfg, l) for l in range(layers)]
    rec = torch.zeros(layers + 1, 2, 1, cfg.D, dtype=torch.float32, device="cuda")
    v_gpu = torch.from_numpy(seedgen.activation(cfg, 0)).cuda()
    v_orc = seedgen.activation(cfg, 0)
    stats = {} if stats is None else stats
    for t in range(tokens):
        if not feedback and t > 0:
            v_gpu = torch.from_numpy(seedgen.activation(cfg, t)).cuda()
            v_orc = seedgen.activation(cfg, t)
        r, x = v_gpu.clone().view(1, -1), v_gpu.clone().view(1, -1)
        st.step(r, x, record=rec)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0, "device error flags"
        R = rec.cpu().numpy()
        sel = st.topk_idx.cpu().numpy()
        w = st.topk_w.cpu().numpy()
        ro, xo = v_orc.copy(), v_orc.copy()
        for l in range(layers):
            res = W.check_layer(refs[l], ro, xo, sel[l, 0], w[l, 0], R[l + 1, 0, 0], R[l + 1, 1, 0], stats)
            ro, xo = res["r"].astype(np.float32), res["x"].astype(np.float32)
        v_gpu = x.view(-1).clone()
        v_orc = xo
    return st, stats


@pytest.mark.parametrize("bits", [4, 2])
def test_tiny_stack_feedback(bits):
    cfg = seedgen.CONFIGS["tiny"].replace(bits=bits, layers=6, gamma_sigma=0.25, eps=3e-4, seed=0x5EED00D0 + bits)
    print(f"[gpu case] tiny stack bits={bits}", flush=True)
    _, stats = run_and_check(cfg, 6, 5)
    assert stats["layers"] == 30
    print(stats)


def test_wide_stack_fresh_tokens():
    cfg = seedgen.CONFIGS["layer"].replace(E=32, layers=4, gamma_sigma=0.25, eps=1e-4, seed=0x5EED00D7)
    print("[gpu case] hidden-4096 stack", flush=True)
    _, stats = run_and_check(cfg, 4, 3, feedback=False)
    assert stats["layers"] == 12


def test_graph_replay_matches_eager():
    cfg = seedgen.CONFIGS["layer"].replace(E=32, layers=5, seed=0x5EED00D8)
    print("[gpu case] graph replay", flush=True)
    st = W.build_stack(cfg, layers=5)
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    r, x = v.clone(), v.clone()
    st.step(r, x)
    torch.cuda.synchronize()
    want = (r.clone(), x.clone(), st.topk_idx.clone())
    rs, xs = torch.empty_like(v), torch.empty_like(v)
    rs.copy_(v)
    xs.copy_(v)
    g = st.capture(rs, xs)
    for rep in range(4):
        rs.copy_(v)
        xs.copy_(v)
        st.topk_idx.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(rs, want[0]) and torch.equal(xs, want[1]), rep
        assert torch.equal(st.topk_idx, want[2]), rep
        # eager work between replays
        r2, x2 = v.clone(), v.clone()
        st.step(r2, x2)
        torch.cuda.synchronize()
        assert torch.equal(r2, want[0])


@pytest.mark.parametrize("name,bits,layers", [("tiny", 4, 6), ("tiny", 2, 5), ("layer32", 4, 4), ("tiny", 4, 70)])
def test_stack_launch_equals_layer_by_layer(name, bits, layers):
    """moe_stack_step (persistent launches of up to 64 layers) gives the same
    bits as one moe_layer_step per layer, records included."""
    base = seedgen.CONFIGS["layer"].replace(E=32) if name == "layer32" else seedgen.CONFIGS[name]
    cfg = base.replace(bits=bits, layers=layers, gamma_sigma=0.25, seed=0x5EED00E0 + layers + bits)
    print(f"[gpu case] stack launch vs layer steps {name} bits={bits} layers={layers}", flush=True)
    st = W.build_stack(cfg, layers=layers)
    v = torch.from_numpy(seedgen.activation(cfg, 0)).cuda().view(1, -1)
    rec_a = torch.zeros(layers + 1, 2, 1, cfg.D, dtype=torch.float32, device="cuda")
    rec_b = torch.zeros_like(rec_a)
    for t in range(2):
        r1, x1 = v.clone(), v.clone()
        st.step(r1, x1, record=rec_a)
        torch.cuda.synchronize()
        idx1, w1 = st.topk_idx.clone(), st.topk_w.clone()
        r2, x2 = v.clone(), v.clone()
        st.step_layers(r2, x2, record=rec_b)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0, "device error flags"
        assert torch.equal(idx1, st.topk_idx) and torch.equal(w1, st.topk_w)
        assert torch.equal(r1, r2) and torch.equal(x1, x2)
        assert torch.equal(rec_a, rec_b)
        v = x1.clone()


def test_stack_topk_exact_ties_pick_lower_index():
    """Logits that tie exactly, within one lane's elements (indices 64 apart)
    and across lanes, go to the lower expert index in the stack kernel's
    top-K, as in the oracle; the weights follow the oracle's softmax."""
    cfg = seedgen.CONFIGS["tiny"].replace(E=512, K=4, layers=2, seed=0x5EED00F0)
    print("[gpu case] stack top-K exact ties", flush=True)
    st = W.build_stack(cfg, layers=2)
    Wr = np.zeros((cfg.E, cfg.D), np.float32)
    Wr[:, 0] = np.random.default_rng(7).uniform(-1.0, 1.0, cfg.E).astype(np.float32)
    for e in (400, 17):
        Wr[e, 0] = 5.0
    for e in (134, 6, 300, 70):
        Wr[e, 0] = 2.0
    st.router[0].copy_(torch.from_numpy(Wr))
    x = np.zeros(cfg.D, np.float32)
    x[0] = 1.0
    r, xx = torch.from_numpy(x).cuda().view(1, -1), torch.from_numpy(x).cuda().view(1, -1)
    st.step(r, xx)
    torch.cuda.synchronize()
    assert int(st.workspace[:4].view(torch.int32).item()) == 0, "device error flags"
    lo = Wr.astype(np.float64) @ x.astype(np.float64)
    osel, _ = oracle.topk(lo, cfg.K)
    sel = st.topk_idx.cpu().numpy()[0, 0]
    assert list(sel) == list(osel) == [17, 400, 6, 70]
    W.assert_close(st.topk_w.cpu().numpy()[0, 0], oracle.route_weights(lo, osel), "routing weights", rel=1e-5)


def test_layer_plan_is_fused_at_the_pages_shape():
    import expert_weight_streaming_amd as ews
    for bits in (4, 2):
        cfg = seedgen.CONFIGS["layer"].replace(bits=bits)
        st = W.build_stack(cfg.replace(E=8), layers=1)
        d = ews.make_desc(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, n_shared=1, bits=bits,
                          router_w=st.router[0], gamma=st.gamma[0], experts=st.arena, shared=st.shared)
        plan = ews.moe_layer_plan(d, 1)
        print(bits, plan)
        assert plan["fused"] == 1 and plan["scratch"] == 0 and plan["grid"] == plan["n_cu"]
