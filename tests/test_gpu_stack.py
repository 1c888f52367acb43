"""GPU parity of multi-layer stacks: every layer of every token is compared
with the oracle's own chained evaluation (the oracle feeds itself its own
previous outputs; only a near-tie routing choice is taken from the GPU, as a
valid alternative).  Also: HIP-graph replay equals eager execution bitwise.
"""
import numpy as np
import pytest

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
    cfg = seedgen.CONFIGS["tiny"].replace(bits=bits, layers=6, seed=0x5EED00D0 + bits)
    print(f"[gpu case] tiny stack bits={bits}", flush=True)
    _, stats = run_and_check(cfg, 6, 5)
    assert stats["layers"] == 30
    print(stats)


def test_wide_stack_fresh_tokens():
    cfg = seedgen.CONFIGS["layer"].replace(E=32, layers=4, seed=0x5EED00D7)
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
