"""One routing per streamed layer, at near ties.

The streamed pipeline routes a layer with moe_route, copies the selected
experts into the slab in rank order, and then runs the layer step on the
slab.  Router inputs from tests/ties.py give two experts logits that are
equal in exact arithmetic but not in fp32, so which of the two is taken (or
in which order) is decided by rounding.  Here:

- moe_route and the fused layer step give the same selection and weights,
  bit for bit (they share the router reduction and the top-K);
- a streamed token equals the resident token bit for bit, every layer;
- the streamed layer's selection is the one moe_route chose, and the slab
  holds exactly those experts' bytes in that order;
- every layer agrees with the oracle (the tie accepts either expert).
"""
import numpy as np
import pytest

import seedgen
import workloads as W
from ties import near_tie_case

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import expert_weight_streaming_amd as ews  # noqa: E402

SHAPES = {
    "tiny_k2": seedgen.CONFIGS["tiny"],
    "tiny_k4": seedgen.CONFIGS["tiny"].replace(K=4),
    "hidden4096": seedgen.CONFIGS["layer"].replace(E=64),
}


@pytest.mark.parametrize("where", ["boundary", "inside"])
@pytest.mark.parametrize("shape", list(SHAPES))
def test_streamed_layer_uses_the_copied_routing(shape, where):
    cfg = SHAPES[shape].replace(layers=2, gamma_sigma=0.25, eps=3e-4, seed=0x5EED0D00 + len(shape))
    print(f"[gpu case] near-tie routing {shape} {where}", flush=True)
    st = W.build_streamed(cfg, layers=2)
    rs = W.resident_twin(st)
    K = cfg.K
    idx = torch.zeros(K, dtype=torch.int32, device="cuda")
    w = torch.zeros(K, dtype=torch.float32, device="cuda")
    rec_s = torch.zeros(3, 2, 1, cfg.D, dtype=torch.float32, device="cuda")
    rec_r = torch.zeros_like(rec_s)
    picks = []
    for seed in range(4):
        Wr, x0, e1, e2 = near_tie_case(cfg.D, cfg.E, K, seed, where)
        st.router[0].copy_(torch.from_numpy(Wr))
        rs.router[0].copy_(torch.from_numpy(Wr))
        v = torch.from_numpy(x0).cuda().view(1, -1)
        # moe_route (what the pipeline copies) against the fused step's own routing
        ews.moe_route(rs.descs[0], v, 1, idx, w, None, rs.workspace)
        r1, x1 = v.clone(), v.clone()
        rs.layer_step(0, r1, x1)
        torch.cuda.synchronize()
        assert torch.equal(idx, rs.topk_idx[0, 0]) and torch.equal(w, rs.topk_w[0, 0]), seed
        # streamed token == resident token
        r_s, x_s, r_r, x_r = v.clone(), v.clone(), v.clone(), v.clone()
        st.step(r_s, x_s, record=rec_s)
        rs.step(r_r, x_r, record=rec_r)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        assert int(rs.workspace[:4].view(torch.int32).item()) == 0
        assert torch.equal(st.topk_idx, rs.topk_idx) and torch.equal(st.topk_w, rs.topk_w), seed
        assert torch.equal(rec_s, rec_r) and torch.equal(x_s, x_r), seed
        # the streamed layer ran under moe_route's routing, on exactly the
        # bytes of those experts in that order (layer 0 used slab slot 0)
        sel0 = [int(e) for e in st.topk_idx[0, 0].tolist()]
        assert sel0 == [int(e) for e in idx.tolist()], seed
        slab0 = st.slab[0].cpu()
        for k, e in enumerate(sel0):
            assert torch.equal(slab0[k * st.bb:(k + 1) * st.bb], st.host_blob(0, e)), (seed, k, e)
        # the oracle, layer by layer, on the recorded inputs
        refs = [W.LayerRef(cfg, l, arena_blobs=st.P) for l in range(2)]
        refs[0].Wr = Wr
        W.check_record(refs, rec_s.cpu().numpy(), st.topk_idx.cpu().numpy(), st.topk_w.cpu().numpy())
        chosen = {e1, e2} & set(sel0)
        if where == "boundary":
            assert len(chosen) == 1, (seed, sel0, e1, e2)
        else:
            assert chosen == {e1, e2} and set(sel0[:2]) == {e1, e2}, (seed, sel0, e1, e2)
        picks.append((e1, e2, sel0))
    print(f"[{shape} {where}] pair and selection per seed: {picks}", flush=True)
