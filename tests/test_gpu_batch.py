"""GPU parity of batched steps (T > 1 tokens per call).

Routing per token as in the single-token tests; the token -> expert grouping
(counts, offsets, stable permutation) bit-exact against the oracle's
grouping of the same selections; every token's layer output against the
oracle; a batch equal (within tolerance) to the same tokens one at a time.
"""
import numpy as np
import pytest

import oracle
import seedgen
import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import expert_weight_streaming_amd as ews  # noqa: E402

CFG = seedgen.CONFIGS


def _grouping(st, T):
    off = ews.moe_workspace_grouping(st.descs[0], T)
    ws = st.workspace.cpu().numpy()
    E, K = st.E, st.K

    def arr(name, n):
        return ws[off[name]:off[name] + 4 * n].view(np.int32).copy()
    return arr("count", E), arr("offset", E + 1), arr("perm", T * K), arr("pos", T * K), arr("act", E), arr("n_act", 1)


def _run_batch(cfg, T, token0=0, r_scale=None):
    st = W.build_stack(cfg, layers=1, T=T)
    x = seedgen.activations(cfg, token0, T)
    r = x.copy() if r_scale is None else (r_scale * seedgen.activations(cfg, token0 + 1000, T)).astype(np.float32)
    rd, xd = torch.from_numpy(r.copy()).cuda(), torch.from_numpy(x.copy()).cuda()
    st.layer_step(0, rd, xd)
    torch.cuda.synchronize()
    return st, r, x, rd.cpu().numpy(), xd.cpu().numpy()


@pytest.mark.parametrize("name,cfg,T", [
    ("tiny_T8", CFG["tiny"], 8),
    ("tiny2_T33", CFG["tiny"].replace(bits=2, gamma_sigma=0.3, eps=1e-3, seed=0x5EED00E1), 33),
    ("ragged_T5_k3", seedgen.Config("rg", D=320, E=24, K=3, I=192, bits=4, router_sigma=0.05, gamma_sigma=0.3,
                                    eps=1e-4, seed=0x5EED00E2), 5),
    ("k8_T64", CFG["tiny"].replace(E=64, K=8, seed=0x5EED00E3), 64),
    ("noshared_T4", CFG["tiny"].replace(n_shared=0, seed=0x5EED00E4), 4),
    ("wide_T20", CFG["tiny"].replace(D=8192, I=64, E=8, K=2, seed=0x5EED00E5), 20),
    ("deep_inter_T6", CFG["tiny"].replace(D=128, I=4096, E=8, K=2, bits=2, seed=0x5EED00E6), 6),
    # 2048 experts (more experts than the other cases by far; top-K over 32 keys per lane)
    ("many_experts_T12", CFG["tiny"].replace(D=256, I=64, E=2048, K=4, seed=0x5EED00E7), 12),
])
def test_batched_layer_step(name, cfg, T):
    print(f"[gpu case] batched layer {name}", flush=True)
    st, r, x, gr, gx = _run_batch(cfg, T, r_scale=2.0)
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    ref = W.LayerRef(cfg, 0)
    sel = st.topk_idx[0].cpu().numpy()
    wts = st.topk_w[0].cpu().numpy()
    stats = {}
    for t in range(T):
        W.check_layer(ref, r[t], x[t], sel[t], wts[t], gr[t], gx[t], stats)
    # grouping: bit-exact against the oracle's grouping of the same selections
    count, offset, perm, pos, act, n_act = _grouping(st, T)
    oc, oo, op = oracle.group(sel, cfg.E)
    assert np.array_equal(count, oc) and np.array_equal(offset, oo) and np.array_equal(perm, op)
    assert np.array_equal(pos[op], np.arange(T * cfg.K))
    assert n_act[0] == int((oc > 0).sum()) and np.array_equal(act[:n_act[0]], np.nonzero(oc)[0])
    print(f"[{name}] {stats}, active experts {n_act[0]}", flush=True)


def test_batched_full_layer_2bit_T32():
    """The 60-layer 2-bit batch workload's layer shape: hidden 4096, 512
    experts, K=4 + shared, 32 tokens."""
    cfg = CFG["stack2_b32"]
    print("[gpu case] batched full layer 2-bit T=32", flush=True)
    st, r, x, gr, gx = _run_batch(cfg, 32)
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    ref = W.LayerRef(cfg, 0)
    sel = st.topk_idx[0].cpu().numpy()
    wts = st.topk_w[0].cpu().numpy()
    stats = {}
    for t in range(32):
        W.check_layer(ref, r[t], x[t], sel[t], wts[t], gr[t], gx[t], stats)
    assert stats["layers"] == 32
    count, offset, perm, _, _, n_act = _grouping(st, 32)
    oc, oo, op = oracle.group(sel, cfg.E)
    assert np.array_equal(count, oc) and np.array_equal(perm, op)
    print(f"[full T=32] {stats} active {n_act[0]}", flush=True)


def test_batched_skewed_routing_many_tokens_per_expert():
    """Tokens close to a common base route mostly to the same experts, so
    experts receive 8+ tokens."""
    cfg = CFG["tiny"].replace(E=16, K=2, seed=0x5EED00E5)
    T = 40
    base = seedgen.activation(cfg, 0)
    x = (base[None, :] + 0.1 * seedgen.activations(cfg, 1, T)).astype(np.float32)
    st = W.build_stack(cfg, layers=1, T=T)
    rd, xd = torch.from_numpy(x.copy()).cuda(), torch.from_numpy(x.copy()).cuda()
    st.layer_step(0, rd, xd)
    torch.cuda.synchronize()
    sel = st.topk_idx[0].cpu().numpy()
    counts = np.bincount(sel.reshape(-1), minlength=cfg.E)
    assert counts.max() >= 8, counts
    ref = W.LayerRef(cfg, 0)
    wts = st.topk_w[0].cpu().numpy()
    gr, gx = rd.cpu().numpy(), xd.cpu().numpy()
    for t in range(T):
        W.check_layer(ref, x[t], x[t], sel[t], wts[t], gr[t], gx[t])


def test_batched_expert_forward_forced_and_batch_equals_singles():
    cfg = CFG["tiny"].replace(seed=0x5EED00E6)
    T = 12
    st = W.build_stack(cfg, layers=1, T=T)
    st1 = W.build_stack(cfg, layers=1, T=1)
    rng = np.random.default_rng(3)
    sel = np.stack([rng.choice(cfg.E, size=cfg.K, replace=False) for _ in range(T)]).astype(np.int32)
    wts = rng.random((T, cfg.K)).astype(np.float32)
    x = seedgen.activations(cfg, 50, T)
    y = torch.zeros(T, cfg.D, device="cuda")
    ews.moe_expert_forward(st.descs[0], torch.from_numpy(x).cuda(), T, torch.from_numpy(sel).cuda(),
                           torch.from_numpy(wts).cuda(), y, st.workspace)
    y1 = torch.zeros(cfg.D, device="cuda")
    ref = W.LayerRef(cfg, 0)
    for t in range(T):
        ews.moe_expert_forward(st1.descs[0], torch.from_numpy(x[t]).cuda(), 1, torch.from_numpy(sel[t]).cuda(),
                               torch.from_numpy(wts[t]).cuda(), y1, st1.workspace)
        torch.cuda.synchronize()
        x64 = x[t].astype(np.float64)
        want = sum(float(wts[t, k]) * oracle.expert(ref.blob(int(sel[t, k])), cfg.D, cfg.I, cfg.bits, cfg.group, x64)[1]
                   for k in range(cfg.K))
        want = want + oracle.expert(ref.shared, cfg.D, cfg.I, cfg.bits, cfg.group, x64)[1]
        W.assert_close(y[t].cpu().numpy(), want, f"batched combine token {t}")
        W.assert_close(y[t].cpu().numpy(), y1.cpu().numpy(), f"batch vs single token {t}", rel=1e-5)


@pytest.mark.parametrize("bits", [4, 2])
def test_batched_matrix_core_path_hidden4096(bits):
    """Hidden 4096, inter 1024, 32 experts, 48 skewed tokens: some selected
    experts receive 8+ tokens (more than one 16-token tile of the grouped
    matrix-core kernels when over 16), a few fewer (one partly filled tile);
    every token against the oracle and against the same token run alone."""
    cfg = CFG["layer"].replace(E=32, bits=bits, gamma_sigma=0.25, eps=1e-4, seed=0x5EED00F0 + bits)
    T = 48
    print(f"[gpu case] hidden-4096 batch bits={bits}", flush=True)
    base = seedgen.activation(cfg, 0)
    x = (base[None, :] + 0.35 * seedgen.activations(cfg, 1, T)).astype(np.float32)
    st = W.build_stack(cfg, layers=1, T=T)
    rd, xd = torch.from_numpy(x.copy()).cuda(), torch.from_numpy(x.copy()).cuda()
    st.layer_step(0, rd, xd)
    torch.cuda.synchronize()
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    sel = st.topk_idx[0].cpu().numpy()
    counts = np.bincount(sel.reshape(-1), minlength=cfg.E)
    big, small = int((counts >= 8).sum()), int(((counts > 0) & (counts < 8)).sum())
    print(f"experts with >= 8 tokens: {big}, with 1..7: {small}", flush=True)
    assert big >= 2 and small >= 1, counts
    ref = W.LayerRef(cfg, 0)
    wts = st.topk_w[0].cpu().numpy()
    gr, gx = rd.cpu().numpy(), xd.cpu().numpy()
    for t in range(T):
        W.check_layer(ref, x[t], x[t], sel[t], wts[t], gr[t], gx[t])
    st1 = W.build_stack(cfg, layers=1, T=1)
    for t in (0, 17, 47):
        r1, x1 = torch.from_numpy(x[t].copy()).cuda().view(1, -1), torch.from_numpy(x[t].copy()).cuda().view(1, -1)
        st1.layer_step(0, r1, x1)
        torch.cuda.synchronize()
        assert sorted(st1.topk_idx[0, 0].cpu().tolist()) == sorted(sel[t].tolist())
        W.assert_close(gx[t], x1[0].cpu().numpy(), f"batch vs single token {t}", rel=1e-5)
