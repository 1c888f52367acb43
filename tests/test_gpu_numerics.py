"""GPU numerics beyond the seeded workloads, each against the oracle:

- an integer probe through moe_expert_forward that both sides must compute
  exactly (scale 1, bias 0, integer codes and activations, gate sums >= 24 so
  that silu(g) == g in fp32, one-hot down codes): GPU == oracle bit for bit,
  and both == the exact integer result;
- a distinct non-unit RMSNorm weight per layer and a non-default epsilon on
  the paths not covered elsewhere: the three-launch stack (a shape the fused
  kernel does not take) and a multi-layer batch, every layer and token;
- activations of wide dynamic range: one +-1e3 value per 32 beside values
  near 1e-3, through x (the input) and through h (up rows whose scale and
  bias are 2^20 times larger), on the fused, three-launch and batched paths;
- one workspace shared by calls with different token counts.
"""
import numpy as np
import pytest

import oracle
import seedgen
import workloads as W
from blobs import pack_blob

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import expert_weight_streaming_amd as ews  # noqa: E402

CFG = seedgen.CONFIGS


# ---- integer probe ------------------------------------------------------------------------

def _probe_blob(D, I, bits, rng, xs):
    """A blob with gate/up codes in [0, 2^bits) (each gate row resampled
    until its sum against every token of xs is >= 24), one-hot down rows
    (code 1), scale 1 and bias 0 everywhere; and its code matrices."""
    top = 1 << bits
    gate = rng.integers(0, top, size=(I, D))
    for i in range(I):
        for _ in range(1000):
            if int(np.min(xs @ gate[i])) >= 24:
                break
            gate[i] = rng.integers(0, top, size=D)
        else:
            raise AssertionError("no gate row with sums >= 24 against every token")
    up = rng.integers(0, top, size=(I, D))
    down = np.zeros((D, I), np.int64)
    down[np.arange(D), rng.integers(0, I, size=D)] = 1
    return pack_blob(gate, up, down, bits), (gate, up, down)


def _exact_expert(mats, x):
    """Integer arithmetic: y = down (g * u) with g = gate x, u = up x (silu(g)
    = g for these g in fp32)."""
    gate, up, down = mats
    g, u = gate @ x, up @ x
    assert np.all(g >= 24)
    h = g * u
    return down @ h, h


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("T", [1, 3])
def test_integer_probe_bit_exact(bits, T):
    D, I, E, K = 256, 128, 4, 2
    print(f"[gpu case] integer probe bits={bits} T={T}", flush=True)
    rng = np.random.default_rng(10 + bits + T)
    # activations in {-1, 0, 1} (mean 0.3, so that gate sums are mostly
    # positive): the fixed-point step (per vector, per chunk or per group of
    # 64) makes them exact digits
    xs = rng.choice([-1, 0, 1], p=[0.2, 0.3, 0.5], size=(T, D))
    blobs, mats = [], []
    for _ in range(E + 1):
        b, m = _probe_blob(D, I, bits, rng, xs)
        blobs.append(b)
        mats.append(m)
    sel = np.stack([rng.permutation(E)[:K] for _ in range(T)]).astype(np.int32)
    wts = np.array([[1.0, 0.5]] * T, np.float32)
    # the exact integer result; every value the GPU forms must be exactly
    # representable (h below 2^21 for the fixed-point digits, sums below 2^22)
    want = np.zeros((T, D))
    for t in range(T):
        ys = [_exact_expert(mats[int(e)], xs[t]) for e in sel[t]]
        ysh = _exact_expert(mats[E], xs[t])
        for (_, h) in ys + [ysh]:
            assert np.max(np.abs(h)) < 2 ** 21
        want[t] = ys[0][0] * 1.0 + ys[1][0] * 0.5 + ysh[0]
        assert np.max(np.abs(ys[0][0]) + 0.5 * np.abs(ys[1][0]) + np.abs(ysh[0])) < 2 ** 22
    # the oracle reaches the same values after its final fp32 rounding
    orc = np.zeros((T, D), np.float32)
    for t in range(T):
        x64 = xs[t].astype(np.float64)
        acc = np.zeros(D)
        for k in range(K):
            acc += float(wts[t, k]) * oracle.expert(blobs[int(sel[t, k])], D, I, bits, 64, x64)[1]
        acc += oracle.expert(blobs[E], D, I, bits, 64, x64)[1]
        orc[t] = acc.astype(np.float32)
    assert np.array_equal(orc.astype(np.float64), want), "oracle differs from the exact integer result"
    # the GPU (T = 1: gate/up and down kernels; T = 3: the grouped matrix-core kernels)
    bb = ews.moe_blob_bytes(D, I, bits, 64)
    arena = torch.from_numpy(np.concatenate(blobs[:E])).cuda()
    shared = torch.from_numpy(blobs[E].copy()).cuda()
    router = torch.zeros(E, D, dtype=torch.float32, device="cuda")
    gamma = torch.ones(D, dtype=torch.float32, device="cuda")
    d = ews.make_desc(hidden=D, n_experts=E, top_k=K, inter=I, n_shared=1, bits=bits, router_w=router,
                      gamma=gamma, experts=arena, shared=shared, blob_bytes=bb)
    ws = torch.zeros(ews.moe_workspace_bytes(d, T), dtype=torch.uint8, device="cuda")
    y = torch.zeros(T, D, dtype=torch.float32, device="cuda")
    xd = torch.from_numpy(xs.astype(np.float32)).cuda()
    ews.moe_expert_forward(d, xd, T, torch.from_numpy(sel).cuda(), torch.from_numpy(wts).cuda(), y, ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 0
    got = y.cpu().numpy()
    bad = np.nonzero(got != orc)
    assert bad[0].size == 0, (bad[0].size, got[bad][:6].tolist(), orc[bad][:6].tolist())


# ---- RMSNorm weight and epsilon on the remaining paths --------------------------------------

def test_gamma_eps_three_launch_stack():
    """600 experts: more than the fused kernel's top-K takes, so every layer
    runs as three launches (route, gate/up, down + norm), chained through
    moe_stack_step; each layer has its own RMSNorm weight."""
    cfg = CFG["tiny"].replace(E=600, K=3, layers=4, gamma_sigma=0.3, eps=1e-3, seed=0x5EED0F10)
    print("[gpu case] three-launch stack with per-layer gamma", flush=True)
    st = W.build_stack(cfg, layers=4)
    assert ews.moe_layer_plan(st.descs[0])["fused"] == 0
    refs = [W.LayerRef(cfg, l) for l in range(4)]
    rec = torch.zeros(5, 2, 1, cfg.D, dtype=torch.float32, device="cuda")
    stats = {}
    for t in range(3):
        v = torch.from_numpy(seedgen.activation(cfg, t)).cuda().view(1, -1)
        r, x = v.clone(), v.clone()
        st.step(r, x, record=rec)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0
        W.check_record(refs, rec.cpu().numpy(), st.topk_idx.cpu().numpy(), st.topk_w.cpu().numpy(), stats)
    assert stats["layers"] == 12


@pytest.mark.parametrize("bits", [4, 2])
def test_gamma_eps_batched_stack(bits):
    """Three layers of 12 tokens each through the grouped path, per-layer
    RMSNorm weights, every layer of every token against the oracle."""
    cfg = CFG["tiny"].replace(bits=bits, layers=3, gamma_sigma=0.3, eps=1e-3, seed=0x5EED0F20 + bits)
    T = 12
    print(f"[gpu case] batched stack with per-layer gamma bits={bits}", flush=True)
    st = W.build_stack(cfg, layers=3, T=T)
    refs = [W.LayerRef(cfg, l) for l in range(3)]
    rec = torch.zeros(4, 2, T, cfg.D, dtype=torch.float32, device="cuda")
    x0 = seedgen.activations(cfg, 0, T)
    r, x = torch.from_numpy(x0.copy()).cuda(), torch.from_numpy(x0.copy()).cuda()
    st.step(r, x, record=rec)
    torch.cuda.synchronize()
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    R = rec.cpu().numpy()
    sel, w = st.topk_idx.cpu().numpy(), st.topk_w.cpu().numpy()
    stats = {}
    for t in range(T):
        W.check_record(refs, R[:, :, t], sel[:, t], w[:, t], stats)
    assert stats["layers"] == 3 * T


# ---- wide dynamic range -------------------------------------------------------------------

def _wide_x(cfg, token):
    v = seedgen.activation(cfg, token).astype(np.float64)
    x = 1e-3 * v
    x[::32] = np.where(v[::32] >= 0, 1e3, -1e3)
    return x.astype(np.float32)


def _loud_rows(blob, cfg):
    """Up rows i = 0 mod 32 with scale and bias 2^20 times larger (bf16
    exponent + 20): h = silu(g) * u then holds one value about 10^6 times
    larger than its neighbours in every 32 (silu(g) is nonzero for every g
    these rows produce)."""
    b = blob.copy()
    mat_q = cfg.D * cfg.I * cfg.bits // 8
    gpr = cfg.D // 64
    off = 3 * mat_q + cfg.I * gpr * 4  # up.sb
    words = b[off:off + cfg.I * gpr * 4].view("<u4").reshape(cfg.I, gpr)
    for half in (0, 16):
        f = (words[::32] >> half) & 0xFFFF
        exp = (f >> 7) & 0xFF
        ok = (exp > 0) & (exp < 200)
        f = np.where(ok, f + (20 << 7), f)
        words[::32] = (words[::32] & ~np.uint32(0xFFFF << half)) | (f.astype(np.uint32) << half)
    return b


class _LoudRef(W.LayerRef):
    def __init__(self, cfg, layer):
        super().__init__(cfg, layer)
        self.shared = _loud_rows(self.shared, cfg) if self.shared is not None else None

    def blob(self, e):
        if e not in self._blobs:
            self._blobs[e] = _loud_rows(seedgen.blob(self.cfg, self.layer, e), self.cfg)
        return self._blobs[e]


@pytest.mark.parametrize("path", ["fused", "three_launch", "batched"])
@pytest.mark.parametrize("loud_h", [False, True])
@pytest.mark.parametrize("bits", [4, 2])
def test_wide_dynamic_range(path, loud_h, bits):
    E = 600 if path == "three_launch" else 16
    cfg = CFG["tiny"].replace(E=E, bits=bits, gamma_sigma=0.2, seed=0x5EED0F30 + bits)
    T = 6 if path == "batched" else 1
    print(f"[gpu case] wide range {path} loud_h={loud_h} bits={bits}", flush=True)
    st = W.build_stack(cfg, layers=1, T=T)
    ref = _LoudRef(cfg, 0) if loud_h else W.LayerRef(cfg, 0)
    if loud_h:
        for e in range(E):
            st.arena[e * st.bb:(e + 1) * st.bb].copy_(torch.from_numpy(ref.blob(e)))
        st.shared[:st.bb].copy_(torch.from_numpy(ref.shared))
    plan = ews.moe_layer_plan(st.descs[0])
    assert plan["fused"] == (1 if path == "fused" else 0) or T > 1
    xs = np.stack([_wide_x(cfg, t) if not loud_h else seedgen.activation(cfg, t) for t in range(T)])
    r, x = torch.from_numpy(xs.copy()).cuda(), torch.from_numpy(xs.copy()).cuda()
    st.layer_step(0, r, x)
    torch.cuda.synchronize()
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    sel, w = st.topk_idx[0].cpu().numpy(), st.topk_w[0].cpu().numpy()
    gr, gx = r.cpu().numpy(), x.cpu().numpy()
    for t in range(T):
        res = W.check_layer(ref, xs[t], xs[t], sel[t], w[t], gr[t], gx[t])
        if loud_h:
            assert np.max(np.abs(res["c"])) > 1e3  # the loud rows did reach the output


# ---- one workspace, several token counts --------------------------------------------------

def test_workspace_shared_by_token_counts():
    """A workspace sized for 40 tokens serves a fused one-token step, a
    40-token batched step and the one-token step again: the batched call's
    scratch never touches the state the fused step hands on (flags stay
    clear, results match fresh runs)."""
    cfg = CFG["layer"].replace(E=64, seed=0x5EED0F40)
    T = 40
    print("[gpu case] workspace shared by token counts", flush=True)
    st = W.build_stack(cfg, layers=2, T=T)
    st1 = W.build_stack(cfg, layers=2, T=1)
    assert ews.moe_workspace_state_bytes(st.descs[0]) == ews.moe_workspace_state_bytes(st1.descs[0])
    v = seedgen.activation(cfg, 0)
    xb = seedgen.activations(cfg, 1, T)

    idx = torch.zeros(2, 1, cfg.K, dtype=torch.int32, device="cuda")
    w = torch.zeros(2, 1, cfg.K, dtype=torch.float32, device="cuda")

    def one(stack):
        r, x = torch.from_numpy(v.copy()).cuda().view(1, -1), torch.from_numpy(v.copy()).cuda().view(1, -1)
        ews.moe_stack_step(stack.desc_array, r, x, idx, w, stack.workspace)
        torch.cuda.synchronize()
        return r.clone(), x.clone()

    want = one(st1)
    for rep in range(2):
        got = one(st)
        assert int(st.workspace[:4].view(torch.int32).item()) == 0, rep
        assert torch.equal(got[0], want[0]) and torch.equal(got[1], want[1]), rep
        rb, xb_d = torch.from_numpy(xb.copy()).cuda(), torch.from_numpy(xb.copy()).cuda()
        st.layer_step(0, rb, xb_d)
        torch.cuda.synchronize()
        assert int(st.workspace[:4].view(torch.int32).item()) == 0, rep
