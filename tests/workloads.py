"""Seeded workloads on the GPU and the parity rules used by the GPU tests.

Inputs come from seedgen only (the device generator fills expert arenas,
the host generator router weights and activations); expected values come
from the oracle only.
"""
import numpy as np

import oracle
import seedgen

REL_L2 = 1e-4          # fp32 outputs: relative L2 error bound
MAX_ABS_REL = 1e-3     # and max abs error <= this * max|ref|
NEAR_TIE = 1e-5        # logit gap under which a different top-K set is tolerated


def build_stack(cfg, layers=None, T=1):
    import torch
    from expert_weight_streaming_amd.stack import ResidentStack
    st = ResidentStack(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits,
                       layers=layers or cfg.layers, n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps, n_tokens=T)
    s = torch.cuda.current_stream().cuda_stream
    for l in range(st.layers):
        seedgen.dev_blobs(cfg, l, 0, cfg.E, st.expert_ptr(l, 0), s)
        if cfg.n_shared:
            seedgen.dev_blobs(cfg, l, seedgen.SHARED_ID, 1, st.shared_ptr(l), s)
        st.router[l].copy_(torch.from_numpy(seedgen.router(cfg, l)))
        st.gamma[l].copy_(torch.from_numpy(seedgen.gamma(cfg, l)))
    torch.cuda.synchronize()
    return st


def rel_l2(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def assert_close(got, ref, what, rel=REL_L2, max_abs_rel=MAX_ABS_REL):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    e = rel_l2(got, ref)
    m = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    bound = max_abs_rel * float(np.max(np.abs(ref))) if ref.size else 0.0
    assert e <= rel, f"{what}: rel-L2 {e:.3e} > {rel:.1e}"
    assert m <= bound, f"{what}: max-abs {m:.3e} > {bound:.3e}"
    return e


class LayerRef:
    """Oracle evaluation of one layer of a config, blobs regenerated on the
    host and cached."""

    def __init__(self, cfg, layer, shared=True, arena_blobs=None):
        """arena_blobs: the host arena of a streamed stack holds that many
        blobs and expert (layer, e) reads blob (layer*E + e) mod arena_blobs,
        which holds the seeded blob of (p // E, p % E)."""
        self.cfg, self.layer = cfg, layer
        self.Wr = seedgen.router(cfg, layer)
        self.gamma = seedgen.gamma(cfg, layer)
        self.P = arena_blobs
        self._blobs = {}
        self.shared = seedgen.blob(cfg, layer, seedgen.SHARED_ID) if (shared and cfg.n_shared) else None

    def blob(self, e):
        if e not in self._blobs:
            if self.P is None:
                self._blobs[e] = seedgen.blob(self.cfg, self.layer, e)
            else:
                p = (self.layer * self.cfg.E + e) % self.P
                self._blobs[e] = seedgen.blob(self.cfg, p // self.cfg.E, p % self.cfg.E)
        return self._blobs[e]

    def run(self, r, x, forced_sel=None):
        c = self.cfg
        return oracle.layer(c.D, c.E, c.K, c.I, c.bits, c.group, c.eps, self.Wr, self.gamma, self.blob, self.shared,
                            r, x, forced_sel=forced_sel)


def check_layer(ref: LayerRef, r_in, x_in, gpu_sel, gpu_w, gpu_r, gpu_x, stats=None):
    """Compare one GPU layer step with the oracle on the same (r, x) input.

    Top-K sets must match; a different set is accepted only at a near tie
    (oracle gap < NEAR_TIE), in which case the oracle is rerun with the GPU's
    selection (a valid routing) and the outputs compared against that."""
    res = ref.run(r_in, x_in)
    gsel = [int(e) for e in gpu_sel]
    if sorted(gsel) != sorted(int(e) for e in res["sel"]):
        assert res["gap"] < NEAR_TIE, f"top-K differs ({gsel} vs {list(res['sel'])}) at gap {res['gap']:.3e}"
        if stats is not None:
            stats["near_ties"] = stats.get("near_ties", 0) + 1
        res = ref.run(r_in, x_in, forced_sel=np.array(gsel, np.int32))
    w_ref = dict(zip((int(e) for e in res["sel"]), res["w"]))
    assert_close([gpu_w[k] for k in range(len(gsel))], [w_ref[e] for e in gsel], "routing weights")
    assert_close(gpu_r, res["r"], "residual")
    assert_close(gpu_x, res["x"], "normalised output")
    if stats is not None:
        stats["layers"] = stats.get("layers", 0) + 1
    return res


def check_record(refs, rec, sel, w, stats=None):
    """Every layer of a recorded chain against the oracle, each on the
    (resid, x) the GPU recorded entering it (rec [L+1][2][1][D] or
    [L+1][2][D]; sel, w [L][1][K] or [L][K])."""
    R = np.asarray(rec, np.float32).reshape(len(refs) + 1, 2, -1)
    sel = np.asarray(sel).reshape(len(refs), -1)
    w = np.asarray(w).reshape(len(refs), -1)
    stats = {} if stats is None else stats
    for l, ref in enumerate(refs):
        check_layer(ref, R[l, 0], R[l, 1], sel[l], w[l], R[l + 1, 0], R[l + 1, 1], stats)
    return stats


def build_streamed(cfg, layers=None, arena_blobs=None):
    """A StreamedStack whose host arena holds the seeded blobs: host blob p
    is expert (p // E, p % E); expert (l, e) streams host blob
    (l * E + e) mod arena_blobs."""
    import torch
    from expert_weight_streaming_amd.stack import StreamedStack
    L = layers or cfg.layers
    st = StreamedStack(hidden=cfg.D, n_experts=cfg.E, top_k=cfg.K, inter=cfg.I, bits=cfg.bits, layers=L,
                       n_shared=cfg.n_shared, group=cfg.group, eps=cfg.eps, arena_blobs=arena_blobs)
    s = torch.cuda.current_stream().cuda_stream
    tmp = torch.empty(cfg.E * st.bb, dtype=torch.uint8, device="cuda")
    for p0 in range(0, st.P, cfg.E):
        n = min(cfg.E, st.P - p0)
        seedgen.dev_blobs(cfg, p0 // cfg.E, 0, n, tmp.data_ptr(), s)
        st.host_arena[p0 * st.bb:(p0 + n) * st.bb].copy_(tmp[:n * st.bb])
    for l in range(L):
        if cfg.n_shared:
            seedgen.dev_blobs(cfg, l, seedgen.SHARED_ID, 1, tmp.data_ptr(), s)
            st.host_shared_blob(l).copy_(tmp[:st.bb])
        st.router[l].copy_(torch.from_numpy(seedgen.router(cfg, l)))
        st.gamma[l].copy_(torch.from_numpy(seedgen.gamma(cfg, l)))
    torch.cuda.synchronize()
    return st


def resident_twin(st):
    """A ResidentStack holding exactly the bytes a StreamedStack streams."""
    import torch
    from expert_weight_streaming_amd.stack import ResidentStack
    rs = ResidentStack(hidden=st.D, n_experts=st.E, top_k=st.K, inter=st.I, bits=st.bits, layers=st.layers,
                       n_shared=st.n_shared, group=st.group, eps=st.eps)
    for l in range(st.layers):
        for e in range(st.E):
            rs.arena[(l * st.E + e) * st.bb:(l * st.E + e + 1) * st.bb].copy_(st.host_blob(l, e))
        if st.n_shared:
            rs.shared[l * st.bb:(l + 1) * st.bb].copy_(st.host_shared_blob(l))
    rs.router.copy_(st.router)
    rs.gamma.copy_(st.gamma)
    torch.cuda.synchronize()
    return rs
