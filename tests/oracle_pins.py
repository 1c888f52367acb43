"""Pins of the CPU oracle to facts fixed outside it.

Each pin takes a loaded oracle library handle and raises AssertionError when
the oracle disagrees with what the pages, a closed form, a library routine or
a brute-force evaluation fix.  test_oracle_pins.py runs them on the oracle;
test_oracle_mutants.py runs them on copies of the oracle with planted
mistakes and requires every mistake to trip at least one pin.
"""
import json
import math
import os

import numpy as np
import scipy.special

import oracle
import seedgen
import npref

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
MAT_ID = {"gate": 0, "up": 1, "down": 2}


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def _random_blob(D, I, bits, group, seed, s_lo=0.005, s_hi=0.02, b_lo=-0.1, b_hi=0.0):
    cfg = seedgen.Config("pin", D=D, E=4, K=1, I=I, bits=bits, group=group, seed=seed,
                         s_lo=s_lo, s_hi=s_hi, b_lo=b_lo, b_hi=b_hi)
    return seedgen.blob(cfg, 0, 0)


# ---------------------------------------------------------------- sizes
def pin_blob_bytes(L):
    g = _golden("blob_sizes.json")
    D, I, grp = g["expert"]["D"], g["expert"]["I"], g["expert"]["group"]
    b4 = oracle.blob_bytes(D, I, 4, grp, L=L)
    assert b4 / 2**20 == g["per_expert_4bit_printed_mib"], b4
    b2 = oracle.blob_bytes(D, I, 2, grp, L=L)
    total2 = b2 * g["stack"]["layers"] * g["stack"]["experts"]
    assert abs(total2 / 1e9 - g["stack_2bit_printed_gb"]) / g["stack_2bit_printed_gb"] < g["tolerance_2bit_total_rel"], total2
    for D_, I_, bits in [(256, 128, 4), (256, 128, 2), (64, 64, 4), (128, 192, 2)]:
        want = 3 * D_ * I_ * bits // 8 + 3 * D_ * I_ // 64 * 4
        assert oracle.blob_bytes(D_, I_, bits, 64, L=L) == want


# ---------------------------------------------------------------- layout
def pin_layout_golden(L):
    g = _golden("layout_bytes.json")
    D, I, grp = g["D"], g["I"], g["group"]
    for case in g["cases"]:
        bits = case["bits"]
        assert oracle.blob_bytes(D, I, bits, grp, L=L) == case["blob_bytes"]
        blob = np.zeros(case["blob_bytes"], dtype=np.uint8)
        for off, val in case["bytes"].items():
            blob[int(off)] = int(val, 16)
        for mat, r, c, want in case["q"]:
            got = oracle.q(blob, D, I, bits, MAT_ID[mat], r, c, L=L)
            assert got == want, (bits, mat, r, c, got, want)
        for mat, r, c, s, b in case["sb"]:
            got = oracle.sb(blob, D, I, bits, grp, MAT_ID[mat], r, c, L=L)
            assert got == (s, b), (bits, mat, r, c, got, (s, b))
        for mat, r, c, want in case["w"]:
            got = oracle.w(blob, D, I, bits, grp, MAT_ID[mat], r, c, L=L)
            assert got == want, (bits, mat, r, c, got, want)


def pin_unpack_matches_bytewise(L):
    """Every code, scale and bias of a random blob equals the byte-wise numpy
    reading (a differently structured decoder)."""
    for bits, (D, I) in [(4, (128, 64)), (2, (64, 128))]:
        blob = _random_blob(D, I, bits, 64, seed=11 + bits)
        ref = npref.unpack(blob, D, I, bits, 64)
        rng = np.random.default_rng(bits)
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            for _ in range(200):
                r, c = int(rng.integers(rows)), int(rng.integers(cols))
                assert oracle.q(blob, D, I, bits, MAT_ID[name], r, c, L=L) == ref[name + "_q"][r, c]
                assert oracle.w(blob, D, I, bits, 64, MAT_ID[name], r, c, L=L) == ref[name][r, c]


# ---------------------------------------------------------------- dequant
def pin_dequant_closed_form(L):
    """All 2^bits codes times a sweep of bf16 (scale, bias): w == q*s + b."""
    D = I = 64
    s_vals = [0.0, 0.005, 0.0078125, 0.01953125, 0.25, 1.5, -0.75]
    b_vals = [0.0, -0.1, -0.0625, 0.03125, -1.0, 2.5]
    for bits in (4, 2):
        nq = 1 << bits
        rng = np.random.default_rng(bits)
        qs, scales, biases = {}, {}, {}
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            qs[name] = (np.arange(rows * cols) % nq).reshape(rows, cols)
            sv = np.array([npref.bf16_bits(_bf16(v)) for v in s_vals])
            bv = np.array([npref.bf16_bits(_bf16(v)) for v in b_vals])
            scales[name] = sv[rng.integers(len(sv), size=rows)]
            biases[name] = bv[rng.integers(len(bv), size=rows)]
        blob = npref.pack(qs, scales, biases, D, I, bits, 64)
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            for r in range(0, rows, 7):
                s = _bf16_val(scales[name][r])
                b = _bf16_val(biases[name][r])
                for c in range(0, cols, 3):
                    want = int(qs[name][r, c]) * s + b
                    got = oracle.w(blob, D, I, bits, 64, MAT_ID[name], r, c, L=L)
                    assert got == want, (bits, name, r, c, got, want)


def _bf16(v):
    u = int(np.float32(v).view(np.uint32))
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return float(np.uint32(u).view(np.float32))


def _bf16_val(bits16):
    return float(np.uint32(int(bits16) << 16).view(np.float32))


def pin_one_hot(L):
    """x = e_j makes the row product equal the single weight W[i][j]."""
    for bits in (4, 2):
        D, I = 128, 64
        blob = _random_blob(D, I, bits, 64, seed=21 + bits)
        ref = npref.unpack(blob, D, I, bits, 64)
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            for i in (0, rows // 3, rows - 1):
                for j in range(cols):
                    x = np.zeros(cols)
                    x[j] = 1.0
                    for form in (0, 1, 2):
                        got = oracle.row_dot(blob, D, I, bits, 64, MAT_ID[name], i, x, form, L=L)
                        assert got == ref[name][i, j], (bits, name, i, j, form, got, ref[name][i, j])


def pin_fma_forms(L):
    """(q*s+b)*x, fma(q, s*x, b*x) and s*sum(q*x) + b*sum(x) are the same
    number up to fp64 rounding, and equal the dense product."""
    rng = np.random.default_rng(5)
    for bits in (4, 2):
        D, I = 256, 128
        blob = _random_blob(D, I, bits, 64, seed=31 + bits)
        ref = npref.unpack(blob, D, I, bits, 64)
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            x = rng.standard_normal(cols)
            for i in range(0, rows, max(1, rows // 8)):
                vals = [oracle.row_dot(blob, D, I, bits, 64, MAT_ID[name], i, x, f, L=L) for f in (0, 1, 2)]
                want = float(ref[name][i] @ x)
                scale = float(np.abs(ref[name][i]) @ np.abs(x))
                for v in vals:
                    assert abs(v - want) <= 1e-12 * scale, (bits, name, i, vals, want)


def pin_integer_probe(L):
    """scale 1, bias 0 or -8, integer x in [-2, 2]: every row product is an
    exact integer that numpy's integer matmul reproduces."""
    D, I = 128, 64
    rng = np.random.default_rng(9)
    for bits in (4, 2):
        for bias in (0.0, -8.0):
            qs, scales, biases = {}, {}, {}
            for name in npref.MATS:
                rows, cols = npref.dims(D, I, name)
                qs[name] = rng.integers(0, 1 << bits, size=(rows, cols))
                scales[name] = np.full(rows * cols // 64, npref.bf16_bits(1.0))
                biases[name] = np.full(rows * cols // 64, npref.bf16_bits(bias))
            blob = npref.pack(qs, scales, biases, D, I, bits, 64)
            for name in npref.MATS:
                rows, cols = npref.dims(D, I, name)
                x = rng.integers(-2, 3, size=cols)
                want = (qs[name].astype(np.int64) + int(bias)) @ x
                for i in range(rows):
                    got = oracle.row_dot(blob, D, I, bits, 64, MAT_ID[name], i, x.astype(np.float64), 0, L=L)
                    assert got == want[i], (bits, bias, name, i, got, want[i])


# ---------------------------------------------------------------- routing
def pin_topk_sort(L):
    """Top-K equals the first K of a full stable sort by (-logit, index);
    gap = K-th selected minus the best unselected logit."""
    rng = np.random.default_rng(3)
    for E in (1, 2, 16, 512):
        for trial in range(20):
            logits = rng.standard_normal(E)
            order = np.lexsort((np.arange(E), -logits))
            for K in sorted(k for k in {1, 2, min(4, E), E} if k <= E):
                sel, gap = oracle.topk(logits, K, L=L)
                assert list(sel) == list(order[:K]), (E, K, sel, order[:K])
                want_gap = logits[order[K - 1]] - logits[order[K]] if K < E else math.inf
                assert gap == want_gap, (E, K, gap, want_gap)


def pin_topk_ties(L):
    """Exact ties go to the lower index."""
    logits = np.array([0.5, 2.0, 1.0, 2.0, 1.0, 2.0, -3.0, 1.0])
    sel, gap = oracle.topk(logits, 4, L=L)
    assert list(sel) == [1, 3, 5, 2], sel
    assert gap == 0.0, gap
    sel, _ = oracle.topk(np.zeros(16), 3, L=L)
    assert list(sel) == [0, 1, 2], sel
    # the exhaustive tiny case: every K on every permutation-like pattern of ties
    rng = np.random.default_rng(4)
    for _ in range(200):
        logits = rng.integers(0, 4, size=16).astype(np.float64)
        for K in range(1, 17):
            sel, _ = oracle.topk(logits, K, L=L)
            assert list(sel) == list(np.lexsort((np.arange(16), -logits))[:K])


def pin_route_weights(L):
    """w = softmax over the selected logits = the softmax over all E
    renormalised over the selection; sums to 1; non-increasing in rank."""
    rng = np.random.default_rng(6)
    for E, K in [(16, 2), (512, 4), (8, 8), (1, 1)]:
        for _ in range(20):
            logits = rng.standard_normal(E) * 3
            sel, _ = oracle.topk(logits, K, L=L)
            w = oracle.route_weights(logits, sel, L=L)
            assert abs(w.sum() - 1.0) <= 1e-12
            assert np.allclose(w, scipy.special.softmax(logits[sel]), rtol=1e-13, atol=0)
            full = scipy.special.softmax(logits)
            assert np.allclose(w, full[sel] / full[sel].sum(), rtol=1e-12, atol=0)
            assert np.all(np.diff(w) <= 0)


# ---------------------------------------------------------------- expert / layer
def pin_expert_dense(L):
    """One expert equals the dense SwiGLU MLP computed by numpy matmuls."""
    rng = np.random.default_rng(7)
    for bits, (D, I) in [(4, (256, 128)), (2, (128, 192))]:
        blob = _random_blob(D, I, bits, 64, seed=41 + bits)
        ref = npref.unpack(blob, D, I, bits, 64)
        x = rng.standard_normal(D)
        h, y = oracle.expert(blob, D, I, bits, 64, x, L=L)
        h_ref, y_ref = npref.expert(ref, x)
        assert _rel(h, h_ref) < 1e-12, _rel(h, h_ref)
        assert _rel(y, y_ref) < 1e-12, _rel(y, y_ref)


def _dense_layer(cfg, Wr, gamma, blobs, shared, r, x, K):
    """Brute force: evaluate every expert densely, then mask by selection."""
    x64 = x.astype(np.float64)
    logits = Wr.astype(np.float64) @ x64
    order = np.lexsort((np.arange(cfg.E), -logits))
    sel = order[:K]
    ys = np.stack([npref.expert(npref.unpack(b, cfg.D, cfg.I, cfg.bits, cfg.group), x64)[1] for b in blobs])
    mask = np.zeros(cfg.E)
    mask[sel] = scipy.special.softmax(logits[sel])
    c = mask @ ys
    if shared is not None:
        c = c + npref.expert(npref.unpack(shared, cfg.D, cfg.I, cfg.bits, cfg.group), x64)[1]
    rr = r.astype(np.float64) + c
    xx = rr / np.sqrt(np.mean(rr * rr) + cfg.eps) * gamma.astype(np.float64)
    return logits, sel, mask[sel], c, rr, xx


def _check_layer(L, cfg, K, with_shared, gamma=None, r=None, tol=1e-11):
    Wr = seedgen.router(cfg, 0)
    gamma = seedgen.gamma(cfg) if gamma is None else gamma
    blobs = [seedgen.blob(cfg, 0, e) for e in range(cfg.E)]
    shared = seedgen.blob(cfg, 0, seedgen.SHARED_ID) if with_shared else None
    x = seedgen.activation(cfg, 0)
    r = x if r is None else r
    res = oracle.layer(cfg.D, cfg.E, K, cfg.I, cfg.bits, cfg.group, cfg.eps, Wr, gamma, lambda e: blobs[e],
                       shared, r, x, L=L)
    logits, sel, w, c, rr, xx = _dense_layer(cfg, Wr, gamma, blobs, shared, r, x, K)
    assert _rel(res["logits"], logits) < 1e-13
    assert list(res["sel"]) == list(sel), (res["sel"], sel)
    assert _rel(res["w"], w) < 1e-12
    assert _rel(res["c"], c) < tol, _rel(res["c"], c)
    assert _rel(res["r"], rr) < tol
    assert _rel(res["x"], xx) < tol


def pin_layer_tiny_bruteforce(L):
    """The tiny workload (hidden 256, 16 experts, K=2, shared, I=128):
    sparse oracle == dense evaluation of all 17 experts, masked."""
    cfg = seedgen.CONFIGS["tiny"]
    _check_layer(L, cfg, cfg.K, True)
    _check_layer(L, cfg.replace(bits=2), cfg.K, True)


def pin_layer_special_cases(L):
    """K = E (dense softmax mixture) and E = K = 1 without a shared expert
    (a plain SwiGLU MLP followed by residual + RMSNorm)."""
    base = seedgen.CONFIGS["tiny"].replace(E=4, D=128, I=64, seed=77)
    _check_layer(L, base.replace(K=4), 4, True)
    _check_layer(L, base.replace(E=1, K=1), 1, False)


def pin_layer_residual_gamma(L):
    """Separate residual stream r != x and a non-unit gamma."""
    cfg = seedgen.CONFIGS["tiny"].replace(E=4, D=128, I=64, seed=78)
    rng = np.random.default_rng(8)
    gamma = (0.5 + rng.random(cfg.D)).astype(np.float32)
    r = (3.0 * rng.standard_normal(cfg.D)).astype(np.float32)
    _check_layer(L, cfg, 2, True, gamma=gamma, r=r)


def pin_rmsnorm(L):
    """mean(x'^2) = ms/(ms+eps) for gamma = 1; x' is invariant to scaling
    r' as eps -> 0; gamma scales elementwise."""
    rng = np.random.default_rng(10)
    D = 64
    r = rng.standard_normal(D)
    c = rng.standard_normal(D)
    ones = np.ones(D, np.float32)
    for eps in (1e-6, 0.5):
        ro, xo = oracle.resnorm(r, c, ones, eps, L=L)
        assert np.array_equal(ro, r + c)
        ms = np.mean((r + c) ** 2)
        assert abs(np.mean(xo ** 2) - ms / (ms + eps)) < 1e-14
    _, x1 = oracle.resnorm(r, c, ones, 0.0, L=L)
    _, x2 = oracle.resnorm(8 * r, 8 * c, ones, 0.0, L=L)
    assert np.allclose(x1, x2, rtol=1e-14, atol=0)
    gamma = (rng.random(D) + 0.5).astype(np.float32)
    _, xg = oracle.resnorm(r, c, gamma, 0.0, L=L)
    assert np.allclose(xg, x1 * gamma.astype(np.float64), rtol=1e-14, atol=0)


def pin_uniform_layer_golden(L):
    g = _golden("uniform_layer.json")
    sh = g["shape"]
    D, E, K, I, bits, grp, eps = sh["D"], sh["E"], sh["K"], sh["I"], sh["bits"], sh["group"], sh["eps"]

    def uniform_blob(spec):
        qs, sc, bi = {}, {}, {}
        for name in npref.MATS:
            rows, cols = npref.dims(D, I, name)
            qs[name] = np.full((rows, cols), spec["q"])
            sc[name] = np.full(rows * cols // grp, npref.bf16_bits(spec["scale"]))
            bi[name] = np.full(rows * cols // grp, npref.bf16_bits(spec["bias"]))
        return npref.pack(qs, sc, bi, D, I, bits, grp)

    blobs = [uniform_blob(g["experts"][str(e)]) for e in range(E)]
    shared = uniform_blob(g["experts"]["shared"])
    Wr = np.stack([np.full(D, v, np.float32) for v in g["router_rows"]])
    x = np.full(D, g["x"], np.float32)
    res = oracle.layer(D, E, K, I, bits, grp, eps, Wr, np.ones(D, np.float32), lambda e: blobs[e], shared, x, x,
                       L=L)
    e = math.exp
    w0, w1 = 1 / (1 + e(-0.5)), e(-0.5) / (1 + e(-0.5))
    y2 = 1024 / (1 + e(-8))
    y1 = -1024 / (1 + e(8))
    ys = 8192 / (1 + e(-16))
    c = w0 * y2 + w1 * y1 + ys
    rr = 0.5 + c
    xx = rr / math.sqrt(rr * rr + eps)
    assert list(res["sel"]) == [2, 1], res["sel"]
    assert res["gap"] == 0.5
    assert np.allclose(res["logits"], [0.5, 1.0, 1.5], rtol=0, atol=0)
    assert np.allclose(res["w"], [w0, w1], rtol=1e-14, atol=0)
    assert np.allclose(res["c"], c, rtol=1e-13, atol=0)
    assert np.allclose(res["r"], rr, rtol=1e-13, atol=0)
    assert np.allclose(res["x"], xx, rtol=1e-13, atol=0)


# ---------------------------------------------------------------- batching
def pin_group(L):
    """count/offset/perm equal a stable argsort of the flattened selections."""
    rng = np.random.default_rng(12)
    for T, K, E in [(32, 4, 512), (1, 4, 512), (5, 2, 16), (64, 4, 8)]:
        idx = np.stack([rng.choice(E, size=K, replace=False) for _ in range(T)]).astype(np.int32)
        count, offset, perm = oracle.group(idx, E, L=L)
        flat = idx.reshape(-1)
        assert np.array_equal(count, np.bincount(flat, minlength=E))
        assert np.array_equal(offset, np.concatenate([[0], np.cumsum(count)]))
        assert np.array_equal(perm, np.argsort(flat, kind="stable"))


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
