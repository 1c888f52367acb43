"""GPU parity of moe_expert_gemv (the dequantised expert GEMVs alone) against
the oracle's expert FFN: every listed expert's h and y, on small and ragged
shapes, a range longer than the grid (workgroups running several experts),
and all 512 experts of a hidden-4096 layer in one launch (sampled experts
compared in full, every output finite)."""
import numpy as np
import pytest

import oracle
import seedgen
import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import expert_weight_streaming_amd as ews  # noqa: E402

CFG = seedgen.CONFIGS
CASES = {
    "tiny4": (CFG["tiny"], 0, 16),
    "tiny2": (CFG["tiny"].replace(bits=2), 0, 16),
    "ragged4": (seedgen.Config("rg", D=320, E=24, K=3, I=192, bits=4, seed=0x5EED0C01), 3, 17),
    "ragged2": (seedgen.Config("rg", D=448, E=40, K=5, I=320, bits=2, seed=0x5EED0C02), 11, 29),
    "deep_inter": (CFG["tiny"].replace(D=128, I=4096, E=8, seed=0x5EED0C03), 1, 6),
    "wide": (CFG["tiny"].replace(D=8192, I=64, E=8, seed=0x5EED0C04), 0, 8),
    "many": (CFG["tiny"].replace(E=900, seed=0x5EED0C05), 0, 900),
}


def run(cfg, first, count, token=0):
    st = W.build_stack(cfg, layers=1)
    x = seedgen.activation(cfg, token)
    h = torch.zeros(count, cfg.I, dtype=torch.float32, device="cuda")
    y = torch.zeros(count, cfg.D, dtype=torch.float32, device="cuda")
    ews.moe_expert_gemv(st.descs[0], torch.from_numpy(x).cuda(), first, count, h, y)
    torch.cuda.synchronize()
    return st, x, h.cpu().numpy(), y.cpu().numpy()


def check(cfg, x, first, h, y, ns):
    x64 = x.astype(np.float64)
    for n in ns:
        oh, oy = oracle.expert(seedgen.blob(cfg, 0, first + n), cfg.D, cfg.I, cfg.bits, cfg.group, x64)
        W.assert_close(h[n], oh, f"h of expert {first + n}")
        W.assert_close(y[n], oy, f"y of expert {first + n}")


@pytest.mark.parametrize("name", list(CASES))
def test_expert_gemv(name):
    cfg, first, count = CASES[name]
    print(f"[gpu case] expert gemv {name}", flush=True)
    st, x, h, y = run(cfg, first, count)
    ns = range(count) if count <= 64 else list(range(0, count, 37)) + [count - 1]
    check(cfg, x, first, h, y, ns)
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(y))


@pytest.mark.parametrize("bits", [4, 2])
def test_expert_gemv_all_512_experts(bits):
    cfg = CFG["layer"].replace(bits=bits, seed=0x5EED0C10 + bits)
    print(f"[gpu case] expert gemv 512 experts bits={bits}", flush=True)
    st, x, h, y = run(cfg, 0, cfg.E, token=3)
    assert np.all(np.isfinite(h)) and np.all(np.isfinite(y))
    check(cfg, x, 0, h, y, [0, 1, 63, 64, 255, 256, 257, 300, 447, 510, 511])
    plan = ews.moe_layer_plan(st.descs[0])
    print(f"[512 experts bits={bits}] stack plan {plan}", flush=True)


def test_expert_gemv_rejects_bad_ranges():
    cfg = CFG["tiny"]
    st = W.build_stack(cfg, layers=1)
    x = torch.zeros(cfg.D, device="cuda")
    h = torch.zeros(cfg.E, cfg.I, device="cuda")
    y = torch.zeros(cfg.E, cfg.D, device="cuda")
    for first, count in ((-1, 2), (0, 0), (10, 7), (0, cfg.E + 1)):
        with pytest.raises(ews.MoeError):
            ews.moe_expert_gemv(st.descs[0], x, first, count, h, y)
