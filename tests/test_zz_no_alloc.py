"""moe_stack_step_noalloc (the stack step on the library's own device
scratch, for callers that cannot allocate) against moe_stack_step with a
caller workspace, through the C ABI: two calls in a row, the second with a
smaller input, then a shape that takes the three-launch path, then the first
shape again (the scratch keeps the state one call hands to the next).
Outputs, selections, weights and per-layer records must be equal bit for
bit, and the caller's error word must stay clear."""
import ctypes

import pytest

import seedgen
import workloads as W

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

import expert_weight_streaming_amd as ews  # noqa: E402


def _pair(cfg, layers, token):
    st = W.build_stack(cfg, layers=layers)
    v = torch.from_numpy(seedgen.activation(cfg, token)).cuda().view(1, -1)
    rec_a = torch.zeros(layers + 1, 2, 1, cfg.D, dtype=torch.float32, device="cuda")
    rec_b = torch.zeros_like(rec_a)
    r_a, x_a = v.clone(), v.clone()
    st.step(r_a, x_a, record=rec_a)
    torch.cuda.synchronize()
    idx_a, w_a = st.topk_idx.clone(), st.topk_w.clone()
    assert int(st.workspace[:4].view(torch.int32).item()) == 0
    flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    r_b, x_b = v.clone(), v.clone()
    idx_b, w_b = torch.zeros_like(idx_a), torch.zeros_like(w_a)
    L = ews.lib()
    rc = L.moe_stack_step_noalloc(st.desc_array, layers, r_b.data_ptr(), x_b.data_ptr(), idx_b.data_ptr(),
                                  w_b.data_ptr(), rec_b.data_ptr(), flags.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == ews.MOE_OK, ews.moe_last_error()
    torch.cuda.synchronize()
    assert int(flags.item()) == 0
    assert torch.equal(idx_a, idx_b) and torch.equal(w_a, w_b)
    assert torch.equal(r_a, r_b) and torch.equal(x_a, x_b)
    assert torch.equal(rec_a, rec_b)
    return st


def test_noalloc_equals_the_workspace_entry_point():
    big = seedgen.CONFIGS["layer"].replace(E=64, gamma_sigma=0.25, seed=0x5EED0B01)
    small = seedgen.CONFIGS["tiny"].replace(gamma_sigma=0.25, seed=0x5EED0B02)
    three = seedgen.CONFIGS["tiny"].replace(E=600, K=3, seed=0x5EED0B03)
    print("[gpu case] noalloc: hidden-4096, 5 layers", flush=True)
    _pair(big, 5, 0)
    print("[gpu case] noalloc: tiny, 3 layers (smaller input)", flush=True)
    _pair(small, 3, 1)
    print("[gpu case] noalloc: three-launch shape", flush=True)
    st = _pair(three, 2, 2)
    assert ews.moe_layer_plan(st.descs[0])["fused"] == 0
    print("[gpu case] noalloc: hidden-4096 again", flush=True)
    _pair(big, 5, 3)


def test_noalloc_rejects_bad_arguments():
    L = ews.lib()
    cfg = seedgen.CONFIGS["tiny"]
    st = W.build_stack(cfg, layers=1)
    v = torch.zeros(1, cfg.D, device="cuda")
    r = torch.zeros(1, cfg.D, device="cuda")
    bad_flags = torch.zeros(4, dtype=torch.int32, device="cuda").data_ptr() + 2
    args = (r.data_ptr(), v.data_ptr(), st.topk_idx.data_ptr(), st.topk_w.data_ptr(), None)
    assert L.moe_stack_step_noalloc(st.desc_array, 0, *args, None, None) == ews.MOE_EINVAL
    assert L.moe_stack_step_noalloc(st.desc_array, 1, *args, ctypes.c_void_p(bad_flags), None) == ews.MOE_EINVAL
    assert L.moe_stack_step_noalloc(st.desc_array, 1, v.data_ptr(), v.data_ptr(), *args[2:], None, None) \
        == ews.MOE_EINVAL
