"""The allocation-free forward (moe_experts_forward_noalloc) against the forward with a
caller workspace (moe_experts_forward), through the C ABI, on two calls in a row on one GPU,
the second with a smaller input, so the second call runs on the array the first one left
behind.  Paths with a fixed summation order (per-slot rows, the decode path, the
deterministic mode) must agree bit for bit; the float-atomic combine within the bf16
tolerance, and both against the oracle."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import device_layer
from moe_helpers import assert_close, gpu_out_f64, oracle_out, prefetched_weights

pytestmark = pytest.mark.gpu


def _both(D, flags):
    kw = {}
    if "w_gate_up_scale" in D:
        kw = dict(w_gate_up_scale=D["w_gate_up_scale"], w_down_scale=D["w_down_scale"])
    args = (D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"])
    ref = m.experts_forward(*args, flags=flags, **kw)
    out = torch.empty_like(D["x"])
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    got = m.experts_forward_noalloc(*args, out=out, flags=flags, **kw)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    return ref, got


CASES = {
    # name: (layer shapes, flags, bitwise)
    "bf16_slots": (dict(H=2048, I=1408, E=60, k=4, act="bf16", weight="bf16"), m.FLAG_FORCE_GROUPED, True),
    "bf16_atomic": (dict(H=2048, I=1408, E=60, k=4, act="bf16", weight="bf16"),
                    m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE, False),
    "bf16_deterministic": (dict(H=1024, I=512, E=16, k=2, act="bf16", weight="bf16"), m.FLAG_DETERMINISTIC, True),
    "bf16_decode": (dict(H=2048, I=1408, E=60, k=4, act="bf16", weight="bf16"), m.FLAG_FORCE_DECODE, True),
    "fp8_f32_scales": (dict(H=1024, I=512, E=16, k=4, act="bf16", weight="fp8", scale="f32"), 0, True),
    "fp8_ue8m0_scales": (dict(H=1024, I=512, E=16, k=4, act="bf16", weight="fp8", scale="ue8m0"), 0, True),
    "fp4": (dict(H=1024, I=512, E=16, k=4, act="bf16", weight="fp4", scale="ue8m0"), 0, True),
    "f32": (dict(H=256, I=128, E=8, k=2, act="f32", weight="f32"), m.FLAG_FORCE_GROUPED, True),
}


@pytest.mark.parametrize("case", list(CASES))
def test_noalloc_matches_forward_on_two_calls(case):
    shape, flags, bitwise = CASES[case]
    sizes = (96, 17) if flags & m.FLAG_FORCE_DECODE else (1024, 100)   # second call smaller
    for n, T in enumerate(sizes):
        spec = synth.Spec(f"noalloc_{case}", T=T, renorm=True, seed=31 + n, **shape)
        D = device_layer(spec)
        prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D.get("w_gate_up_scale"), flags)
        assert m.workspace_size(prob) <= m.lib().moe_noalloc_scratch_bytes()
        ref, got = _both(D, flags)
        print(f"{case} call {n + 1}: T={T} plan: {m.plan_describe(prob).split(' kernels')[0]}")
        if bitwise:
            assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                               ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32)), \
                f"{case} call {n + 1}: outputs differ"
        act = spec.act
        assert_close(gpu_out_f64(got), gpu_out_f64(ref), act, f"{case} call {n + 1} vs forward")
        if spec.weight not in ("fp8", "fp4"):
            W = prefetched_weights(spec, D["active"])
            oref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], W)
            assert_close(gpu_out_f64(got), oref, act, f"{case} call {n + 1} vs oracle")


def test_noalloc_rejects_a_layer_beyond_its_array():
    spec = synth.Spec("noalloc_big", T=2048, H=7168, I=2048, E=8, k=8, act="bf16", weight="bf16", seed=3)
    prob = m.Problem(spec.T, spec.H, spec.I, spec.E, spec.k, m.BF16, m.BF16, m.SCALE_NONE, 0)
    assert m.workspace_size(prob) > m.lib().moe_noalloc_scratch_bytes()
    x = torch.zeros((spec.T, spec.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.zeros((spec.T, spec.k), dtype=torch.int32, device="cuda")
    w = torch.zeros((spec.T, spec.k), dtype=torch.float32, device="cuda")
    gu = torch.zeros((spec.E, 2 * spec.I, spec.H), dtype=torch.bfloat16, device="cuda")
    dn = torch.zeros((spec.E, spec.H, spec.I), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError, match="workspace"):
        m.experts_forward_noalloc(x, idx, w, gu, dn)
