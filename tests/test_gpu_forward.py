"""GPU experts forward vs the fp64 oracle, per element, within the stated tolerance.

fp32 layers: |gpu - oracle| <= 1e-4 + 1e-4 |oracle|; bf16 (and fp8) layers:
|gpu - oracle| <= 2e-2 + 2e-2 |oracle|.  Unselected experts are NaN-poisoned in
every layer staged by synth.device_layer, so any read of them shows up as NaN.
"""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import device_layer
from moe_helpers import assert_close, gpu_out_f64, oracle_out, oracle_weights, sample_tokens

pytestmark = pytest.mark.gpu

PATHS = {"default": 0, "grouped": m.FLAG_FORCE_GROUPED, "det": m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED}


def _run(D, flags=0):
    kw = {}
    if "w_gate_up_scale" in D:
        kw = dict(w_gate_up_scale=D["w_gate_up_scale"], w_down_scale=D["w_down_scale"])
    out = m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], flags=flags, **kw)
    torch.cuda.synchronize()
    return out


def _full_check(spec, flags, tokens=None, what=""):
    D = device_layer(spec)
    out = gpu_out_f64(_run(D, flags))
    W = oracle_weights(spec)
    ref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], W, tokens=tokens)
    got = out if tokens is None else out[tokens]
    print(f"{what or spec.name} flags={flags}: T={spec.T} active={len(D['active'])}")
    return assert_close(got, ref, spec.act, what or spec.name)


@pytest.mark.parametrize("path", list(PATHS))
def test_tiny_fp32(path):
    _full_check(synth.spec_for("tiny_fp32"), PATHS[path])


@pytest.mark.parametrize("path", ["grouped", "det"])
@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=192, E=7, k=3),      # several M tiles, ragged tails
    dict(T=1, H=128, I=64, E=4, k=2),
    dict(T=37, H=384, I=128, E=1, k=1),       # a single expert
    dict(T=50, H=128, I=64, E=6, k=6),        # k == E
    dict(T=129, H=256, I=128, E=64, k=2),     # many empty experts
])
def test_small_bf16(path, shape):
    spec = synth.Spec("small_bf16", act="bf16", weight="bf16", renorm=True, seed=7, **shape)
    _full_check(spec, PATHS[path])


@pytest.mark.parametrize("shape", [dict(T=200, H=128, I=64, E=5, k=2), dict(T=3, H=256, I=128, E=3, k=3)])
def test_small_fp32(shape):
    spec = synth.Spec("small_fp32", act="f32", weight="f32", renorm=False, seed=3, **shape)
    _full_check(spec, m.FLAG_FORCE_GROUPED)
    _full_check(spec, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED)


def test_all_tokens_one_expert():
    spec = synth.Spec("one", T=700, H=256, I=128, E=8, k=1, act="bf16", weight="bf16", seed=1)
    D = device_layer(spec, poison_inactive=False)
    D["idx"].fill_(5)
    D["idx_host"][:] = 5
    out = gpu_out_f64(_run(D, m.FLAG_FORCE_GROUPED))
    ref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], oracle_weights(spec))
    assert_close(out, ref, "bf16", "all tokens on one expert")


def test_qwen_prefill_sampled():
    spec = synth.spec_for("qwen_prefill_bf16")
    _full_check(spec, 0, tokens=sample_tokens(spec.T, 192))


def test_qwen_decode_full():
    spec = synth.spec_for("qwen_decode_bf16")
    _full_check(spec, m.FLAG_FORCE_GROUPED, what="qwen_decode grouped")


def test_deterministic_is_bitwise_repeatable():
    spec = synth.Spec("det", T=257, H=256, I=128, E=9, k=4, act="bf16", weight="bf16", seed=2)
    D = device_layer(spec)
    a = _run(D, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED).clone()
    b = _run(D, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_empty_batch_is_noop():
    spec = synth.Spec("e", T=0, H=128, I=64, E=4, k=2, act="bf16", weight="bf16")
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((0, 2), dtype=torch.int32, device="cuda")
    w = torch.empty((0, 2), dtype=torch.float32, device="cuda")
    gu = torch.zeros((4, 128, 128), dtype=torch.bfloat16, device="cuda")
    dn = torch.zeros((4, 128, 64), dtype=torch.bfloat16, device="cuda")
    out = m.experts_forward(x, idx, w, gu, dn)
    torch.cuda.synchronize()
    assert out.shape == (0, 128)


def test_bad_index_flag():
    spec = synth.Spec("bad", T=40, H=128, I=64, E=4, k=2, act="bf16", weight="bf16", seed=4)
    D = device_layer(spec, poison_inactive=False)
    D["idx"][7, 1] = 4
    with pytest.raises(IndexError):
        _run(D, m.FLAG_CHECK_INDICES | m.FLAG_FORCE_GROUPED)
    # without the flag the slot contributes nothing
    out = gpu_out_f64(_run(D, m.FLAG_FORCE_GROUPED))
    w = D["w_host"].copy()
    idx = D["idx_host"].copy()
    w[7, 1] = 0.0
    idx[7, 1] = 0
    ref = oracle_out(spec, D["x_host"], idx, w, oracle_weights(spec))
    assert_close(out, ref, "bf16", "out-of-range slot ignored")
