"""Pins of the oracle's experts forward.

Each test checks the oracle against something other than itself: a hand-reduced
closed-form instance, a dense all-experts evaluation with a routing mask, a
single dense SwiGLU MLP built from torch library routines, invariants of the
definition, and the literal/fast cross-check.
"""

import math

import numpy as np
import pytest
import torch

import synth
from oracle import moe, numerics as nu
from oracle.moe import ExpertWeights, forward, silu


def _weights(layer):
    s = layer["spec"]
    return ExpertWeights(s.weight, layer["w_gate_up"], layer["w_down"], s.scale,
                         layer.get("w_gate_up_scale"), layer.get("w_down_scale"))


def _small(name="tiny_fp32", **kw):
    return synth.dense_layer(synth.spec_for(name, **kw))


# ----------------------------------------------------------------------------- closed form

def test_hand_reduced_instance():
    # Two experts, H=2, I=1.  Expert 0: gate row (1,0), up row (0,1), down column (1,-1).
    # Expert 1: gate row (0,1), up row (1,1), down column (2,0).
    wgu = np.array([[[1, 0], [0, 1]], [[0, 1], [1, 1]]], dtype=np.float32)
    wd = np.array([[[1], [-1]], [[2], [0]]], dtype=np.float32)
    x = np.array([[1, 2], [0.5, -1]], dtype=np.float32)
    idx = np.array([[0, 1], [1, 1]], dtype=np.int32)      # token 1 picks expert 1 twice
    w = np.array([[0.25, 0.75], [0.5, 0.5]], dtype=np.float32)
    acc, out = forward(x, idx, w, ExpertWeights("f32", wgu, wd), act="f32")
    s1 = 1 / (1 + math.exp(-1))          # silu(1)
    s2 = 2 / (1 + math.exp(-2))          # silu(2)
    # token 0: expert 0 -> g=1, u=2, a=2*silu(1), y=(a,-a); expert 1 -> g=2, u=3, a=3*silu(2), y=(2a,0)
    exp0 = [0.25 * 2 * s1 + 0.75 * 2 * 3 * s2, -0.25 * 2 * s1]
    # token 1: expert 1 twice -> g=-1, u=-0.5, a=-0.5*silu(-1)=0.5/(1+e), y=(2a,0), weights sum to 1
    exp1 = [1.0 / (1 + math.e), 0.0]
    assert np.allclose(acc, [exp0, exp1], rtol=1e-15, atol=1e-15)
    assert out.dtype == np.float32


def test_silu_closed_forms():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0, 100.0, -100.0, -800.0, 2.5])
    s = silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 1 / (1 + math.exp(-1))) < 1e-16
    assert abs(s[3] - 30.0) < 1e-11 and abs(s[5] - 100.0) < 1e-30
    assert -1e-11 < s[4] < 0 and -1e-40 < s[6] < 0
    assert s[7] == 0.0 and math.copysign(1, s[7]) == -1.0     # exp overflow -> -0
    # identity: silu(z) - silu(-z) = z
    zz = np.linspace(-50, 50, 1001)
    assert np.allclose(silu(zz) - silu(-zz), zz, rtol=0, atol=1e-12)
    # library routine
    assert np.allclose(silu(zz), torch.nn.functional.silu(torch.from_numpy(zz)).numpy(),
                       rtol=1e-15, atol=1e-300)


# ----------------------------------------------------------------------------- brute force

def _dense_all_experts(x64, idx, w, wgu64, wd64):
    """sum_e M[t,e] MLP_e(x_t) over all E experts; M[t,e] = sum_j w[t,j] [idx[t,j]=e]."""
    T, k = idx.shape
    E, twoI, H = wgu64.shape
    I = twoI // 2
    M = np.zeros((T, E))
    for j in range(k):
        M[np.arange(T), idx[:, j]] += w[:, j].astype(np.float64)
    gu = np.einsum("eoh,th->teo", wgu64, x64)              # [T, E, 2I]
    a = torch.nn.functional.silu(torch.from_numpy(gu[..., :I])).numpy() * gu[..., I:]
    y = np.einsum("ehi,tei->teh", wd64, a)                 # [T, E, H]
    return np.einsum("te,teh->th", M, y)


@pytest.mark.parametrize("weight", ["f32", "bf16"])
def test_dense_bruteforce(weight):
    act = "f32" if weight == "f32" else "bf16"
    spec = synth.Spec("t", T=9, H=64, I=32, E=5, k=3, act=act, weight=weight, seed=11)
    L = synth.dense_layer(spec)
    acc, _ = forward(L["x"], L["idx"], L["w"], _weights(L), act=act)
    conv = (lambda a: a.astype(np.float64)) if weight == "f32" else nu.bf16_bits_to_f64
    ref = _dense_all_experts(conv(L["x"]), L["idx"], L["w"], conv(L["w_gate_up"]), conv(L["w_down"]))
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-13)


def _torch_quant_rows(v32):
    """Per-row, per-128 dynamic quantisation using torch's float8 cast for the rounding."""
    R, C = v32.shape
    g = v32.reshape(R, C // 128, 128)
    amax = np.abs(g).max(axis=2)
    s = np.where(amax == 0, np.float32(1), amax / np.float32(448)).astype(np.float32)
    q = torch.from_numpy((g / s[..., None]).astype(np.float32)).to(torch.float8_e4m3fn)
    return (q.double().numpy() * s[..., None].astype(np.float64)).reshape(R, C)


@pytest.mark.parametrize("scale", ["f32", "ue8m0"])
def test_fp8_dense_bruteforce(scale):
    spec = synth.Spec("t8", T=6, H=256, I=128, E=4, k=2, act="bf16", weight="fp8",
                      scale=scale, seed=5)
    L = synth.dense_layer(spec)
    acc, _ = forward(L["x"], L["idx"], L["w"], _weights(L), act="bf16")
    # independent dequantisation of the weights with torch's float8 decode
    def deq(codes, sc):
        v = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
        s = sc.astype(np.float64) if scale == "f32" else np.ldexp(1.0, sc.astype(np.int64) - 127)
        return v * np.repeat(np.repeat(s, 128, axis=-2), 128, axis=-1)
    wgu = deq(L["w_gate_up"], L["w_gate_up_scale"])
    wd = deq(L["w_down"], L["w_down_scale"])
    x32 = nu.bf16_bits_to_f64(L["x"]).astype(np.float32)
    xq = _torch_quant_rows(x32)
    T, k = L["idx"].shape
    I = spec.I
    ref = np.zeros((T, spec.H))
    for t in range(T):
        for j in range(k):
            e = L["idx"][t, j]
            gu = wgu[e] @ xq[t]
            a = torch.nn.functional.silu(torch.from_numpy(gu[:I])).numpy() * gu[I:]
            aq = _torch_quant_rows(a.astype(np.float32)[None])[0]
            ref[t] += float(L["w"][t, j]) * (wd[e] @ aq)
    assert np.allclose(acc, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- special case

TORCH_GATES = {"silu": torch.nn.functional.silu,
               "gelu": lambda v: torch.nn.functional.gelu(v, approximate="none"),
               "relu": torch.nn.functional.relu}


@pytest.mark.parametrize("gate", ["silu", "gelu", "relu"])
def test_k1_unit_weight_is_dense_gated_mlp(gate):
    spec = synth.Spec("k1", T=12, H=96, I=48, E=4, k=1, act="f32", weight="f32", seed=3)
    L = synth.dense_layer(spec)
    w1 = np.ones_like(L["w"])
    acc, out = forward(L["x"], L["idx"], w1, _weights(L), act="f32", gate=gate)
    I = spec.I
    for t in range(spec.T):
        e = L["idx"][t, 0]
        W = torch.from_numpy(L["w_gate_up"][e].astype(np.float64))
        wg, wu = W[:I], W[I:]
        xd = torch.from_numpy(L["x"][t].astype(np.float64))
        h = TORCH_GATES[gate](torch.nn.functional.linear(xd, wg)) * torch.nn.functional.linear(xd, wu)
        y = torch.nn.functional.linear(h, torch.from_numpy(L["w_down"][e].astype(np.float64)))
        assert np.allclose(acc[t], y.numpy(), rtol=1e-13, atol=1e-14)


def test_gelu_and_relu_gates():
    from oracle.moe import gelu, relu
    # Phi(1) and Phi(-1) of the standard normal CDF
    assert gelu(np.array([1.0]))[0] == pytest.approx(0.8413447460685429, rel=1e-15)
    assert gelu(np.array([-1.0]))[0] == pytest.approx(-0.15865525393145707, rel=1e-14)
    assert gelu(np.array([0.0]))[0] == 0.0
    zz = np.linspace(-30, 30, 601)
    # Phi(z) + Phi(-z) = 1  =>  gelu(z) - gelu(-z) = z
    assert np.allclose(gelu(zz) - gelu(-zz), zz, rtol=0, atol=1e-13)
    # library routine (its 1 + erf form rounds the far negative tail to 0, hence the atol)
    assert np.allclose(gelu(zz), torch.nn.functional.gelu(torch.from_numpy(zz), approximate="none").numpy(),
                       rtol=1e-13, atol=1e-15)
    assert (relu(zz) == np.where(zz > 0, zz, 0.0)).all()


def test_gated_literal_equals_fast():
    spec = synth.Spec("g", T=10, H=64, I=32, E=5, k=3, act="f32", weight="f32", seed=9)
    L = synth.dense_layer(spec)
    W = _weights(L)
    for gate in ("gelu", "relu"):
        a1, _ = forward(L["x"], L["idx"], L["w"], W, act="f32", mode="literal", gate=gate)
        a2, _ = forward(L["x"], L["idx"], L["w"], W, act="f32", mode="fast", gate=gate)
        assert np.allclose(a1, a2, rtol=1e-12, atol=1e-14)
        a3, _ = forward(L["x"], L["idx"], L["w"], W, act="f32", gate="silu")
        assert not np.allclose(a1, a3)          # the gate is really applied


# ----------------------------------------------------------------------------- invariants

@pytest.fixture(scope="module")
def tiny():
    return _small()


def test_literal_equals_fast(tiny):
    W = _weights(tiny)
    a1, o1 = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32", mode="literal")
    a2, o2 = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32", mode="fast")
    assert np.allclose(a1, a2, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("scale", ["f32", "ue8m0"])
def test_literal_equals_fast_fp8(scale):
    spec = synth.Spec("t8", T=10, H=256, I=256, E=6, k=3, act="bf16", weight="fp8",
                      scale=scale, seed=9)
    L = synth.dense_layer(spec)
    W = _weights(L)
    a1, _ = forward(L["x"], L["idx"], L["w"], W, act="bf16", mode="literal")
    a2, _ = forward(L["x"], L["idx"], L["w"], W, act="bf16", mode="fast")
    assert np.allclose(a1, a2, rtol=1e-10, atol=1e-12)


def test_weight_scaling_is_linear(tiny):
    W = _weights(tiny)
    a1, _ = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32")
    a2, _ = forward(tiny["x"], tiny["idx"], tiny["w"] * np.float32(0.5), W, act="f32")
    assert np.allclose(a2, 0.5 * a1, rtol=1e-13, atol=1e-15)


def test_slot_swap_and_token_permutation(tiny):
    W = _weights(tiny)
    a1, _ = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32")
    a2, _ = forward(tiny["x"], tiny["idx"][:, ::-1], tiny["w"][:, ::-1], W, act="f32")
    assert np.allclose(a1, a2, rtol=1e-13, atol=1e-15)
    p = np.random.default_rng(0).permutation(tiny["x"].shape[0])
    a3, _ = forward(tiny["x"][p], tiny["idx"][p], tiny["w"][p], W, act="f32")
    assert np.allclose(a3, a1[p], rtol=1e-13, atol=1e-15)


def test_expert_relabelling(tiny):
    E = tiny["spec"].E
    r = np.random.default_rng(1).permutation(E)          # new label of old expert e is r[e]
    inv = np.argsort(r)
    W2 = ExpertWeights("f32", tiny["w_gate_up"][inv], tiny["w_down"][inv])
    a1, _ = forward(tiny["x"], tiny["idx"], tiny["w"], _weights(tiny), act="f32")
    a2, _ = forward(tiny["x"], r[tiny["idx"]].astype(np.int32), tiny["w"], W2, act="f32")
    assert np.allclose(a1, a2, rtol=1e-13, atol=1e-15)


def test_zero_weight_slot_contributes_nothing(tiny):
    W = _weights(tiny)
    w = tiny["w"].copy()
    w[:, 1] = 0
    idx2 = tiny["idx"].copy()
    idx2[:, 1] = (idx2[:, 1] + 3) % tiny["spec"].E
    a1, _ = forward(tiny["x"], tiny["idx"], w, W, act="f32")
    a2, _ = forward(tiny["x"], idx2, w, W, act="f32")
    # equal up to BLAS blocking (the other experts' row blocks change size)
    assert np.allclose(a1, a2, rtol=1e-13, atol=1e-15)
    a3, _ = forward(tiny["x"], idx2, w, W, act="f32", mode="literal")
    a4, _ = forward(tiny["x"], tiny["idx"], w, W, act="f32", mode="literal")
    assert np.array_equal(a3, a4)


def test_token_subset_matches_full(tiny):
    W = _weights(tiny)
    a1, o1 = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32")
    sub = [5, 0, 31, 7]
    a2, o2 = forward(tiny["x"], tiny["idx"], tiny["w"], W, act="f32", tokens=sub)
    assert np.allclose(a2, a1[sub], rtol=1e-13, atol=1e-15)


def test_out_of_range_expert_raises(tiny):
    idx = tiny["idx"].copy()
    idx[3, 0] = tiny["spec"].E
    with pytest.raises(IndexError):
        forward(tiny["x"], idx, tiny["w"], _weights(tiny), act="f32")


def test_bf16_output_is_single_rne_of_acc():
    spec = synth.Spec("b", T=4, H=128, I=64, E=3, k=2, act="bf16", weight="bf16", seed=4)
    L = synth.dense_layer(spec)
    acc, out = forward(L["x"], L["idx"], L["w"], _weights(L), act="bf16")
    ref = torch.from_numpy(acc).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    # torch rounds fp64 -> bf16 in one step as well; agreement on these values
    assert np.array_equal(out, ref)


# ----------------------------------------------------------------------------- fp8 rows

def test_quant_rows_properties():
    rng = np.random.default_rng(8)
    v = (rng.standard_normal((5, 384)) * rng.uniform(0.01, 100, (5, 1))).astype(np.float32)
    v[2, 128:256] = 0                               # all-zero group -> scale 1, codes 0
    q, s = moe.quant_rows(v)
    assert q.dtype == np.uint8 and s.shape == (5, 3)
    assert s[2, 1] == 1.0 and (q[2, 128:256] == 0).all()
    d = moe.dequant_rows(q, s)
    g = v.reshape(5, 3, 128)
    for r in range(5):
        for c in range(3):
            if r == 2 and c == 1:
                continue
            m = np.argmax(np.abs(g[r, c]))
            assert q[r, c * 128 + m] in (0x7E, 0xFE)    # the group max lands on +-448
    # error bound: half an e4m3 ulp (2^-4 relative for normals; 2^-10 * s in the subnormal range)
    sfull = np.repeat(s, 128, axis=1).astype(np.float64)
    err = np.abs(d - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, sfull * 2.0 ** -10) * (1 + 1e-6)
    assert (err <= bound).all()
