"""Pins of the oracle's FP4 (e2m1) expert weights against facts outside the oracle.

The Experts backends page ("FP8 and FP4 quantized experts" section) names FP4 expert
weights packed two per int8 with UE8M0 scales.  The value set of the 4-bit element is
the OCP Microscaling Formats (MX) v1.0 specification's FP4 (E2M1) table; the scale block
(1 x 32) and the nibble order (element 2j in the low nibble) are readings.
"""

import numpy as np
import pytest
import torch

import synth
from oracle.moe import ExpertWeights, forward
from oracle.numerics import e2m1_decode, fp4_unpack

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

# OCP MX v1.0, FP4 E2M1: the eight non-negative magnitudes, codes 0..7 in order
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_matches_ocp():
    got = e2m1_decode(np.arange(16, dtype=np.uint8))
    assert got[:8].tolist() == OCP_E2M1
    # sign bit: code | 8 is the negation (-0 for code 8)
    assert (-got[:8]).tolist() == got[8:].tolist()
    assert np.signbit(got[8])


def test_e2m1_values_exact_in_e4m3():
    # every e2m1 value is an e4m3 value: torch's float8 cast round-trips them
    v = torch.tensor(OCP_E2M1 + [-x for x in OCP_E2M1], dtype=torch.float32)
    assert torch.equal(v.to(torch.float8_e4m3fn).to(torch.float32), v)


def test_nibble_order():
    packed = np.array([[0x21, 0xF9, 0x70]], dtype=np.uint8)
    codes = fp4_unpack(packed)
    assert codes.tolist() == [[0x1, 0x2, 0x9, 0xF, 0x0, 0x7]]
    assert e2m1_decode(codes).tolist() == [[0.5, 1.0, -0.5, -6.0, 0.0, 6.0]]


def _one_hot_weights(R, C, r, c, code, scale_b):
    packed = np.zeros((R, C // 2), dtype=np.uint8)
    packed[r, c // 2] = code if c % 2 == 0 else code << 4
    scales = np.full((R, C // 32), 127, dtype=np.uint8)
    scales[r, c // 32] = scale_b
    return packed, scales


@pytest.mark.parametrize("r,c,code,b", [(0, 0, 0x3, 127), (5, 33, 0x7, 130), (7, 63, 0xD, 120),
                                        (2, 31, 0x1, 100), (3, 32, 0x6, 150)])
def test_dequant_one_element(r, c, code, b):
    R, C = 8, 64
    packed, scales = _one_hot_weights(R, C, r, c, code, b)
    W = ExpertWeights("fp4", packed[None], packed[None], "ue8m0", scales[None], scales[None])
    d = W.gate_up_f64(0)
    expect = np.zeros((R, C))
    sign = -1.0 if code & 8 else 1.0
    expect[r, c] = sign * OCP_E2M1[code & 7] * 2.0 ** (b - 127)
    assert np.array_equal(d, expect)


def test_scale_block_is_32_columns():
    R, C = 4, 128
    rng = np.random.default_rng(0)
    packed = rng.integers(0, 256, size=(R, C // 2), dtype=np.uint8)
    s0 = np.full((R, C // 32), 127, dtype=np.uint8)
    s1 = s0.copy()
    s1[2, 1] = 131                     # row 2, columns 32..63 times 16
    W0 = ExpertWeights("fp4", packed[None], packed[None], "ue8m0", s0[None], s0[None]).gate_up_f64(0)
    W1 = ExpertWeights("fp4", packed[None], packed[None], "ue8m0", s1[None], s1[None]).gate_up_f64(0)
    ratio = np.ones((R, C))
    ratio[2, 32:64] = 16.0
    assert np.array_equal(W1, W0 * ratio)


def _fp8_twin(packed, scales):
    """The same weights as e4m3 codes (torch's cast of the OCP values) with one UE8M0 scale
    per 128 x 128 block, for fp4 scales that are constant over each such block."""
    R, C2 = packed.shape
    C = 2 * C2
    lo = (packed & 0x0F).astype(np.int64)
    hi = (packed >> 4).astype(np.int64)
    table = np.array(OCP_E2M1 + [-x for x in OCP_E2M1], dtype=np.float32)
    vals = np.empty((R, C), dtype=np.float32)
    vals[:, 0::2] = table[lo]
    vals[:, 1::2] = table[hi]
    codes = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    blk = scales[::128, ::4]
    assert np.array_equal(np.repeat(np.repeat(blk, 128, 0), 4, 1), scales)
    return codes, blk


@pytest.mark.parametrize("gate", ["silu", "gelu"])
def test_forward_equals_fp8_path(gate):
    """With scales constant over 128 x 128 blocks the fp4 forward is the (pinned) fp8
    forward of the same values: same quantised activations, same dequantised weights."""
    T, H, I, E, k = 9, 256, 256, 3, 2
    rng = np.random.default_rng(11)
    spec = synth.Spec("t4", T=T, H=H, I=I, E=E, k=k, act="bf16", weight="fp4", scale="ue8m0", seed=3)
    x = synth.hidden(spec)
    idx, w = synth.routing(spec)
    gu, gus, dn, dns = [], [], [], []
    for _ in range(E):
        p1 = rng.integers(0, 256, size=(2 * I, H // 2), dtype=np.uint8)
        b1 = rng.integers(118, 123, size=(2 * I // 128, H // 128)).astype(np.uint8)
        p2 = rng.integers(0, 256, size=(H, I // 2), dtype=np.uint8)
        b2 = rng.integers(118, 123, size=(H // 128, I // 128)).astype(np.uint8)
        gu.append(p1); gus.append(np.repeat(np.repeat(b1, 128, 0), 4, 1))
        dn.append(p2); dns.append(np.repeat(np.repeat(b2, 128, 0), 4, 1))
    W4 = ExpertWeights("fp4", np.stack(gu), np.stack(dn), "ue8m0", np.stack(gus), np.stack(dns))
    tw = [_fp8_twin(a, b) for a, b in zip(gu, gus)]
    td = [_fp8_twin(a, b) for a, b in zip(dn, dns)]
    W8 = ExpertWeights("fp8", np.stack([t[0] for t in tw]), np.stack([t[0] for t in td]), "ue8m0",
                       np.stack([t[1] for t in tw]), np.stack([t[1] for t in td]))
    a4, o4 = forward(x, idx, w, W4, act="bf16", E=E, gate=gate)
    a8, o8 = forward(x, idx, w, W8, act="bf16", E=E, gate=gate)
    assert np.array_equal(a4, a8)
    assert np.array_equal(o4, o8)


def test_literal_equals_fast_fp4():
    spec = synth.Spec("t4l", T=7, H=128, I=128, E=4, k=3, act="bf16", weight="fp4", scale="ue8m0", seed=8)
    L = synth.dense_layer(spec, threads=2)
    W = ExpertWeights("fp4", L["w_gate_up"], L["w_down"], "ue8m0", L["w_gate_up_scale"], L["w_down_scale"])
    a1, _ = forward(L["x"], L["idx"], L["w"], W, act="bf16", mode="literal")
    a2, _ = forward(L["x"], L["idx"], L["w"], W, act="bf16", mode="fast")
    assert np.allclose(a1, a2, rtol=1e-12, atol=1e-12)


def test_synth_fp4_shapes_and_rms():
    spec = synth.spec_for("dsv3_fp4_ue8m0", T=4, E=2)
    p, s = synth.expert_gate_up(spec, 1)
    assert p.shape == (2 * spec.I, spec.H // 2) and p.dtype == np.uint8
    assert s.shape == (2 * spec.I, spec.H // 32) and s.dtype == np.uint8
    W = ExpertWeights("fp4", lambda e: p, lambda e: p, "ue8m0", lambda e: s, lambda e: s)
    rms = np.sqrt(np.mean(W.gate_up_f64(0) ** 2))
    assert 0.5 / np.sqrt(spec.H) < rms < 2.0 / np.sqrt(spec.H)
