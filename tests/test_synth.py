"""Properties of the seeded synthetic-layer generator."""

import numpy as np
import pytest

import synth
from oracle.numerics import bf16_bits_to_f64, e4m3_decode


def test_deterministic_and_shapes():
    a = synth.dense_layer(synth.spec_for("tiny_fp32"))
    b = synth.dense_layer(synth.spec_for("tiny_fp32"))
    for k in ("x", "idx", "w", "w_gate_up", "w_down"):
        assert np.array_equal(a[k], b[k])
    assert a["x"].shape == (32, 128) and a["w_gate_up"].shape == (8, 512, 128)
    assert a["w_down"].shape == (8, 128, 256) and a["idx"].dtype == np.int32


def test_router_rules():
    s = synth.spec_for("tiny_fp32")
    idx, w = synth.routing(s)
    assert np.allclose(w.sum(axis=1), 1, atol=1e-6)              # renormalised
    assert (np.diff(w, axis=1) <= 0).all()                        # descending
    assert all(len(set(r)) == len(r) for r in idx)                # distinct experts
    p = synth.layers.router_probs(s)
    assert np.array_equal(idx[:, 0], p.argmax(axis=1))            # argmax takes the lowest index on ties
    s2 = synth.spec_for("qwen_decode_bf16")
    _, w2 = synth.routing(s2)
    assert (w2.sum(axis=1) < 1).all()                             # no renormalisation


def test_ties_go_to_lower_index():
    s = synth.Spec("tie", T=3, H=128, I=128, E=6, k=2, act="f32", weight="f32")
    p = np.array([[0.1, 0.3, 0.3, 0.1, 0.1, 0.1]])
    order = np.argsort(-p, axis=1, kind="stable")[:, :2]
    assert order.tolist() == [[1, 2]]


def test_prefix_sharing():
    s4 = synth.spec_for("dsv3_prefill_bf16")
    s5 = synth.spec_for("dsv3_fp8_f32scale")
    i4, w4 = synth.routing(s4.with_(T=64))
    i5, w5 = synth.routing(s5.with_(T=32))
    assert np.array_equal(i4[:32], i5) and np.array_equal(w4[:32], w5)
    h2 = synth.hidden(synth.spec_for("qwen_prefill_bf16").with_(T=32))
    h3 = synth.hidden(synth.spec_for("qwen_decode_bf16"))
    assert np.array_equal(h2[:16], h3)


def test_weight_distribution():
    s = synth.spec_for("qwen_prefill_bf16")
    g = bf16_bits_to_f64(synth.expert_gate_up(s, 7))
    d = bf16_bits_to_f64(synth.expert_down(s, 7))
    assert abs(g.std() * np.sqrt(s.H) - 1) < 0.01 and abs(g.mean()) < 1e-3
    assert abs(d.std() * np.sqrt(s.I) - 1) < 0.01


def test_zipf_skew_has_empty_and_hot_experts():
    s = synth.spec_for("dsv3_prefill_bf16").with_(T=1024)
    idx, w = synth.routing(s)
    counts = np.bincount(idx.ravel(), minlength=s.E)
    assert (counts == 0).sum() > 20
    assert counts.max() > 0.9 * s.T


@pytest.mark.parametrize("fmt", ["f32", "ue8m0"])
def test_fp8_block_scales(fmt):
    s = synth.spec_for("dsv3_fp8_f32scale").with_(scale=fmt, H=256, I=256)
    codes, sc = synth.expert_gate_up(s, 3)
    assert codes.shape == (512, 256) and sc.shape == (4, 2)
    raw = synth.layers._draw(s, 3, 0)
    deq = e4m3_decode(codes).reshape(4, 128, 2, 128)
    sv = sc.astype(np.float64) if fmt == "f32" else np.ldexp(1.0, sc.astype(np.int64) - 127)
    deq = (deq * sv[:, None, :, None]).reshape(512, 256)
    # every code decodes within half an e4m3 ulp of the fp32 draw
    rel = np.abs(deq - raw) / np.maximum(np.abs(raw), 1e-30)
    small = np.abs(raw) < np.repeat(np.repeat(sv, 128, 0), 128, 1) * 2.0 ** -6
    assert (rel[~small] <= 2.0 ** -4 + 1e-7).all()
    assert np.isfinite(deq).all()
    if fmt == "ue8m0":
        blocks = np.abs(raw).reshape(4, 128, 2, 128).max(axis=(1, 3))
        assert (blocks / sv <= 448).all() and (blocks / sv > 224).all()
