"""GPU experts forward vs the fp64 oracle, per element, within the stated tolerance.

fp32 layers: |gpu - oracle| <= 1e-4 + 1e-4 |oracle|; bf16 (and fp8, fp4) layers:
|gpu - oracle| <= 2e-2 + 2e-2 |oracle|.  fp8 and fp4 layers requantise the SwiGLU rows to
e4m3 on float32 values; there the requantised rows are read back from the workspace and
checked first (moe_helpers.check_requantised: codes and scales equal to the oracle's except
where an a-priori error bound admits the other rounding, and every GPU choice admissible),
and the output bound is widened by exactly the effect of those admissible differences.
Full-size layers are compared on a set of tokens that reaches every active expert.
Unselected experts are NaN-poisoned in every layer staged by synth.device_layer, so any
read of them shows up as NaN.
"""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import device_layer
import json
import os

from moe_helpers import (assert_close, check_requantised, cover_tokens, covered_experts, err_ratio, gpu_out_f64,
                         oracle_out, oracle_out_threaded, oracle_weights, prefetched_weights, read_requantised)

pytestmark = pytest.mark.gpu

# "grouped": expert-sorted grouped GEMMs with the float-atomic combine; "det": the same
# with per-slot rows summed in slot order (also the default combine for small layers)
PATHS = {"default": 0, "grouped": m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE,
         "slots": m.FLAG_FORCE_GROUPED,   # default combine of small layers (bf16 rows for bf16)
         "det": m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED}


def _run(D, flags=0, workspace=None):
    kw = {}
    if "w_gate_up_scale" in D:
        kw = dict(w_gate_up_scale=D["w_gate_up_scale"], w_down_scale=D["w_down_scale"])
    out = m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], flags=flags,
                            workspace=workspace, **kw)
    torch.cuda.synchronize()
    return out


def _gate(flags):
    return "gelu" if flags & m.FLAG_ACT_GELU else ("relu" if flags & m.FLAG_ACT_RELU else "silu")


def _record(entry: dict):
    """Append one parity record (JSON line) to $MOE_PARITY_LOG when it is set."""
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        with open(path, "a") as fh:
            fh.write(json.dumps(entry) + "\n")


def _full_check(spec, flags, tokens=None, what="", threads=16, D=None):
    """GPU forward of `spec` (staged by device_layer, or the given layer D with its keys) against
    the oracle on `tokens` (all by default), fp8 / fp4 requantised rows checked first."""
    D = device_layer(spec) if D is None else D
    quant = spec.weight in ("fp8", "fp4")
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D.get("w_gate_up_scale"), flags)
    ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device=D["x"].device)
    out = gpu_out_f64(_run(D, flags, ws))
    rows = np.arange(spec.T) if tokens is None else np.asarray(tokens)
    W = prefetched_weights(spec, np.unique(D["idx_host"][rows]))
    gate = _gate(flags)
    capture = {} if quant else None
    ref = oracle_out_threaded(spec, D["x_host"], D["idx_host"], D["w_host"], W, rows, threads=threads, gate=gate,
                              capture=capture)
    got = out[rows]
    name = what or spec.name
    rec = dict(test=name, weight=spec.weight, scale=spec.scale, T=spec.T, H=spec.H, I=spec.I, E=spec.E, k=spec.k,
               flags=flags, tokens=len(rows), active=len(D["active"]),
               covered=len(covered_experts(D["idx_host"], rows)),
               err_over_tol=err_ratio(got, ref, spec.act))
    extra = None
    if quant:
        codes_g, scales_g = read_requantised(ws, m.plan_describe(prob), spec.A, spec.I)
        extra, st = check_requantised(spec, D["x_host"], D["idx_host"], D["w_host"], W, capture, codes_g, scales_g,
                                      gate=gate, tokens=rows)
        atol, rtol = (2e-2, 2e-2)
        rec.update(st, err_over_tol_with_allowance=err_ratio(got, ref, spec.act, extra),
                   allowance_over_tol_mean=float(np.mean(extra / (atol + rtol * np.abs(ref)))) if extra.size else 0.0)
        assert st["bad_scales"] == 0, f"{name}: {st['bad_scales']} requantisation scales outside the admissible range"
        assert st["bad_codes"] == 0, f"{name}: {st['bad_codes']} requantised codes outside the admissible roundings"
    print(f"{name} flags={flags}: " + " ".join(f"{k}={v}" for k, v in rec.items() if k not in ("test",)))
    _record(rec)
    return assert_close(got, ref, spec.act, name, extra)


def _layer_cover(spec, flags=0, what=""):
    """A full-size layer compared on tokens that reach every active expert."""
    idx, _ = synth.routing(spec)
    toks = cover_tokens(idx, spec.E)
    active = np.unique(idx)
    assert np.array_equal(covered_experts(idx, toks), active), "the token cover misses an active expert"
    return _full_check(spec, flags, tokens=toks, what=what or f"{spec.name} (cover of all {len(active)} active experts)")


@pytest.mark.parametrize("path", list(PATHS))
def test_tiny_fp32(path):
    _full_check(synth.spec_for("tiny_fp32"), PATHS[path])


@pytest.mark.parametrize("path", ["grouped", "slots", "det", "decode"])
@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=192, E=7, k=3),      # several M tiles, ragged tails
    dict(T=1, H=128, I=64, E=4, k=2),
    dict(T=37, H=384, I=128, E=1, k=1),       # a single expert
    dict(T=50, H=128, I=64, E=6, k=6),        # k == E
    dict(T=129, H=256, I=128, E=64, k=2),     # many empty experts
])
def test_small_bf16(path, shape):
    if path == "decode" and shape["I"] % 128:
        pytest.skip("the decode path takes I % 128 == 0")
    spec = synth.Spec("small_bf16", act="bf16", weight="bf16", renorm=True, seed=7, **shape)
    _full_check(spec, m.FLAG_FORCE_DECODE if path == "decode" else PATHS[path])


@pytest.mark.parametrize("shape", [dict(T=200, H=128, I=64, E=5, k=2), dict(T=3, H=256, I=128, E=3, k=3)])
def test_small_fp32(shape):
    spec = synth.Spec("small_fp32", act="f32", weight="f32", renorm=False, seed=3, **shape)
    _full_check(spec, m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE)
    _full_check(spec, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_GROUPED)


def test_all_tokens_one_expert():
    spec = synth.Spec("one", T=700, H=256, I=128, E=8, k=1, act="bf16", weight="bf16", seed=1)
    D = device_layer(spec, poison_inactive=False)
    D["idx"].fill_(5)
    D["idx_host"][:] = 5
    ref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], oracle_weights(spec))
    for flags in (m.FLAG_FORCE_GROUPED, m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE):
        out = gpu_out_f64(_run(D, flags))
        assert_close(out, ref, "bf16", f"all tokens on one expert, flags {flags}")


@pytest.mark.parametrize("flags", [0, m.FLAG_ATOMIC_COMBINE])   # per-slot rows / float atomics
def test_qwen_prefill_cover(flags):
    _layer_cover(synth.spec_for("qwen_prefill_bf16"), flags)


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


# ----------------------------------------------------------------------------- decode path

@pytest.mark.parametrize("flags", [0, m.FLAG_FORCE_DECODE, m.FLAG_FORCE_DECODE | m.FLAG_DETERMINISTIC,
                                   m.FLAG_FORCE_DECODE | m.FLAG_ATOMIC_COMBINE])
def test_qwen_decode_path(flags):
    spec = synth.spec_for("qwen_decode_bf16")
    D = device_layer(spec)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], flags=flags)
    assert "path=decode" in m.plan_describe(prob)
    _full_check(spec, flags, what=f"qwen_decode decode-path flags={flags}")


@pytest.mark.parametrize("shape", [
    dict(T=64, H=256, I=256, E=4, k=2),       # > 16 tokens per expert: several token passes
    dict(T=1, H=128, I=128, E=8, k=8),        # k == E, one token
    dict(T=33, H=2304, I=128, E=16, k=3),     # H above one staged K slice (2048)
    dict(T=5, H=384, I=2176, E=3, k=1),       # I above one staged K slice for the down projection
])
def test_decode_shapes(shape):
    spec = synth.Spec("decode_bf16", act="bf16", weight="bf16", renorm=True, seed=11, **shape)
    _full_check(spec, m.FLAG_FORCE_DECODE)


@pytest.mark.parametrize("T,flags", [(16, 0), (64, m.FLAG_FORCE_DECODE)])
def test_dsv3_shaped_decode(T, flags):
    # the DeepSeek-V3-shaped bf16 layer with few tokens: K steps of 256 in both decode GEMMs,
    # Zipf-skewed routing (T = 64: hot experts take several 16-row passes)
    spec = synth.spec_for("dsv3_prefill_bf16", T=T)
    D = device_layer(spec)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], flags=flags)
    assert "path=decode" in m.plan_describe(prob)
    out = gpu_out_f64(_run(D, flags))
    ref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], prefetched_weights(spec, D["active"]))
    assert_close(out, ref, "bf16", f"dsv3-shaped decode T={T}")


def test_decode_most_slots():
    # T * k = 2048, the decode path's limit: 32 rounds of the in-LDS ranking, and 51 slots
    # per expert on average, so several 16-row passes per expert
    spec = synth.Spec("decode_max", T=64, H=256, I=128, E=40, k=32, act="bf16", weight="bf16", renorm=True,
                      seed=13)
    _full_check(spec, m.FLAG_FORCE_DECODE)


def test_decode_bad_index_and_repeatability():
    spec = synth.Spec("bad_dec", T=40, H=128, I=128, E=4, k=2, act="bf16", weight="bf16", seed=4)
    D = device_layer(spec, poison_inactive=False)
    D["idx"][7, 1] = 4
    D["idx"][11, 0] = -1
    with pytest.raises(IndexError):
        _run(D, m.FLAG_CHECK_INDICES | m.FLAG_FORCE_DECODE)
    # without the flag the slots contribute nothing
    out = gpu_out_f64(_run(D, m.FLAG_FORCE_DECODE))
    w = D["w_host"].copy()
    idx = D["idx_host"].copy()
    w[7, 1] = w[11, 0] = 0.0
    idx[7, 1] = idx[11, 0] = 0
    ref = oracle_out(spec, D["x_host"], idx, w, oracle_weights(spec))
    assert_close(out, ref, "bf16", "out-of-range slots ignored on the decode path")
    a = _run(D, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_DECODE).clone()
    b = _run(D, m.FLAG_DETERMINISTIC | m.FLAG_FORCE_DECODE)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_decode_matches_grouped_on_tiny_prefill():
    # both paths on the same 96-token layer
    spec = synth.Spec("both", T=96, H=256, I=128, E=6, k=2, act="bf16", weight="bf16", seed=12)
    _full_check(spec, m.FLAG_FORCE_DECODE)
    _full_check(spec, m.FLAG_FORCE_GROUPED)


# ----------------------------------------------------------------------------- fp8 experts

@pytest.mark.parametrize("scale", ["f32", "ue8m0"])
@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=256, E=7, k=3),
    dict(T=1, H=128, I=128, E=4, k=2),
    dict(T=200, H=384, I=128, E=64, k=2),     # many empty experts
    dict(T=40, H=128, I=256, E=3, k=3),       # k == E
])
@pytest.mark.parametrize("flags", [0, m.FLAG_ATOMIC_COMBINE])
def test_small_fp8(scale, shape, flags):
    spec = synth.Spec("small_fp8", act="bf16", weight="fp8", scale=scale, renorm=True, seed=5, **shape)
    _full_check(spec, flags)


@pytest.mark.parametrize("scale", ["f32", "ue8m0"])
def test_small_fp8_deterministic(scale):
    spec = synth.Spec("small_fp8d", T=129, H=256, I=256, E=5, k=2, act="bf16", weight="fp8", scale=scale, seed=6)
    _full_check(spec, m.FLAG_DETERMINISTIC)


@pytest.mark.parametrize("name", ["dsv3_fp8_f32scale", "dsv3_fp8_ue8m0"])
def test_dsv3_fp8_cover(name):
    _layer_cover(synth.spec_for(name))


# ----------------------------------------------------------------------------- fp4 experts

@pytest.mark.parametrize("shape", [
    dict(T=300, H=256, I=256, E=7, k=3),      # several M tiles, ragged tails
    dict(T=1, H=128, I=128, E=4, k=2),
    dict(T=200, H=384, I=128, E=64, k=2),     # many empty experts, a half N tile in down
    dict(T=40, H=128, I=256, E=3, k=3),       # k == E
    dict(T=129, H=512, I=384, E=5, k=2),
    dict(T=37, H=256, I=128, E=1, k=1),       # a single expert
])
@pytest.mark.parametrize("flags", [0, m.FLAG_ATOMIC_COMBINE, m.FLAG_DETERMINISTIC])
def test_small_fp4(shape, flags):
    spec = synth.Spec("small_fp4", act="bf16", weight="fp4", scale="ue8m0", renorm=True, seed=23, **shape)
    _full_check(spec, flags)


def test_fp4_plan():
    spec = synth.Spec("plan_fp4", T=16, H=256, I=128, E=4, k=2, act="bf16", weight="fp4", scale="ue8m0")
    D = device_layer(spec)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D["w_gate_up_scale"])
    assert prob.weight_dtype == m.FP4_E2M1
    assert "weights=fp4_e2m1" in m.plan_describe(prob)


def test_dsv3_fp4_cover():
    _layer_cover(synth.spec_for("dsv3_fp4_ue8m0"))


def test_dsv3_bf16_cover():
    _layer_cover(synth.spec_for("dsv3_prefill_bf16"))


def test_quantize_rows_bit_exact():
    from oracle.moe import quant_rows
    from oracle.numerics import bf16_bits_to_f64
    rng = np.random.default_rng(0)
    x = (rng.standard_normal((37, 384)) * rng.uniform(1e-3, 1e3, (37, 1))).astype(np.float32)
    x[5, 128:256] = 0.0
    x[6, :128] = -0.0
    bits = torch.from_numpy(x).to(torch.bfloat16)
    q, s = m.quantize_rows_fp8(bits.cuda())
    torch.cuda.synchronize()
    xr = bf16_bits_to_f64(bits.view(torch.int16).numpy().view(np.uint16)).astype(np.float32)
    rq, rs = quant_rows(xr)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


def test_quantize_rows_config_hidden_bit_exact():
    # the fp8 layer's own hidden states, all 4096 x 7168
    from oracle.moe import quant_rows
    from oracle.numerics import bf16_bits_to_f64
    spec = synth.spec_for("dsv3_fp8_f32scale")
    xh = synth.hidden(spec)
    q, s = m.quantize_rows_fp8(torch.from_numpy(xh.view(np.int16)).view(torch.bfloat16).cuda())
    torch.cuda.synchronize()
    rq, rs = quant_rows(bf16_bits_to_f64(xh).astype(np.float32))
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), rs.view(np.uint32))


# ----------------------------------------------------------------------------- GeGLU / ReGLU

GATED_CASES = {
    "bf16_grouped": (dict(T=300, H=256, I=192, E=7, k=3, act="bf16", weight="bf16"), m.FLAG_FORCE_GROUPED),
    "bf16_decode": (dict(T=40, H=256, I=256, E=6, k=2, act="bf16", weight="bf16"), m.FLAG_FORCE_DECODE),
    "f32": (dict(T=200, H=128, I=64, E=5, k=2, act="f32", weight="f32"), m.FLAG_FORCE_GROUPED),
    "fp8": (dict(T=200, H=256, I=256, E=5, k=2, act="bf16", weight="fp8", scale="f32"), 0),
    "fp4": (dict(T=200, H=256, I=256, E=5, k=2, act="bf16", weight="fp4", scale="ue8m0"), 0),
}


@pytest.mark.parametrize("gate", ["gelu", "relu"])
@pytest.mark.parametrize("case", list(GATED_CASES))
def test_gated_activations(gate, case):
    shape, flags = GATED_CASES[case]
    spec = synth.Spec(f"gated_{case}", renorm=True, seed=13, **shape)
    gflag = m.FLAG_ACT_GELU if gate == "gelu" else m.FLAG_ACT_RELU
    D = device_layer(spec)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"],
                         D.get("w_gate_up_scale"), flags | gflag)
    assert ("activation=geglu" if gate == "gelu" else "activation=reglu") in m.plan_describe(prob)
    _full_check(spec, flags | gflag, what=f"{case} {gate}")


# ----------------------------------------------------------------------------- limits

@pytest.mark.parametrize("weight", ["bf16", "fp8", "fp4"])
def test_max_experts(weight):
    # E at the library's maximum (1024): most experts empty, 16-bit M-tile tables in LDS
    shape = dict(T=700, H=256, I=128, E=1024, k=8) if weight == "bf16" else dict(T=300, H=256, I=128, E=1024, k=4)
    extra = dict(scale="ue8m0") if weight != "bf16" else {}
    spec = synth.Spec(f"maxE_{weight}", act="bf16", weight=weight, renorm=True, seed=17, **shape, **extra)
    _full_check(spec, m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE)
    _full_check(spec, m.FLAG_FORCE_GROUPED)


@pytest.mark.parametrize("weight", ["bf16", "fp8", "fp4"])
def test_wide_hidden(weight):
    # a long K loop in gate_up (H = 16384: 256 bf16 slices / 128 e4m3 scale blocks) and
    # 64 output tiles in down
    extra = {"bf16": {}, "fp8": dict(scale="f32"), "fp4": dict(scale="ue8m0")}[weight]
    spec = synth.Spec(f"wideH_{weight}", T=96, H=16384, I=128, E=4, k=2, act="bf16", weight=weight,
                      renorm=True, seed=19, **extra)
    _full_check(spec, m.FLAG_FORCE_GROUPED)
