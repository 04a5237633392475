"""Seeded synthetic MoE layers shaped like the models the Experts backends page names.

The page (Hugging Face Transformers docs, "Experts backends", introduction) states
the problem: a router picks k experts per token, and the token's hidden state is
projected through the chosen experts and aggregated with the routing weights.  The
page gives no sizes and no data; the five workloads below are synthetic stand-ins
for its example checkpoints (Qwen1.5-MoE-A2.7B and DeepSeek-V3 shaped layers), with
random weights instead of trained ones.

Everything here is input preparation:
  * hidden states: N(0, 1) draws (fp32, or rounded to bf16 by torch's CPU cast);
  * router: logits N(0, 1) (+ a Zipf-like log-rank bias for the skewed layers),
    softmax in fp64, top-k by descending probability with ties to the lower
    expert index, optional renormalisation, weights handed over as fp32;
  * expert weights: N(0, std = 1/sqrt(fan_in)) fp32 draws, stored as fp32, bf16,
    or OCP e4m3 codes with one scale per 128x128 block (float32 amax/448 scales or
    UE8M0 power-of-two scales), the codes produced by torch's CPU float8 cast;
  * FP4 expert weights (DeepSeek-V4 style packing, two 4-bit codes per byte) are
    drawn as codes directly: uniform random bytes, and one UE8M0 exponent per row and
    32 input channels, uniform in [b0 - 1, b0 + 1] with b0 = 127 - 2 -
    round(log2(sqrt(fan_in))), which keeps the weights' RMS near 1/sqrt(fan_in).

Random streams: numpy PCG64 seeded through SeedSequence(seed).spawn(4) in the
order hidden, logits, expert ranks, weights; the weights child spawns 2*E
children (gate_up of expert e, then down of expert e).  Arrays are filled
sequentially, so layers that differ only in T share their first rows, and layers
with the same (H, I, E, seed) share their weights.
"""

from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np
import torch

# ----------------------------------------------------------------------------- specs


@dataclass(frozen=True)
class Spec:
    """One synthetic MoE layer.

    act:     "f32" | "bf16"            dtype of hidden and out
    weight:  "f32" | "bf16" | "fp8" | "fp4"  storage of W_gate_up / W_down
    scale:   "none" | "f32" | "ue8m0"  block-scale format (fp8; fp4 takes ue8m0)
    routing: "normal" | "zipf"         router logits N(0,1), optionally + log-rank bias
    """

    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    act: str
    weight: str
    scale: str = "none"
    renorm: bool = True
    routing: str = "normal"
    zipf_s: float = 1.1
    seed: int = 0

    @property
    def A(self) -> int:
        return self.T * self.k

    def with_(self, **kw) -> "Spec":
        return replace(self, **kw)


CONFIGS = {
    # Tiny layer, fp32, top-2 of 8 with renormalisation.
    "tiny_fp32": Spec("tiny_fp32", T=32, H=128, I=256, E=8, k=2, act="f32", weight="f32",
                      renorm=True),
    # Qwen1.5-MoE-A2.7B-shaped layer, bf16 prefill, top-4 of 60, no renormalisation.
    "qwen_prefill_bf16": Spec("qwen_prefill_bf16", T=4096, H=2048, I=1408, E=60, k=4,
                              act="bf16", weight="bf16", renorm=False),
    # Same layer, decode regime: 16 tokens (one per sequence).
    "qwen_decode_bf16": Spec("qwen_decode_bf16", T=16, H=2048, I=1408, E=60, k=4,
                             act="bf16", weight="bf16", renorm=False),
    # DeepSeek-V3-shaped routed-expert layer, bf16 prefill, skewed routing, top-8 of 256.
    "dsv3_prefill_bf16": Spec("dsv3_prefill_bf16", T=8192, H=7168, I=2048, E=256, k=8,
                              act="bf16", weight="bf16", renorm=True, routing="zipf"),
    # Same layer with fp8-e4m3 experts, 128x128 float32 block scales.
    "dsv3_fp8_f32scale": Spec("dsv3_fp8_f32scale", T=4096, H=7168, I=2048, E=256, k=8,
                              act="bf16", weight="fp8", scale="f32", renorm=True,
                              routing="zipf"),
    # Same layer with UE8M0 (power-of-two) block scales.
    "dsv3_fp8_ue8m0": Spec("dsv3_fp8_ue8m0", T=4096, H=7168, I=2048, E=256, k=8,
                           act="bf16", weight="fp8", scale="ue8m0", renorm=True,
                           routing="zipf"),
    # Same layer with FP4 (e2m1, two per byte) experts and UE8M0 scales per 1x32 block.
    "dsv3_fp4_ue8m0": Spec("dsv3_fp4_ue8m0", T=4096, H=7168, I=2048, E=256, k=8,
                           act="bf16", weight="fp4", scale="ue8m0", renorm=True,
                           routing="zipf"),
}


def spec_for(name: str, **overrides) -> Spec:
    s = CONFIGS[name]
    return s.with_(**overrides) if overrides else s


# ----------------------------------------------------------------------------- streams

def _children(spec: Spec):
    root = np.random.SeedSequence(spec.seed)
    hid, logit, rank, wts = root.spawn(4)
    return hid, logit, rank, wts


def _weight_child(spec: Spec, e: int, which: int) -> np.random.SeedSequence:
    # Regenerating the spawn list is cheap and keeps expert e's stream a pure
    # function of (seed, E, e, which).
    wts = _children(spec)[3]
    kids = wts.spawn(2 * spec.E)
    return kids[2 * e + which]


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


# ----------------------------------------------------------------------------- casts
# All rounding to storage formats goes through torch's CPU casts (library routines).

def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even (torch cast)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_codes(a: np.ndarray) -> np.ndarray:
    """fp32 array with |a| <= 448 -> OCP e4m3fn codes (uint8) via torch's cast."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


# ----------------------------------------------------------------------------- inputs

def hidden(spec: Spec) -> np.ndarray:
    """Hidden states [T, H]: fp32 (act f32) or bf16 bit patterns (act bf16)."""
    x = _rng(_children(spec)[0]).standard_normal((spec.T, spec.H), dtype=np.float32)
    return x if spec.act == "f32" else to_bf16_bits(x)


def router_probs(spec: Spec) -> np.ndarray:
    """Softmax router probabilities [T, E] in fp64."""
    _, logit_ss, rank_ss, _ = _children(spec)
    logits = _rng(logit_ss).standard_normal((spec.T, spec.E))  # fp64
    if spec.routing == "zipf":
        # Skewed routing: a fixed per-expert bias equal to the log of a Zipf(s)
        # probability mass over a seeded ranking of the experts (up to a constant).
        ranks = _rng(rank_ss).permutation(spec.E) + 1
        logits = logits + (-spec.zipf_s * np.log(ranks.astype(np.float64)))[None, :]
    elif spec.routing != "normal":
        raise ValueError(f"unknown routing {spec.routing!r}")
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    return ex / ex.sum(axis=1, keepdims=True)


def routing(spec: Spec):
    """(topk_idx int32 [T, k], topk_w float32 [T, k]).

    Top-k by descending probability; equal probabilities go to the lower expert
    index (a stable sort of -p keeps index order among ties).
    """
    p = router_probs(spec)
    order = np.argsort(-p, axis=1, kind="stable")[:, : spec.k]
    w = np.take_along_axis(p, order, axis=1)
    if spec.renorm:
        w = w / w.sum(axis=1, keepdims=True)
    return order.astype(np.int32), w.astype(np.float32)


def active_experts(idx: np.ndarray, E: int) -> np.ndarray:
    """Sorted ids of experts that received at least one slot."""
    seen = np.zeros(E, dtype=bool)
    seen[idx.ravel()] = True
    return np.nonzero(seen)[0]


def _draw(spec: Spec, e: int, which: int) -> np.ndarray:
    if which == 0:
        shape, fan_in = (2 * spec.I, spec.H), spec.H
    else:
        shape, fan_in = (spec.H, spec.I), spec.I
    w = _rng(_weight_child(spec, e, which)).standard_normal(shape, dtype=np.float32)
    w *= np.float32(1.0 / math.sqrt(fan_in))
    return w


def _block_quant(w: np.ndarray, fmt: str):
    """128x128 block quantisation of one fp32 expert matrix -> (codes, scales)."""
    R, C = w.shape
    assert R % 128 == 0 and C % 128 == 0
    blocks = w.reshape(R // 128, 128, C // 128, 128)
    amax = np.abs(blocks).max(axis=(1, 3))  # fp32 [R/128, C/128]
    if fmt == "f32":
        s = (amax / np.float32(448.0)).astype(np.float32)
        s[amax == 0] = np.float32(1.0)
        sb = s[:, None, :, None]
        v = np.clip(blocks / sb, np.float32(-448.0), np.float32(448.0))
        scales = s
    elif fmt == "ue8m0":
        r = amax.astype(np.float64) / 448.0
        m, ex = np.frexp(r)  # r = m * 2**ex, m in [0.5, 1)
        n = np.where(m == 0.5, ex - 1, ex).astype(np.int64)  # ceil(log2 r)
        n[amax == 0] = 0
        if (n + 127).min() < 0 or (n + 127).max() > 254:
            raise ValueError("block amax outside the UE8M0 range")
        sb = np.ldexp(np.float32(1.0), n).astype(np.float32)[:, None, :, None]
        v = blocks / sb  # exact: division by a power of two
        scales = (n + 127).astype(np.uint8)
    else:
        raise ValueError(f"unknown scale format {fmt!r}")
    codes = to_e4m3_codes(v.reshape(R, C))
    return codes, scales


def _fp4_codes(spec: Spec, e: int, which: int):
    """Packed FP4 codes [rows, cols/2] and UE8M0 exponents [rows, cols/32] of one matrix."""
    rows, cols = (2 * spec.I, spec.H) if which == 0 else (spec.H, spec.I)
    rng = _rng(_weight_child(spec, e, which))
    packed = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    b0 = 127 - 2 - int(round(math.log2(math.sqrt(cols))))
    scales = rng.integers(b0 - 1, b0 + 2, size=(rows, cols // 32)).astype(np.uint8)
    return packed, scales


def _expert_matrix(spec: Spec, e: int, which: int):
    if spec.weight == "fp4":
        return _fp4_codes(spec, e, which)
    w = _draw(spec, e, which)
    if spec.weight == "f32":
        return w
    if spec.weight == "bf16":
        return to_bf16_bits(w)
    if spec.weight == "fp8":
        return _block_quant(w, spec.scale)
    raise ValueError(f"unknown weight format {spec.weight!r}")


def expert_gate_up(spec: Spec, e: int):
    """W_gate_up[e] [2I, H]: rows [0, I) gate, rows [I, 2I) up.

    fp32 array, bf16 bits, (e4m3 codes, scales [2I/128, H/128]) for fp8, or
    (packed e2m1 bytes [2I, H/2], UE8M0 scales [2I, H/32]) for fp4.
    """
    return _expert_matrix(spec, e, 0)


def expert_down(spec: Spec, e: int):
    """W_down[e] [H, I]; same storage conventions as expert_gate_up."""
    return _expert_matrix(spec, e, 1)


def _stack(spec: Spec, fn, experts, threads: int):
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda e: fn(spec, e), experts))
    if spec.weight in ("fp8", "fp4"):
        return (np.stack([p[0] for p in parts]), np.stack([p[1] for p in parts]))
    return np.stack(parts)


def dense_layer(spec: Spec, threads: int = 8) -> dict:
    """All inputs as host arrays (for layers that fit comfortably in host RAM).

    Keys: x, idx, w, w_gate_up, w_down, and for fp8 / fp4 w_gate_up_scale, w_down_scale.
    """
    idx, w = routing(spec)
    out = {"spec": spec, "x": hidden(spec), "idx": idx, "w": w}
    experts = range(spec.E)
    gu = _stack(spec, expert_gate_up, experts, threads)
    dn = _stack(spec, expert_down, experts, threads)
    if spec.weight in ("fp8", "fp4"):
        out["w_gate_up"], out["w_gate_up_scale"] = gu
        out["w_down"], out["w_down_scale"] = dn
    else:
        out["w_gate_up"], out["w_down"] = gu, dn
    return out
