"""GPU experts forward vs the fp64 oracle on seeded random layer shapes.

Every case draws its shape, weight format, routing skew, gate and combine/path flags from one
seeded generator, so the shapes between the hand-picked ones (ragged M tiles, half N tiles,
one-slice K loops, empty and single-row experts, k == E) are covered too; the comparison is
the same as in test_gpu_forward (per element within the stated tolerance, and on fp8 / fp4
layers the requantised SwiGLU rows checked against the a-priori admissible roundings).
The mid-size layers (up to 4096 tokens: experts with many M tiles, the blocked work-item
order over ragged blocks) are compared on a token cover of every active expert.
"""

import numpy as np
import pytest

import mixture_experts_routed_topk_amd as m
import synth

from test_gpu_forward import _full_check, _layer_cover

pytestmark = pytest.mark.gpu

N_CASES = 48


def _case(i: int):
    rng = np.random.default_rng([2026, i])
    weight = ["bf16", "bf16", "fp8", "fp4"][i % 4]
    scale = {"bf16": "none", "fp8": ["f32", "ue8m0"][int(rng.integers(2))], "fp4": "ue8m0"}[weight]
    T = int(rng.integers(1, 320))
    H = 128 * int(rng.integers(1, 5))
    I = (64 if weight == "bf16" else 128) * int(rng.integers(1, 5))
    E = int(rng.integers(1, 49))
    k = int(rng.integers(1, min(E, 8) + 1))
    routing = ["normal", "zipf"][int(rng.integers(2))]
    flags = [0, m.FLAG_FORCE_GROUPED, m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE,
             m.FLAG_FORCE_GROUPED | m.FLAG_DETERMINISTIC][int(rng.integers(4))]
    if weight == "bf16" and I % 128 == 0 and T * k <= 2048 and rng.integers(3) == 0:
        flags = m.FLAG_FORCE_DECODE
    flags |= [0, 0, m.FLAG_ACT_GELU, m.FLAG_ACT_RELU][int(rng.integers(4))]
    spec = synth.Spec(f"random_{i}", T=T, H=H, I=I, E=E, k=k, act="bf16", weight=weight, scale=scale,
                      renorm=bool(rng.integers(2)), routing=routing, seed=100 + i)
    return spec, flags


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_shape(i):
    spec, flags = _case(i)
    _full_check(spec, flags, what=f"random_{i} {spec.weight} T={spec.T} H={spec.H} I={spec.I} E={spec.E} "
                                  f"k={spec.k} {spec.routing} flags={flags}")


N_MID = 6


def _mid_case(i: int):
    rng = np.random.default_rng([2027, i])
    weight = ["bf16", "fp8", "fp4"][i % 3]
    scale = {"bf16": "none", "fp8": ["f32", "ue8m0"][int(rng.integers(2))], "fp4": "ue8m0"}[weight]
    T = int(rng.integers(600, 4097))
    H = 256 * int(rng.integers(2, 9))
    I = 128 * int(rng.integers(2, 9))
    E = int(rng.integers(8, 65))
    k = int(rng.integers(2, min(E, 8) + 1))
    routing = ["normal", "zipf"][int(rng.integers(2))]
    flags = [0, m.FLAG_ATOMIC_COMBINE, m.FLAG_DETERMINISTIC][int(rng.integers(3))]
    spec = synth.Spec(f"random_mid_{i}", T=T, H=H, I=I, E=E, k=k, act="bf16", weight=weight, scale=scale,
                      renorm=bool(rng.integers(2)), routing=routing, seed=200 + i)
    return spec, flags


@pytest.mark.parametrize("i", range(N_MID))
def test_random_mid_layer(i):
    spec, flags = _mid_case(i)
    _layer_cover(spec, flags, what=f"random_mid_{i} {spec.weight} T={spec.T} H={spec.H} I={spec.I} E={spec.E} "
                                   f"k={spec.k} {spec.routing} flags={flags}")
