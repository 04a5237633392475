"""Shared helpers of the GPU parity tests: oracle evaluation and tolerance checks."""

from __future__ import annotations

import numpy as np
import torch

import synth
from oracle.moe import ExpertWeights, forward, out_as_f64

# Per-element bound |gpu - oracle| <= ATOL + RTOL * |oracle|
TOL = {"f32": (1e-4, 1e-4), "bf16": (2e-2, 2e-2)}


def oracle_weights(spec: synth.Spec, layer: dict | None = None) -> ExpertWeights:
    """Oracle view of the expert weights: host arrays if given, else regenerated per expert."""
    if layer is not None and "w_gate_up" in layer and isinstance(layer["w_gate_up"], np.ndarray):
        return ExpertWeights(spec.weight, layer["w_gate_up"], layer["w_down"], spec.scale,
                             layer.get("w_gate_up_scale"), layer.get("w_down_scale"))
    if spec.weight in ("fp8", "fp4"):
        return ExpertWeights(spec.weight, lambda e: synth.expert_gate_up(spec, e)[0],
                             lambda e: synth.expert_down(spec, e)[0], spec.scale,
                             lambda e: synth.expert_gate_up(spec, e)[1],
                             lambda e: synth.expert_down(spec, e)[1])
    return ExpertWeights(spec.weight, lambda e: synth.expert_gate_up(spec, e),
                         lambda e: synth.expert_down(spec, e))


def prefetched_weights(spec: synth.Spec, experts, threads: int = 16) -> ExpertWeights:
    """Oracle view of the given experts' weights, generated on the host in parallel."""
    from concurrent.futures import ThreadPoolExecutor

    experts = sorted(set(int(e) for e in experts))
    with ThreadPoolExecutor(max_workers=threads) as ex:
        gu = dict(zip(experts, ex.map(lambda e: synth.expert_gate_up(spec, e), experts)))
        dn = dict(zip(experts, ex.map(lambda e: synth.expert_down(spec, e), experts)))
    if spec.weight in ("fp8", "fp4"):
        return ExpertWeights(spec.weight, lambda e: gu[e][0], lambda e: dn[e][0], spec.scale,
                             lambda e: gu[e][1], lambda e: dn[e][1])
    return ExpertWeights(spec.weight, lambda e: gu[e], lambda e: dn[e])


def oracle_out(spec, x, idx, w, weights, tokens=None, mode="fast", gate="silu"):
    """Oracle result (rounded to the output type) as fp64, for all tokens or a subset."""
    _, out = forward(x, idx, w, weights, act=spec.act, E=spec.E, mode=mode, tokens=tokens, gate=gate)
    return out_as_f64(out, spec.act)


def gpu_out_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float64).cpu().numpy()


def err_ratio(got: np.ndarray, ref: np.ndarray, act: str) -> float:
    atol, rtol = TOL[act]
    tol = atol + rtol * np.abs(ref)
    r = np.abs(got - ref) / tol
    if not np.isfinite(got).all():
        return float("inf")
    return float(r.max()) if r.size else 0.0


def assert_close(got, ref, act, what=""):
    r = err_ratio(got, ref, act)
    assert r <= 1.0, f"{what}: max |gpu-oracle|/tol = {r:.4g}"
    return r


def sample_tokens(T: int, n: int, seed: int = 123) -> np.ndarray:
    """First, last and n-2 random tokens (sorted, unique)."""
    if T <= n:
        return np.arange(T)
    rng = np.random.default_rng(seed)
    pick = rng.choice(np.arange(1, T - 1), size=n - 2, replace=False)
    return np.unique(np.concatenate([[0, T - 1], pick]))
