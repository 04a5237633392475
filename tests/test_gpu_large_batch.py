"""A batch so large that the grouped kernels' M-tile table does not fit their LDS copy.

The grouped kernels keep the per-expert M-tile starts in LDS as 16-bit entries and read them
from global memory instead when the layer has 65 536 tiles or more. These layers (1.4 M tokens,
top-8 of 1024 experts, uniform ids: about 10 900 rows per expert, 69 tiles of 160 rows (bf16)
or 86 of 128 (fp8, fp4) each) cross that line, and their routing (11.2 M slots) takes the
chunked routing kernels. The ids are drawn directly (uniform): a router over 1.4 M x 1024
logits is not what is tested. Each layer is compared with the fp64 oracle on the first and last
tokens and 62 random ones, the fp8 and fp4 layers' requantised rows checked as everywhere else.
"""

import re

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import host_to_tensor

from test_gpu_forward import _full_check

pytestmark = pytest.mark.gpu

T, H, I, E, K = 1_400_000, 128, 128, 1024, 8


def _layer(spec, rng):
    """The layer of `spec` with uniform ids and weights, staged like synth.device_layer."""
    idx = rng.integers(0, spec.E, (spec.T, spec.k)).astype(np.int32)
    w = rng.random((spec.T, spec.k), dtype=np.float32)
    w /= w.sum(axis=1, keepdims=True)
    x = synth.hidden(spec)
    dev = torch.device("cuda")
    D = {"spec": spec, "idx_host": idx, "w_host": w, "x_host": x, "active": np.unique(idx)}
    D["x"] = host_to_tensor(x, "bf16").to(dev)
    D["idx"] = torch.from_numpy(idx).to(dev)
    D["w"] = torch.from_numpy(w).to(dev)
    gu = [synth.expert_gate_up(spec, e) for e in range(spec.E)]
    dn = [synth.expert_down(spec, e) for e in range(spec.E)]
    if spec.weight == "bf16":
        D["w_gate_up"] = host_to_tensor(np.stack(gu), "bf16").to(dev)
        D["w_down"] = host_to_tensor(np.stack(dn), "bf16").to(dev)
    else:
        D["w_gate_up"] = torch.from_numpy(np.stack([c for c, _ in gu])).to(dev)
        D["w_down"] = torch.from_numpy(np.stack([c for c, _ in dn])).to(dev)
        D["w_gate_up_scale"] = torch.from_numpy(np.stack([s for _, s in gu])).to(dev)
        D["w_down_scale"] = torch.from_numpy(np.stack([s for _, s in dn])).to(dev)
    return D


@pytest.mark.parametrize("weight", ["bf16", "fp8", "fp4"])
def test_m_tile_table_beyond_lds(weight):
    scale = {"bf16": "none", "fp8": "f32", "fp4": "ue8m0"}[weight]
    spec = synth.Spec(f"large_batch_{weight}", T=T, H=H, I=I, E=E, k=K, act="bf16", weight=weight, scale=scale,
                      seed=41)
    rng = np.random.default_rng(41)
    D = _layer(spec, rng)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D.get("w_gate_up_scale"))
    plan = m.plan_describe(prob)
    bm = int(re.search(r"_(\d+)x256_", plan).group(1))          # the grouped kernels' tile rows
    counts = np.bincount(D["idx_host"].ravel(), minlength=E)
    n_mt = int(np.sum((counts + bm - 1) // bm))
    assert "path=grouped" in plan and n_mt >= 65536, (plan, n_mt)
    tokens = np.unique(np.concatenate([[0, T - 1], rng.choice(T, 62, replace=False)]))
    _full_check(spec, 0, tokens=tokens, D=D, what=f"large batch {weight} ({n_mt} M tiles of {bm} rows)")
