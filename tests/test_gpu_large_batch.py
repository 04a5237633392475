"""A batch so large that the grouped kernels' M-tile table does not fit their LDS copy.

The grouped kernels keep the per-expert M-tile starts in LDS as 16-bit entries and read them
from global memory instead when the layer has 65 536 tiles or more. This layer (1.4 M tokens,
top-8 of 1024 experts, uniform ids: about 10 900 rows and 69 tiles of 160 rows per expert)
crosses that line, and its routing (11.2 M slots) takes the chunked routing kernels. The ids
are drawn directly (uniform), since a router over 1.4 M x 1024 logits is not what is tested.
The output is compared with the fp64 oracle on the first and last tokens and 62 random ones.
"""

import re

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import host_to_tensor
from moe_helpers import assert_close, gpu_out_f64, oracle_out, oracle_weights

pytestmark = pytest.mark.gpu


def test_m_tile_table_beyond_lds():
    spec = synth.Spec("large_batch", T=1_400_000, H=128, I=128, E=1024, k=8, act="bf16", weight="bf16", seed=41)
    rng = np.random.default_rng(41)
    idx = rng.integers(0, spec.E, (spec.T, spec.k)).astype(np.int32)
    w = rng.random((spec.T, spec.k), dtype=np.float32)
    w /= w.sum(axis=1, keepdims=True)
    x = synth.hidden(spec)
    gu = np.stack([synth.expert_gate_up(spec, e) for e in range(spec.E)])
    dn = np.stack([synth.expert_down(spec, e) for e in range(spec.E)])

    dev = torch.device("cuda")
    X = host_to_tensor(x, "bf16").to(dev)
    IDX = torch.from_numpy(idx).to(dev)
    W = torch.from_numpy(w).to(dev)
    GU = host_to_tensor(gu, "bf16").to(dev)
    DN = host_to_tensor(dn, "bf16").to(dev)
    prob = m.problem_for(X, IDX, GU, DN)
    plan = m.plan_describe(prob)
    bm = int(re.search(r"_(\d+)x256_", plan).group(1))          # the grouped kernels' tile rows
    counts = np.bincount(idx.ravel(), minlength=spec.E)
    n_mt = int(np.sum((counts + bm - 1) // bm))
    assert "path=grouped" in plan and n_mt >= 65536, (plan, n_mt)

    out = gpu_out_f64(m.experts_forward(X, IDX, W, GU, DN))
    tokens = np.unique(np.concatenate([[0, spec.T - 1], rng.choice(spec.T, 62, replace=False)]))
    ref = oracle_out(spec, x, idx, w, oracle_weights(spec), tokens=tokens)
    print(f"large batch: {n_mt} M tiles of {bm} rows, plan {plan}")
    assert_close(out[tokens], ref, "bf16", f"large batch ({n_mt} M tiles)")
