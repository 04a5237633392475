"""GPU router step + bookkeeping (moe_route_logits) vs the oracle: chosen ids and the
bookkeeping bit-exact, weights within the float32 tolerance."""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
from oracle.moe import route as oracle_route
from oracle.moe import router_topk

pytestmark = pytest.mark.gpu


def _logits(T, E, seed, ties=True, masked=True):
    rng = np.random.default_rng(seed)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    if ties and E > 3:
        lg[:, E // 2] = lg[:, 1]                 # equal logits: the lower id first
        lg[T // 2, :] = lg[T // 2, 0]            # a row of ties
    if masked and E > 4:
        lg[0, : E // 3] = -np.inf                # masked experts (probability 0)
    return lg


@pytest.mark.parametrize("T,E,k,renorm", [
    (1, 8, 2, False), (16, 60, 4, False), (64, 60, 4, True),        # one-workgroup path
    (4096, 60, 4, False), (3000, 256, 8, True),                     # router kernel + chunks
    (5, 1024, 64, True), (200, 16, 16, False), (1100, 128, 1, True),  # k = 64, k = E, k = 1
])
def test_route_logits(T, E, k, renorm):
    lg = _logits(T, E, seed=T + 7 * E + k)
    idx, w, c, o, p, i = m.route_logits(torch.from_numpy(lg).cuda(), k, renorm)
    torch.cuda.synchronize()
    ridx, rw = router_topk(lg, k, renorm)
    assert np.array_equal(idx.cpu().numpy(), ridx), "chosen experts differ"
    got = w.cpu().numpy().astype(np.float64)
    err = np.abs(got - rw)
    assert (err <= 1e-4 + 1e-4 * np.abs(rw)).all(), f"max weight error {err.max():.3e}"
    for name, g, r in zip(("counts", "offsets", "perm", "inv"), (c, o, p, i), oracle_route(ridx, E)):
        assert np.array_equal(g.cpu().numpy(), r), f"{name} differs"


def test_route_logits_empty_and_bad_k():
    lg = torch.empty((0, 8), dtype=torch.float32, device="cuda")
    idx, w, c, o, p, i = m.route_logits(lg, 2)
    torch.cuda.synchronize()
    assert idx.shape == (0, 2) and (c.cpu() == 0).all() and (o.cpu() == 0).all()
    with pytest.raises(ValueError):
        m.route_logits(torch.zeros((4, 100), dtype=torch.float32, device="cuda"), 65)


@pytest.mark.parametrize("E,k,renorm", [(16, 4, False), (256, 8, True)])
def test_router_then_forward(E, k, renorm):
    """Logits -> the library's router -> the experts forward on its ids and weights, against
    the oracle's router and forward from the same logits (the whole layer after the gate)."""
    import synth
    from synth.device import host_to_tensor
    from moe_helpers import assert_close, gpu_out_f64, oracle_out, oracle_weights
    spec = synth.Spec(f"router_forward_{E}", T=300, H=256, I=256, E=E, k=k, act="bf16", weight="bf16", seed=E + k)
    lg = _logits(spec.T, E, seed=E * 3 + k, ties=True, masked=True)
    idx, w, *_ = m.route_logits(torch.from_numpy(lg).cuda(), k, renorm)
    x = synth.hidden(spec)
    X = host_to_tensor(x, "bf16").cuda()
    ridx, rw = router_topk(lg, k, renorm)
    active = np.unique(ridx)
    gu = np.zeros((E, 2 * spec.I, spec.H), np.uint16)
    dn = np.zeros((E, spec.H, spec.I), np.uint16)
    for e in active:
        gu[e], dn[e] = synth.expert_gate_up(spec, e), synth.expert_down(spec, e)
    out = m.experts_forward(X, idx, w, host_to_tensor(gu, "bf16").cuda(), host_to_tensor(dn, "bf16").cuda())
    ref = oracle_out(spec, x, ridx, rw.astype(np.float32), oracle_weights(spec))
    assert_close(gpu_out_f64(out), ref, "bf16", f"router + forward, E={E}, k={k}")
