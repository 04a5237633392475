"""The experts forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The Experts backends page notes that data-dependent expert computation gets in the way of
CUDA graphs.  Here every launch of the forward has a grid fixed by host-known sizes (T, k,
E, H, I) and the call never waits on the host, so one capture serves any routing: the test
replays the graph several times, with eager work between replays, and once after writing a
different routing into the captured id and weight tensors.  Every replay is checked against
the fp64 oracle of the routing it saw, and deterministic modes bit for bit against the eager
call as well.
"""

import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import device_layer
from moe_helpers import assert_close, gpu_out_f64, oracle_out, oracle_weights

pytestmark = pytest.mark.gpu

CASES = {
    "decode": m.FLAG_FORCE_DECODE,
    "decode_det": m.FLAG_FORCE_DECODE | m.FLAG_DETERMINISTIC,
    "grouped_det": m.FLAG_FORCE_GROUPED | m.FLAG_DETERMINISTIC,
    "grouped_atomic": m.FLAG_FORCE_GROUPED | m.FLAG_ATOMIC_COMBINE,
}


@pytest.mark.parametrize("case", list(CASES))
def test_forward_replays_in_a_graph(case):
    flags = CASES[case]
    spec = synth.Spec("graph", T=96, H=256, I=128, E=6, k=2, act="bf16", weight="bf16", renorm=True, seed=21)
    other = synth.Spec("graph", T=96, H=256, I=128, E=6, k=2, act="bf16", weight="bf16", renorm=True, seed=22)
    D = device_layer(spec, poison_inactive=False)
    weights = oracle_weights(spec)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], flags=flags)
    ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(D["x"])

    def fwd():
        m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], out=out, flags=flags,
                          workspace=ws)

    fwd()
    torch.cuda.synchronize()
    eager = out.clone()
    ref = oracle_out(spec, D["x_host"], D["idx_host"], D["w_host"], weights)
    assert_close(gpu_out_f64(eager), ref, "bf16", f"{case}: eager")

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()

    for i in range(3):
        out.fill_(0.0)          # eager work between replays, on outputs and scratch
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_close(gpu_out_f64(out), ref, "bf16", f"{case}: replay {i}")
        if flags & m.FLAG_DETERMINISTIC:
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"{case}: replay {i} differs"

    # a different routing written into the captured tensors: the same graph follows it
    idx2, w2 = synth.routing(other)
    D["idx"].copy_(torch.from_numpy(idx2))
    D["w"].copy_(torch.from_numpy(w2))
    out.fill_(0.0)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ref2 = oracle_out(spec, D["x_host"], idx2, w2, weights)
    assert_close(gpu_out_f64(out), ref2, "bf16", f"{case}: replay with a new routing")


@pytest.mark.parametrize("weight,scale,flags", [
    ("fp8", "f32", m.FLAG_DETERMINISTIC), ("fp8", "ue8m0", 0), ("fp4", "ue8m0", m.FLAG_DETERMINISTIC),
    ("fp4", "ue8m0", m.FLAG_ATOMIC_COMBINE),
])
def test_quantised_forward_replays_in_a_graph(weight, scale, flags):
    """The e4m3 and FP4 forwards (x quantization, gate_up with the requantising epilogue, down,
    combine) captured once and replayed with eager work in between: every replay equals the
    eager call (bit for bit with the per-slot combine, within float-atomic reordering, far
    inside the tolerance, with the atomic one).  The eager call's parity with the oracle is
    test_gpu_forward's."""
    spec = synth.Spec(f"graph_{weight}", T=160, H=256, I=256, E=6, k=2, act="bf16", weight=weight, scale=scale,
                      seed=23)
    D = device_layer(spec, poison_inactive=False)
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D["w_gate_up_scale"], flags)
    ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(D["x"])

    def fwd():
        m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], D["w_gate_up_scale"],
                          D["w_down_scale"], out=out, flags=flags, workspace=ws)

    fwd()
    torch.cuda.synchronize()
    eager = out.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(0.0)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        if flags & m.FLAG_ATOMIC_COMBINE:
            d = (out.float() - eager.float()).abs()
            assert (d <= 1e-2 * (1 + eager.float().abs())).all(), f"replay {i}: max difference {d.max().item()}"
        else:
            assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs"
