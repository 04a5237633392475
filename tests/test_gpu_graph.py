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
