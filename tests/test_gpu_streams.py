"""Concurrent forwards: layers launched on separate streams, and from separate host threads,
each with its own workspace and output, give bit for bit what the same calls give one after
another.

The library keeps no state between calls except a per-device record that is set up once
under a lock. Every launch of a call reads and writes only that call's buffers, so calls on
different streams may overlap on the device in any order. The layers here use the per-slot
combine (MOE_FLAG_DETERMINISTIC), whose results do not depend on timing, so any
interference between the calls shows up as a bit difference. The layers cover the bf16
grouped kernels, the decode kernels, and the e4m3 and FP4 grouped kernels; the bf16 layers'
serial results are also checked against the fp64 oracle (the e4m3 and FP4 layers' parity,
with its requantisation check, is test_gpu_forward's).
"""

import threading

import pytest
import torch

import mixture_experts_routed_topk_amd as m
import synth
from synth.device import device_layer
from moe_helpers import assert_close, gpu_out_f64, oracle_out, oracle_weights

pytestmark = pytest.mark.gpu

DET = m.FLAG_DETERMINISTIC
LAYERS = [
    (synth.Spec("streams_bf16", T=300, H=256, I=192, E=12, k=3, act="bf16", weight="bf16", seed=31),
     m.FLAG_FORCE_GROUPED | DET),
    (synth.Spec("streams_decode", T=8, H=256, I=256, E=12, k=2, act="bf16", weight="bf16", seed=32),
     m.FLAG_FORCE_DECODE | DET),
    (synth.Spec("streams_fp8", T=200, H=256, I=256, E=8, k=2, act="bf16", weight="fp8", scale="f32", seed=33),
     DET),
    (synth.Spec("streams_fp4", T=130, H=512, I=256, E=8, k=2, act="bf16", weight="fp4", scale="ue8m0", seed=34),
     DET),
]


class _Call:
    """One layer staged on the GPU with its own workspace and output."""

    def __init__(self, spec, flags):
        self.spec, self.flags = spec, flags
        self.D = device_layer(spec)
        self.kw = {}
        if "w_gate_up_scale" in self.D:
            self.kw = dict(w_gate_up_scale=self.D["w_gate_up_scale"], w_down_scale=self.D["w_down_scale"])
        D = self.D
        prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], D.get("w_gate_up_scale"), flags)
        self.ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device="cuda")
        self.out = torch.empty_like(D["x"])

    def launch(self):
        D = self.D
        m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], out=self.out, flags=self.flags,
                          workspace=self.ws, **self.kw)

    def scrub(self):
        self.out.fill_(0.0)
        self.ws.fill_(0xA5)


def _bits(t):
    return t.view(torch.int16).clone()


@pytest.fixture(scope="module")
def calls():
    cs = [_Call(spec, flags) for spec, flags in LAYERS]
    serial = []
    for c in cs:
        c.scrub()
        c.launch()
        torch.cuda.synchronize()
        serial.append(_bits(c.out))
        if c.spec.weight == "bf16":   # (e4m3 / FP4 parity, with its requantisation check: test_gpu_forward)
            ref = oracle_out(c.spec, c.D["x_host"], c.D["idx_host"], c.D["w_host"], oracle_weights(c.spec))
            assert_close(gpu_out_f64(c.out), ref, "bf16", f"{c.spec.name}: serial")
    return cs, serial


def test_forwards_on_separate_streams(calls):
    cs, serial = calls
    streams = [torch.cuda.Stream() for _ in cs]
    for rep in range(3):
        for c in cs:
            c.scrub()
        cur = torch.cuda.current_stream()
        for s in streams:
            s.wait_stream(cur)
        for c, s in zip(cs, streams):       # all launched before any completes
            with torch.cuda.stream(s):
                c.launch()
        for s in streams:
            cur.wait_stream(s)
        torch.cuda.synchronize()
        for c, ref in zip(cs, serial):
            assert torch.equal(_bits(c.out), ref), f"{c.spec.name}: concurrent run {rep} differs from the serial one"


def test_forwards_from_separate_threads(calls):
    cs, serial = calls
    streams = [torch.cuda.Stream() for _ in cs]
    for c in cs:
        c.scrub()
    cur = torch.cuda.current_stream()
    for s in streams:
        s.wait_stream(cur)
    torch.cuda.synchronize()
    start = threading.Barrier(len(cs), timeout=60)
    errors = []

    def work(c, s):
        try:
            start.wait()
            with torch.cuda.stream(s):
                for _ in range(2):
                    c.launch()
            s.synchronize()
        except Exception as exc:   # reported on the main thread
            errors.append(f"{c.spec.name}: {exc!r}")

    threads = [threading.Thread(target=work, args=(c, s), daemon=True) for c, s in zip(cs, streams)]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a forward thread did not finish"
    torch.cuda.synchronize()
    assert not errors, errors
    for c, ref in zip(cs, serial):
        assert torch.equal(_bits(c.out), ref), f"{c.spec.name}: threaded run differs from the serial one"
