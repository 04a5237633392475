#!/usr/bin/env python3
"""Benchmark of the routed top-k experts forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

One step is one full forward -- routing bookkeeping, (fp8/fp4: activation
quantisation,) gate/up GEMM + SwiGLU, down GEMM + weighted combine, finalize --
over one batch of seeded synthetic inputs already resident in HBM.  The default
workload is the DeepSeek-V3-shaped bf16 prefill layer (T=8192, H=7168, I=2048,
E=256, top-8, Zipf-skewed routing), the largest layer of the set that fits one GPU.
Each timed forward is bracketed by HIP events on the library's stream.  Between forwards
(outside the events) 1 GiB of scratch is written and a second 1 GiB buffer is read, so
that every step starts with the 4 MB L2s and the 256 MB Infinity Cache cold and clean
(a write alone would leave dirty lines for the step to write back).  Prints one JSON line:
tokens/s from the median step, the step's median/min/max, the dominant kernel's
roofline figures (its launches bracketed by HIP events in every timed step), and
the CPU oracle timed on bounded samples (expert-major fp64 BLAS over all host
cores, and the per-token loop).
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0                                            # MI355X HBM3E, GB/s
# dense, TFLOP/s; the fp4 experts multiply e4m3 activations by e2m1 weights, a mixed-format
# MFMA that issues at the fp8 rate (the 10.1 PFLOP/s fp4 figure needs 4-bit operands on both
# sides), so they are priced at the fp8 peak
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "fp4": 5000.0, "f32": 157.3}

WORKLOADS = {
    "tiny_fp32": "tiny fp32 MoE layer: T=32 H=128 I=256 E=8 top-2, renormalised",
    "qwen_prefill_bf16": "Qwen1.5-MoE-A2.7B-shaped bf16 prefill: T=4096 H=2048 I=1408 E=60 top-4",
    "qwen_decode_bf16": "Qwen1.5-MoE-A2.7B-shaped bf16 decode: T=16 H=2048 I=1408 E=60 top-4",
    "dsv3_prefill_bf16": "DeepSeek-V3-shaped bf16 prefill, Zipf-skewed routing: T=8192 H=7168 I=2048 E=256 top-8",
    "dsv3_fp8_f32scale": "DeepSeek-V3-shaped fp8-e4m3 experts, 128x128 float32 block scales: T=4096 H=7168 I=2048 E=256 top-8",
    "dsv3_fp8_ue8m0": "DeepSeek-V3-shaped fp8-e4m3 experts, 128x128 UE8M0 block scales: T=4096 H=7168 I=2048 E=256 top-8",
    "dsv3_fp4_ue8m0": "DeepSeek-V3-shaped fp4-e2m1 experts (two per byte), 1x32 UE8M0 scales: T=4096 H=7168 I=2048 E=256 top-8",
}


# hipEventDisableSystemFence: the events only time kernels, so recording one skips the
# system-scope fence (a cache writeback and invalidation) that would slow the work after it
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class HipEvents:
    """hipEvent_t handles (timing only) from the HIP runtime already loaded by torch."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            ev = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(ev), HIP_EVENT_DISABLE_SYSTEM_FENCE) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            out.append(ev.value)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        self.hip.hipEventSynchronize(ctypes.c_void_p(b))
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            self.hip.hipGetLastError()  # an event of a stage the path does not run: clear the error
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(ctypes.c_void_p(e))


def router_step(spec, dev, iters=50):
    """The router step + bookkeeping (moe_route_logits) on seeded float32 logits of this layer's
    [T, E] shape: GPU time per call, from two events around `iters` back-to-back calls on
    torch's stream (which the library uses) with every buffer allocated beforehand, and the
    bytes it must move."""
    import ctypes as C
    import torch
    import mixture_experts_routed_topk_amd as m
    g = torch.Generator().manual_seed(0)
    T, E, k = spec.T, spec.E, spec.k
    lg = torch.randn((T, E), generator=g, dtype=torch.float32).to(dev)
    prob = m.Problem(T, 128, 128, E, k, m.BF16, m.BF16, m.SCALE_NONE, 0)
    ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device=dev)
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    inv = torch.empty(T * k, dtype=torch.int32, device=dev)
    stream = C.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    args = [C.byref(prob), C.c_void_p(lg.data_ptr()), int(spec.renorm)] + \
        [C.c_void_p(t.data_ptr()) for t in (idx, w, cnt, off, perm, inv, ws)] + [ws.numel(), stream]
    call = m.lib().moe_route_logits
    for _ in range(3):
        if call(*args) != 0:
            raise RuntimeError("moe_route_logits failed")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(iters):
        call(*args)
    b.record()
    b.synchronize()
    ms = a.elapsed_time(b) / iters
    byts = T * E * 4 + T * k * 8 + spec.A * 8 + E * 8
    return {"what": "router (softmax, top-k, renorm) + routing bookkeeping from float32 logits",
            "ms": ms, "calls": iters, "bytes": byts, "GB/s": byts / (ms * 1e-3) / 1e9,
            "bound": "launch latency (a few MB at most)"}


def algorithmic(spec, active_count, stage):
    """(flops, bytes) the method must do/move in one launch of a stage.

    Bytes are the active experts' weights and weight scales, the layer's input rows (gate_up:
    x, or its e4m3 codes and row scales on fp8 and fp4 layers) and its output rows (down:
    out).  The SwiGLU rows `a` that pass from gate_up to down, and the combine's accumulator or
    slot rows, belong to this two-kernel design rather than to the method: they are counted
    apart (`intermediate_bytes`), not here."""
    A, H, I = spec.A, spec.H, spec.I
    wb = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[spec.weight]
    xb = {"f32": 4, "bf16": 2}[spec.act]
    q = spec.weight in ("fp8", "fp4")                               # e4m3 input rows
    # weight-scale bytes per weight element: 128x128 blocks (fp8) or 1x32 UE8M0 (fp4)
    sb = 0.0
    if spec.weight == "fp8":
        sb = (4 if spec.scale == "f32" else 1) / (128 * 128)
    elif spec.weight == "fp4":
        sb = 1 / 32
    if stage == "gate_up":
        flops = 4.0 * A * H * I
        byts = active_count * 2 * I * H * (wb + sb)
        byts += spec.T * H * (1 if q else xb)
        if q:
            byts += spec.T * (H // 128) * 4
    elif stage == "down":
        flops = 2.0 * A * H * I
        byts = active_count * H * I * (wb + sb) + spec.T * H * xb
    else:
        raise ValueError(stage)
    return flops, float(byts)


def intermediate_bytes(spec, stage):
    """Bytes of the SwiGLU rows `a` one launch of a stage writes (gate_up) or reads (down):
    bf16 or float32 rows, or e4m3 codes with one float32 scale per 128 columns."""
    A, I = spec.A, spec.I
    if spec.weight in ("fp8", "fp4"):
        return float(A * I + A * (I // 128) * 4)
    return float(A * I * {"f32": 4, "bf16": 2}[spec.weight])


def layer_totals(spec, active_count):
    """Whole-layer algorithmic flops and bytes (active expert weights + x + out + routing)."""
    wb = {"f32": 4, "bf16": 2, "fp8": 1, "fp4": 0.5}[spec.weight]
    xb = {"f32": 4, "bf16": 2}[spec.act]
    flops = 6.0 * spec.A * spec.H * spec.I
    byts = active_count * 3 * spec.I * spec.H * wb + 2 * spec.T * spec.H * xb + 8 * spec.A
    if spec.weight == "fp8":
        sb = 4 if spec.scale == "f32" else 1
        byts += active_count * 3 * (spec.I // 128) * (spec.H // 128) * sb
    elif spec.weight == "fp4":
        byts += active_count * 3 * spec.I * spec.H / 32
    return flops, float(byts)


KERNEL_SOURCES = {   # (path, weight dtype, stage) -> kernel source files, for the traffic record
    ("grouped", "bf16", "gate_up"): ["grouped_bf16.hip"],
    ("grouped", "bf16", "down"): ["grouped_bf16.hip"],
    ("grouped", "fp8", "gate_up"): ["grouped_fp8.hip"],
    ("grouped", "fp8", "down"): ["grouped_fp8.hip"],
    ("grouped", "fp4", "gate_up"): ["grouped_fp4.hip"],
    ("grouped", "fp4", "down"): ["grouped_fp4.hip"],
    ("grouped", "f32", "gate_up"): ["grouped_f32.hip"],
    ("grouped", "f32", "down"): ["grouped_f32.hip"],
    ("decode", "bf16", "gate_up"): ["decode.hip"],
    ("decode", "bf16", "down"): ["decode.hip"],
}


def _code_only(text: str) -> str:
    """C++ source without comments and blank lines (a comment edit does not change a kernel)."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return "\n".join(ln for ln in lines if ln.strip())


def kernel_digest(path: str, weight: str, stage: str) -> tuple[str, str]:
    """(name, sha256) of the dominant kernel's code (its file + the shared device headers,
    comments left out)."""
    import hashlib
    files = KERNEL_SOURCES[(path, weight, stage)]
    csrc = os.path.join(ROOT, "mixture_experts_routed_topk_amd", "csrc")
    h = hashlib.sha256()
    for f in files + ["device_common.h", "internal.h"] + (["act_quant_epilogue.h"] if weight in ("fp8", "fp4") else []):
        with open(os.path.join(csrc, f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return files[0].rsplit(".", 1)[0], h.hexdigest()


def recorded_traffic(kernel: str, stage: str, config: str, digest: str):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE summary of this kernel
    and workload, or None when there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{stage}_{config}_hbm_traffic.md")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if line.startswith("    ") and ":" in line:
                k, v = line.strip().split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("kernel_source_sha256") != digest or "traffic_bytes_per_launch" not in rec:
        return None
    return float(rec["traffic_bytes_per_launch"])


def copy_calibration(nbytes: int = 256 << 20, reps: int = 3):
    """A plain device copy of a known size, run under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
    to scale those counters to bytes: each of the `reps` launches reads and writes nbytes."""
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(reps):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read_per_launch": nbytes, "bytes_written_per_launch": nbytes,
                                           "launches": reps}}), flush=True)


def _blas_info():
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        return (info[0].get("internal_api", "?"), int(max(i.get("num_threads", 1) for i in info))) if info else ("?", 1)
    except Exception:  # pragma: no cover
        return "?", 1


def cpu_baseline(spec, D, seconds: float):
    """The fp64 oracle timed on bounded samples of the same layer, weight generation excluded.

    fast: the oracle's expert-major mode (fp64 BLAS over all host cores) on the first n tokens,
    n doubled from 8 while the run stays short; the largest sample is reported.
    literal: the per-token loop over the k chosen experts on the first tokens, about a third
    of the time budget.
    """
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor
    import synth
    from oracle.moe import ExpertWeights, forward

    cache = {}

    def gen(e):
        return e, synth.expert_gate_up(spec, e), synth.expert_down(spec, e)

    def prefetch(experts):
        todo = [int(e) for e in experts if int(e) not in cache]
        with ThreadPoolExecutor(max_workers=16) as ex:
            for e, g, d in ex.map(gen, todo):
                cache[e] = (g, d)

    if spec.weight in ("fp8", "fp4"):
        W = ExpertWeights(spec.weight, lambda e: cache[e][0][0], lambda e: cache[e][1][0], spec.scale,
                          lambda e: cache[e][0][1], lambda e: cache[e][1][1])
    else:
        W = ExpertWeights(spec.weight, lambda e: cache[e][0], lambda e: cache[e][1])
    vendor, threads = _blas_info()
    idx = D["idx_host"]
    # fast mode on growing token prefixes: most of a small sample's time is converting the
    # experts it touches, so the next sample's time is extrapolated linearly in n
    budget = 2 * seconds / 3
    n, hist, spent = min(spec.T, 256), [], 0.0
    while True:
        toks = np.arange(n)
        prefetch(np.unique(idx[toks]))
        t0 = time.perf_counter()
        forward(D["x_host"], idx, D["w_host"], W, act=spec.act, E=spec.E, mode="fast", tokens=toks)
        dt = time.perf_counter() - t0
        spent += dt
        hist.append((n, dt))
        if n == spec.T:
            break
        nxt = min(2 * n, spec.T)
        if len(hist) > 1:
            (n0, d0), (n1, d1) = hist[-2], hist[-1]
            pred = d1 + max(d1 - d0, 0.0) * (nxt - n1) / (n1 - n0)
        else:
            pred = 2 * dt
        if spent + pred > budget:
            break
        n = nxt
    fast = hist[-1]
    # literal mode on the first tokens, one BLAS thread
    from threadpoolctl import threadpool_limits
    t_lit, n_lit, t = 0.0, 0, 0
    with threadpool_limits(1):
        while t_lit < seconds / 3 and t < spec.T:
            prefetch(np.unique(idx[t]))
            t0 = time.perf_counter()
            forward(D["x_host"], idx, D["w_host"], W, act=spec.act, E=spec.E, mode="literal", tokens=[t])
            t_lit += time.perf_counter() - t0
            n_lit += 1
            t += 1
    n_f, t_f = fast
    return {"value": n_f / t_f, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_f} tokens of the same layer, fp64 oracle in its expert-major mode ({vendor} BLAS, "
                      f"{threads} threads), {t_f:.1f} s; weight generation not timed",
            "blas": vendor, "host_cpus": len(os.sched_getaffinity(0)),
            "literal": {"value": n_lit / t_lit, "unit": "tokens/s", "cores": 1,
                        "sample": f"first {n_lit} tokens, per-token fp64 loop over the k chosen experts, "
                                  f"{t_lit:.1f} s"}}


def machine_peaks(dev, reps: int = 5):
    """What this machine delivers, as context for the published peaks: HBM read bandwidth (a float32
    sum over 2 GiB), copy bandwidth (2 GiB read + 2 GiB written) and a dense 8192^3 bf16 GEMM
    (torch.matmul, hipBLASLt); each the median of `reps` runs timed with events.  None of them
    is part of the experts forward."""
    import torch
    n = 2 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    a = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)
    b = torch.randn((8192, 8192), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        fn()
        out = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            out.append(e0.elapsed_time(e1))
        return sorted(out)[len(out) // 2]

    ms_sum = timed(lambda: torch.sum(x))
    ms_copy = timed(lambda: y.copy_(x))
    ms_mm = timed(lambda: torch.matmul(a, b))
    del x, y, a, b
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9   # noqa: E731
    return {"hbm_read_GBs": gbs(n, ms_sum), "hbm_copy_GBs": gbs(2 * n, ms_copy),
            "bf16_gemm_TFLOPs": 2.0 * 8192 ** 3 / (ms_mm * 1e-3) / 1e12,
            "how": "median of 5: torch.sum over 2 GiB float32 (read), 2 GiB device copy (read + write), "
                   "torch.matmul 8192^3 bf16 (hipBLASLt)"}


def _stats(v):
    v = sorted(v)
    return {"median": v[len(v) // 2], "min": v[0], "max": v[-1], "mean": sum(v) / len(v), "n": len(v)}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # defaults: 100 untimed steps take the GPU to its steady clock (on the Qwen prefill layer
    # the first 50 steps after 10 warm-up steps ran 9% slower than every later 50)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--config", default="dsv3_prefill_bf16", choices=sorted(WORKLOADS))
    ap.add_argument("--flags", type=int, default=0, help="MOE_FLAG_* bits passed to the forward")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--flush-mib", type=int, default=1024,
                    help="MiB of scratch touched between timed steps (outside the step events)")
    ap.add_argument("--flush", choices=("write+read", "write", "read", "none"), default="write+read",
                    help="how scratch evicts the caches between steps: written and then a second buffer "
                         "read (the caches are cold and clean when the step starts), written only (dirty "
                         "lines the step has to write back), read only, or not at all")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 256 MiB device copy (counter calibration for the traffic figure)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this experts forward is a single-GPU library "
              "(no sharding, no collectives); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration()
        return

    import torch
    import mixture_experts_routed_topk_amd as m
    import synth
    from synth.device import device_layer

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    spec = synth.spec_for(args.config)
    D = device_layer(spec, dev)
    n_active = len(D["active"])
    kw = {}
    if spec.weight in ("fp8", "fp4"):
        kw = dict(w_gate_up_scale=D["w_gate_up_scale"], w_down_scale=D["w_down_scale"])
    prob = m.problem_for(D["x"], D["idx"], D["w_gate_up"], D["w_down"], kw.get("w_gate_up_scale"),
                         args.flags)
    ws = torch.empty(m.workspace_size(prob), dtype=torch.uint8, device=dev)
    out = torch.empty_like(D["x"])
    plan = m.plan_describe(prob)

    def step():
        m.experts_forward(D["x"], D["idx"], D["w"], D["w_gate_up"], D["w_down"], out=out,
                          flags=args.flags, workspace=ws, **kw)

    hev = HipEvents()
    nst = len(m.STAGES)
    # warm-up, with every stage bracketed by events to find the dominant kernel
    warm = max(args.warmup, 1)
    wev = hev.create(2 * nst * warm)
    for i in range(warm):
        m.set_stage_events(wev[2 * nst * i: 2 * nst * (i + 1)])
        step()
    m.set_stage_events(None)
    torch.cuda.synchronize()
    stage_ms = {}
    for s, name in enumerate(m.STAGES):
        vals = []
        for i in range(warm):
            a, b = wev[2 * nst * i + 2 * s], wev[2 * nst * i + 2 * s + 1]
            try:
                vals.append(hev.elapsed_ms(a, b))
            except RuntimeError:
                vals = []
                break
        if vals:
            stage_ms[name] = sorted(vals)[len(vals) // 2]
    hev.destroy(wev)
    dominant = max(("gate_up", "down"), key=lambda n: stage_ms.get(n, 0.0))
    dom = m.STAGES.index(dominant)

    # timed region: every forward bracketed by step events, the dominant kernel by stage
    # events; a scratch write between forwards (outside the step events) evicts the cache
    flush = torch.zeros(max(args.flush_mib, 1) << 20, dtype=torch.uint8, device=dev)
    flush_r = torch.zeros_like(flush) if args.flush == "write+read" else flush
    tev = hev.create(2 * args.steps)
    sev = hev.create(2 * args.steps)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rec = hev.hip.hipEventRecord
    rec.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    handles = [None] * (2 * nst)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        if args.flush in ("write", "write+read"):
            flush.fill_(i & 0xFF)
        if args.flush in ("read", "write+read"):
            torch.amax(flush_r)
        handles[2 * dom], handles[2 * dom + 1] = tev[2 * i], tev[2 * i + 1]
        m.set_stage_events(handles)
        rec(ctypes.c_void_p(sev[2 * i]), stream)
        step()
        rec(ctypes.c_void_p(sev[2 * i + 1]), stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    m.set_stage_events(None)
    kern_ms = [hev.elapsed_ms(tev[2 * i], tev[2 * i + 1]) for i in range(args.steps)]
    step_ms = [hev.elapsed_ms(sev[2 * i], sev[2 * i + 1]) for i in range(args.steps)]
    hev.destroy(tev)
    hev.destroy(sev)
    del flush, flush_r

    step_st, kern_st = _stats(step_ms), _stats(kern_ms)
    ms_per_step = step_st["median"]
    tokens_per_s = spec.T / (ms_per_step * 1e-3)
    kavg = kern_st["mean"]
    flops, byts = algorithmic(spec, n_active, dominant)
    peak_f = PEAK_TFLOPS[spec.weight]
    t_mfma = flops / (peak_f * 1e12)
    t_hbm = byts / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        roof = {"bound": "mfma", "achieved": flops / (kavg * 1e-3) / 1e12, "peak": peak_f, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": byts / (kavg * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    kname, digest = kernel_digest(plan.split()[0].split("=")[1], spec.weight, dominant)
    roof["traffic"] = recorded_traffic(kname, dominant, args.config, digest)
    roof.update({"kernel": f"{kname}:{dominant}", "kernel_source_sha256": digest, "avg_ms": kavg,
                 "median_ms": kern_st["median"], "min_ms": kern_st["min"], "max_ms": kern_st["max"],
                 "launches": len(kern_ms),
                 "algorithmic_flops": flops, "algorithmic_bytes": byts,
                 "intermediate_bytes": intermediate_bytes(spec, dominant),
                 "mfma_frac": flops / (kavg * 1e-3) / 1e12 / peak_f,
                 "hbm_frac": byts / (kavg * 1e-3) / 1e9 / PEAK_HBM_GBS})
    lf, lb = layer_totals(spec, n_active)
    sec = ms_per_step * 1e-3
    res = {
        "metric": "MoE-layer tokens/s + achieved TFLOP/s (prefill) / HBM GB/s (decode)",
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "step_ms": {k: step_st[k] for k in ("median", "min", "max", "mean")},
        "ms_per_step_wall": (t1 - t0) * 1e3 / args.steps,
        "cache_flush": {"mib": args.flush_mib if args.flush != "none" else 0, "mode": args.flush},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.weight,
        "data": "synthetic (seeded random weights and routing; no checkpoint)",
        "config": {"workload": WORKLOADS[args.config], "name": args.config, "T": spec.T, "H": spec.H,
                   "I": spec.I, "E": spec.E, "k": spec.k, "active_experts": n_active,
                   "routing": spec.routing, "scales": spec.scale, "plan": plan, "flags": args.flags},
        "tflops": lf / sec / 1e12,
        "hbm_gbps": lb / sec / 1e9,
        "layer_mfma_frac": lf / sec / 1e12 / peak_f,
        "layer_hbm_frac": lb / sec / 1e9 / PEAK_HBM_GBS,
        "stages_ms": stage_ms,
        "roofline": roof,
    }
    res["router_step"] = router_step(spec, dev)
    mp = machine_peaks(dev)
    # context only: torch's read and copy kernels stream below what the decode kernels reach, so
    # the measured-peak fraction is given against the dense bf16 GEMM only
    meas = mp["bf16_gemm_TFLOPs"] if roof["bound"] == "mfma" and spec.weight == "bf16" else None
    res["machine"] = mp
    roof["frac_of_measured"] = roof["achieved"] / meas if meas else None
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(spec, D, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
