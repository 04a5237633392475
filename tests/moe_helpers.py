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


# Accumulation bound of the block-scaled 16x16x128 MFMA (gfx950) that the e4m3 and e2m1
# kernels use for every 128-long block of a dot product: |result - exact block sum| <= 2^-10
# times the largest |product| in the block.  It is a property of the instruction, checked
# directly against exact sums on random, wide-exponent and cancelling operands by
# tests/test_gpu_mfma_bound.py (largest ratio seen there 2^-10.7).
MFMA_BLOCK_BOUND = 2.0 ** -10
# largest |gate'(z)| over all z: silu 1.0998, exact gelu 1.1289, relu 1
GATE_SLOPE = {"silu": 1.1, "gelu": 1.13, "relu": 1.0}
U32 = 2.0 ** -24          # float32 unit roundoff


def _abs_block_max(m: np.ndarray) -> np.ndarray:
    """[R, K] -> [R, K/128]: largest |entry| of each 128-column block."""
    R, K = m.shape
    return np.abs(m).reshape(R, K // 128, 128).max(axis=2)


def swiglu_error_bound(xs: np.ndarray, wgu: np.ndarray, gu: np.ndarray, I: int, gate: str) -> np.ndarray:
    """A-priori bound [n, I] on |GPU float32 SwiGLU value - the exact value rounded to fp32|.

    xs: the rows' dequantised e4m3 hidden states [n, H] (fp64); wgu: the expert's dequantised
    W_gate_up [2I, H]; gu: the exact pre-activations [n, 2I].  Per gate/up column, over the
    H / 128 blocks: the MFMA bound per block (MFMA_BLOCK_BOUND * max|x| * max|w| of the
    block, an upper bound of its largest product), plus the float32 folds (each block's
    result is rounded and added into the running sum: at most 2 u sum_k |x_k w_k| in all,
    u = 2^-24, times the number of blocks).  Through a = gate(g) * u: slope * dg * (|u| + du)
    + |gate(g)| du, plus 8 float32 roundings of the gate and the product.
    """
    nb = xs.shape[1] // 128
    blk = _abs_block_max(xs) @ _abs_block_max(wgu).T                  # [n, 2I]
    sabs = np.abs(xs) @ np.abs(wgu).T                                  # [n, 2I]
    d = MFMA_BLOCK_BOUND * blk + 2.0 * U32 * (nb + 1) * sabs
    from oracle.moe import GATES
    g, u = gu[:, :I], gu[:, I:]
    dg, du = d[:, :I], d[:, I:]
    gv = np.abs(GATES[gate](g))
    L = GATE_SLOPE[gate]
    return L * dg * (np.abs(u) + du) + (gv + L * dg) * du + 8 * U32 * (gv + L * dg) * (np.abs(u) + du)


def _e4m3_grid():
    from oracle.numerics import e4m3_value_table
    tab = e4m3_value_table()
    return np.unique(tab[np.isfinite(tab) & (tab >= 0)])              # 0 .. 448 ascending


def admissible_codes(v_lo: np.ndarray, v_hi: np.ndarray, code: np.ndarray) -> np.ndarray:
    """True where e4m3 `code` is the round-to-nearest-even result of some value in
    [v_lo, v_hi] (values already divided by the scale; beyond 448 the rounding saturates).

    The values rounding to a nonzero code of magnitude g_i lie between the midpoints to its
    neighbours on the e4m3 grid (closed: a tie may go either way here), with the sign of
    the code; +0 and -0 take [-g_1 / 2, g_1 / 2].
    """
    from oracle.numerics import e4m3_decode
    grid = _e4m3_grid()
    val = e4m3_decode(code).reshape(code.shape)
    mag = np.abs(val)
    i = np.searchsorted(grid, mag)                                     # exact grid index
    below = 0.5 * (grid[np.maximum(i - 1, 0)] + mag)
    above = np.where(i < len(grid) - 1, 0.5 * (grid[np.minimum(i + 1, len(grid) - 1)] + mag), np.inf)
    lo = np.where(val < 0, -above, below)
    hi = np.where(val < 0, -below, above)
    lo = np.where(mag == 0, -0.5 * grid[1], lo)
    hi = np.where(mag == 0, 0.5 * grid[1], hi)
    return (v_hi >= lo) & (v_lo <= hi)


def read_requantised(ws: torch.Tensor, plan: str, A: int, I: int):
    """The forward's e4m3 SwiGLU codes [A, I] and scales [A, I/128] (expert-sorted order),
    read back from its workspace at the offsets moe_plan_describe reports."""
    import re
    oq = int(re.search(r"act_codes_offset=(\d+)", plan).group(1))
    os_ = int(re.search(r"act_scales_offset=(\d+)", plan).group(1))
    host = ws.cpu().numpy()
    codes = host[oq: oq + A * I].reshape(A, I)
    scales = host[os_: os_ + 4 * A * (I // 128)].view(np.float32).reshape(A, I // 128)
    return codes, scales


def check_requantised(spec, x, idx, w, weights: ExpertWeights, capture: dict, codes_g, scales_g,
                      gate="silu", tokens=None):
    """Compare what is unique in the requantised SwiGLU rows, validate the rest, and bound
    what the valid alternatives the GPU took do to the output.

    The e4m3 codes of `a` are decided on float32 values: the oracle rounds the exact a to
    float32, the GPU's float32 a carries its accumulation error.  With the a-priori bound da
    of that error (swiglu_error_bound, from the inputs alone):
      * every GPU scale must lie in [amax_lo, amax_hi] / 448 (rounded), amax_lo/hi the group
        maximum of |a| -/+ da;
      * every GPU code must be the rounding of some value in [(a - da) / s, (a + da) / s] with
        the GPU's own scale s (a one-step flip next to a rounding midpoint, or the same code).
    Codes and scales are compared with the oracle's and every difference must pass both.
    Returns (allowance [n, H], stats): allowance = sum over slots of w * |a_gpu - a_oracle|
    (dequantised, per element) @ |W_down|^T, the exact effect bound of the GPU's valid
    alternatives on its token's outputs; the oracle's output itself is unchanged.
    """
    from oracle.moe import _prepare_x, route
    from oracle.numerics import e4m3_decode

    idx = np.asarray(idx)
    T, k = idx.shape
    rows = np.arange(T) if tokens is None else np.asarray(tokens)
    pos = {int(t): n for n, t in enumerate(rows)}
    _, _, _, inv = route(idx, spec.E)
    xs = _prepare_x(np.asarray(x)[rows], spec.act, True)
    ws = np.asarray(w, dtype=np.float32)[rows].astype(np.float64)
    I, H = spec.I, spec.H
    allow = np.zeros((len(rows), H))
    st = dict(elements=0, codes_differ=0, groups=0, scales_differ=0, bad_codes=0, bad_scales=0, max_flip_steps=0)
    sub = idx[rows]
    for e in np.unique(sub):
        rr, jj = np.nonzero(sub == e)
        keys = [(int(rows[r]), int(j)) for r, j in zip(rr, jj)]
        gu = np.stack([capture[kk][0] for kk in keys])
        a32 = np.stack([capture[kk][1] for kk in keys]).astype(np.float64)
        co = np.stack([capture[kk][2] for kk in keys])
        so = np.stack([capture[kk][3] for kk in keys]).astype(np.float64)
        p = inv[np.array([t * k + j for t, j in keys])]
        cg, sg = codes_g[p], scales_g[p].astype(np.float64)
        wgu = weights.gate_up_f64(int(e))
        da = swiglu_error_bound(xs[rr], wgu, gu, I, gate)
        n = len(keys)
        # scales: amax of |a| within +- da per group
        aa = np.abs(a32).reshape(n, I // 128, 128)
        dd = da.reshape(n, I // 128, 128)
        amax_lo = np.maximum(aa - dd, 0).max(axis=2)
        amax_hi = (aa + dd).max(axis=2)
        s_lo = np.where(amax_lo > 0, amax_lo / 448.0, np.minimum(1.0, amax_hi / 448.0)) * (1 - U32)
        s_hi = np.where(amax_hi > 0, np.maximum(amax_hi / 448.0, (amax_lo == 0) * 1.0), 1.0) * (1 + U32)
        ok_s = (sg >= s_lo) & (sg <= s_hi)
        # codes, with the GPU's own scale of each element
        sge = np.repeat(sg, 128, axis=1)
        ok_c = admissible_codes((a32 - da) / sge, (a32 + da) / sge, cg)
        st["elements"] += cg.size
        st["groups"] += sg.size
        vg = e4m3_decode(cg).reshape(cg.shape)
        vo = e4m3_decode(co).reshape(co.shape)
        st["codes_differ"] += int((vg != vo).sum())
        st["scales_differ"] += int((sg != so).sum())
        st["bad_codes"] += int((~ok_c).sum())
        st["bad_scales"] += int((~ok_s).sum())
        ag = vg * sge
        ao = vo * np.repeat(so, 128, axis=1)
        delta = np.abs(ag - ao)
        if (vg != vo).any():
            grid = _e4m3_grid()
            gi, oi = np.searchsorted(grid, np.abs(vg)), np.searchsorted(grid, np.abs(vo))
            steps = np.where((vg < 0) == (vo < 0), np.abs(gi - oi), gi + oi)
            st["max_flip_steps"] = max(st["max_flip_steps"], int(steps[vg != vo].max()))
        if delta.any():
            wd = weights.down_f64(int(e))
            contrib = (delta @ np.abs(wd).T) * ws[rr, jj][:, None]
            np.add.at(allow, rr, contrib)
    return allow, st


def err_ratio(got: np.ndarray, ref: np.ndarray, act: str, extra=None) -> float:
    atol, rtol = TOL[act]
    tol = atol + rtol * np.abs(ref)
    if extra is not None:
        tol = tol + extra
    r = np.abs(got - ref) / tol
    if not np.isfinite(got).all():
        return float("inf")
    return float(r.max()) if r.size else 0.0


def assert_close(got, ref, act, what="", extra=None):
    r = err_ratio(got, ref, act, extra)
    assert r <= 1.0, f"{what}: max |gpu-oracle|/tol = {r:.4g}"
    return r


def cover_tokens(idx: np.ndarray, E: int, n_random: int = 8, seed: int = 123) -> np.ndarray:
    """Tokens whose slots reach every active expert (a greedy set cover: each step takes the
    token that reaches the most experts not yet reached, ties to the lower token), plus the
    first and last token and n_random others; sorted and unique.

    Every expert that received a slot then has at least one of its output rows compared,
    the rare experts with one-row groups and ragged M tiles included (the introduction of
    the page: each chosen expert's projection enters its token's sum).
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    if T == 0:
        return np.zeros(0, dtype=np.int64)
    first = np.ones((T, k), dtype=bool)            # first occurrence of an id within its row
    for j in range(k):
        for jj in range(j):
            first[:, j] &= idx[:, jj] != idx[:, j]
    left = np.zeros(E, dtype=bool)
    left[idx.ravel()] = True
    chosen = []
    while left.any():
        t = int(np.argmax((left[idx] & first).sum(axis=1)))
        chosen.append(t)
        left[idx[t]] = False
    rng = np.random.default_rng(seed)
    extra = rng.choice(T, size=min(n_random, T), replace=False)
    return np.unique(np.concatenate([[0, T - 1], chosen, extra]).astype(np.int64))


def covered_experts(idx: np.ndarray, tokens) -> np.ndarray:
    return np.unique(np.asarray(idx)[np.asarray(tokens)])


def oracle_out_threaded(spec, x, idx, w, weights, tokens, threads: int = 16, gate="silu", capture=None):
    """oracle_out over `tokens`, the tokens split into `threads` chunks evaluated at once
    (each chunk is an independent call of the oracle; BLAS runs one thread per chunk).
    capture: optional dict for the oracle's SwiGLU intermediates (fp8 / fp4 layers)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits

    tokens = np.asarray(tokens)
    chunks = [c for c in np.array_split(tokens, max(1, min(threads, len(tokens)))) if len(c)]
    caps = [dict() if capture is not None else None for _ in chunks]

    def one(i):
        _, out = forward(x, idx, w, weights, act=spec.act, E=spec.E, mode="fast", tokens=chunks[i], gate=gate,
                         capture=caps[i])
        return out_as_f64(out, spec.act)

    with threadpool_limits(1), ThreadPoolExecutor(max_workers=len(chunks)) as ex:
        parts = list(ex.map(one, range(len(chunks))))
    if capture is not None:
        for c in caps:
            capture.update(c)
    return np.concatenate(parts, axis=0)
