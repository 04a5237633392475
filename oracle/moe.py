"""fp64 CPU oracle of the routed top-k experts forward.

Definition (Experts backends page, introduction; the expert is the gated MLP of
the "deepgemm_megamoe" row and the "SonicMoE" section, with silu -> SwiGLU):

    out[t, :] = sum_{j < k} w[t, j] * MLP_{idx[t, j]}(x[t, :])
    MLP_e(v)  = W_down[e] @ ( silu(W_gate[e] @ v) * (W_up[e] @ v) )
    silu(z)   = z / (1 + exp(-z))

W_gate_up[e] is [2I, H] with the gate projection in rows [0, I) and the up
projection in rows [I, 2I); W_down[e] is [H, I]; y = W @ v (rows are outputs).
Every slot (t, j) contributes on its own, so a repeated expert id within one token
counts twice.  An expert id outside [0, E) is an error.

Everything is evaluated in fp64 from the exactly converted inputs and rounded once
(round-to-nearest-even) to the output type.

fp8 experts ("FP8 and FP4 quantized experts" section and note): weights arrive as
e4m3 codes with one float32 or UE8M0 scale per 128x128 block, and dequantise to
code * scale.  Activations get dynamic per-row scales -- one per 128 consecutive
channels of a row -- computed here as
    amax = max |v| over the group (fp32),  s = amax / 448 (fp32, RN; 1 if amax = 0),
    q    = e4m3(v / s)  (fp32 division, then RNE to e4m3 with saturation).
The quantisation points are part of the result: the hidden states are quantised
before the gate/up projection, and the SwiGLU output, rounded to fp32, is
quantised before the down projection.

FP4 experts (same section: weights packed two e2m1 codes per int8 byte, UE8M0 weight
scales, DeepSeek-V4 style checkpoints): the pages fix neither the scale block nor the
nibble order nor the activation format.  Taken here: one UE8M0 scale per row and per
32 consecutive input channels (the OCP MX block, which also expresses any coarser
block scaling exactly by repetition), element 2j in the low nibble of byte j, and
activations quantised exactly as on the fp8 path.  Weight (r, c) dequantises to
e2m1(code) * 2^(scale[r][c / 32] - 127).

Two evaluation orders of the same definition:
  * literal: a loop over tokens and, inside, over the k chosen experts;
  * fast: expert-major, like the page's "eager" backend (loop over the selected
    experts, project the tokens routed to each) -- same arithmetic per element
    up to BLAS summation order.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence, Union

import numpy as np

from .numerics import (
    bf16_bits_to_f64,
    e2m1_decode,
    e4m3_decode,
    fp4_unpack,
    f32_to_e4m3,
    f64_to_bf16_bits,
    f64_to_f32,
    ue8m0_decode,
)

# ----------------------------------------------------------------------------- activation


def silu(z: np.ndarray) -> np.ndarray:
    """z * sigmoid(z) in fp64; exp overflow for very negative z gives -0."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def gelu(z: np.ndarray) -> np.ndarray:
    """z * Phi(z) = z / 2 * erfc(-z / sqrt(2)) in fp64: the exact (erf) form of GELU, the
    gate of GeGLU (SonicMoE section: gated activations silu, gelu or relu map to SwiGLU,
    GeGLU or ReGLU).  erfc keeps the far negative tail accurate (1 + erf would cancel)."""
    from scipy.special import erfc
    z = np.asarray(z, dtype=np.float64)
    return 0.5 * z * erfc(-z / np.sqrt(2.0))


def relu(z: np.ndarray) -> np.ndarray:
    """max(z, 0), the gate of ReGLU."""
    return np.maximum(np.asarray(z, dtype=np.float64), 0.0)


GATES = {"silu": silu, "gelu": gelu, "relu": relu}


# ----------------------------------------------------------------------------- routing

def route(topk_idx: np.ndarray, E: int):
    """Sort the flattened slots a = t*k + j by chosen expert, stably.

    Returns (counts[E], offsets[E+1], perm[A], inv[A]) as int32:
      counts[e]  number of slots that chose e;
      offsets    exclusive prefix sum of counts, offsets[E] = A;
      perm[p]    the slot at position p of the expert-sorted order, slots of one
                 expert kept in increasing slot order (the page's "grouped_mm"
                 row sorts tokens by their selected expert);
      inv[a]     position of slot a in that order (inv[perm[p]] = p).
    Written as a plain counting sort.
    """
    flat = [int(v) for v in np.asarray(topk_idx).reshape(-1)]
    A = len(flat)
    counts = [0] * E
    for e in flat:
        if not 0 <= e < E:
            raise IndexError(f"expert id {e} outside [0, {E})")
        counts[e] += 1
    offsets = [0] * (E + 1)
    for e in range(E):
        offsets[e + 1] = offsets[e] + counts[e]
    fill = offsets[:E]
    perm = [0] * A
    for a, e in enumerate(flat):
        perm[fill[e]] = a
        fill[e] += 1
    inv = [0] * A
    for p, a in enumerate(perm):
        inv[a] = p
    as32 = lambda v: np.asarray(v, dtype=np.int32)  # noqa: E731
    return as32(counts), as32(offsets), as32(perm), as32(inv)


def router_topk(logits: np.ndarray, k: int, renorm: bool):
    """The router step in front of the bookkeeping (softmax -> top-k -> optional renorm).

    logits [T, E] are taken exactly in fp64.  For each token:
      p[e]   = exp(logit[e] - max) / sum_e' exp(logit[e'] - max)   (softmax over all E);
      chosen = the k experts of largest p, taken one at a time, equal p going to the
               lower expert id;
      w[j]   = p[chosen[j]], divided by the sum over the k chosen when renorm.
    Returns (idx int32 [T, k], w fp64 [T, k]), idx in the order chosen.
    """
    lg = np.asarray(logits, dtype=np.float64)
    T, E = lg.shape
    if not 1 <= k <= E:
        raise ValueError(f"k = {k} outside [1, {E}]")
    idx = np.zeros((T, k), dtype=np.int32)
    w = np.zeros((T, k), dtype=np.float64)
    for t in range(T):
        row = lg[t]
        ex = np.exp(row - row.max())
        p = ex / ex.sum()
        left = p.copy()
        for j in range(k):
            e = int(np.argmax(left))     # first of the largest: ties to the lower id
            idx[t, j] = e
            w[t, j] = p[e]
            left[e] = -np.inf
        if renorm:
            w[t] /= w[t].sum()
    return idx, w


# ----------------------------------------------------------------------------- fp8 rows

def quant_rows(v: np.ndarray):
    """Per-row, per-128-channel dynamic e4m3 quantisation of an fp32 matrix.

    Returns (codes uint8 [R, C], scales float32 [R, C/128]).
    """
    v = np.asarray(v, dtype=np.float32)
    R, C = v.shape
    if C % 128:
        raise ValueError("row length must be a multiple of 128")
    g = v.reshape(R, C // 128, 128)
    amax = np.abs(g).max(axis=2)
    s = (amax / np.float32(448.0)).astype(np.float32)
    s[amax == 0] = np.float32(1.0)
    q = f32_to_e4m3((g / s[:, :, None]).astype(np.float32))
    return q.reshape(R, C), s


def dequant_rows(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    R, C = q.shape
    return (e4m3_decode(q).reshape(R, C // 128, 128) * s.astype(np.float64)[:, :, None]).reshape(R, C)


# ----------------------------------------------------------------------------- weights

Storage = Union[np.ndarray, tuple]


@dataclass
class ExpertWeights:
    """Expert weights in their storage format, dequantised to fp64 one expert at a time.

    weight: "f32" | "bf16" | "fp8" | "fp4";  scale: "none" | "f32" | "ue8m0".
    gate_up / down: an indexable [E, ...] array (or a callable e -> matrix), in the
    storage format: fp32 values, bf16 bit patterns, e4m3 codes, or packed e2m1 bytes
    ([rows, cols/2]).  For fp8 the matching scale arrays are [E, rows/128, cols/128],
    for fp4 they are UE8M0 bytes [E, rows, cols/32] (or callables).
    """

    weight: str
    gate_up: Union[np.ndarray, Callable]
    down: Union[np.ndarray, Callable]
    scale: str = "none"
    gate_up_scale: Optional[Union[np.ndarray, Callable]] = None
    down_scale: Optional[Union[np.ndarray, Callable]] = None

    @staticmethod
    def _get(src, e):
        return src(e) if callable(src) else src[e]

    def _deq(self, m, s) -> np.ndarray:
        if self.weight == "f32":
            return np.asarray(m, dtype=np.float32).astype(np.float64)
        if self.weight == "bf16":
            return bf16_bits_to_f64(m)
        if self.weight == "fp8":
            if self.scale == "f32":
                sv = np.asarray(s, dtype=np.float32).astype(np.float64)
            elif self.scale == "ue8m0":
                sv = ue8m0_decode(s)
            else:
                raise ValueError("fp8 weights need block scales")
            R, C = m.shape
            if sv.shape != (R // 128, C // 128):
                raise ValueError("block-scale shape mismatch")
            full = np.repeat(np.repeat(sv, 128, axis=0), 128, axis=1)
            return e4m3_decode(m) * full
        if self.weight == "fp4":
            if self.scale != "ue8m0":
                raise ValueError("fp4 weights need UE8M0 scales")
            codes = fp4_unpack(m)
            R, C = codes.shape
            sv = ue8m0_decode(s)
            if sv.shape != (R, C // 32):
                raise ValueError("fp4 scale shape mismatch")
            return e2m1_decode(codes) * np.repeat(sv, 32, axis=1)
        raise ValueError(f"unknown weight format {self.weight!r}")

    @property
    def quantised(self) -> bool:
        """fp8 and fp4 experts take e4m3 activations with dynamic per-row scales."""
        return self.weight in ("fp8", "fp4")

    def gate_up_f64(self, e: int) -> np.ndarray:
        s = self._get(self.gate_up_scale, e) if self.quantised else None
        return self._deq(self._get(self.gate_up, e), s)

    def down_f64(self, e: int) -> np.ndarray:
        s = self._get(self.down_scale, e) if self.quantised else None
        return self._deq(self._get(self.down, e), s)


# ----------------------------------------------------------------------------- forward

def hidden_f64(x: np.ndarray, act: str) -> np.ndarray:
    if act == "f32":
        return np.asarray(x, dtype=np.float32).astype(np.float64)
    if act == "bf16":
        return bf16_bits_to_f64(x)
    raise ValueError(f"unknown activation format {act!r}")


def _prepare_x(x: np.ndarray, act: str, fp8: bool) -> np.ndarray:
    xf = hidden_f64(x, act)
    if fp8:
        q, s = quant_rows(xf.astype(np.float32))  # exact: bf16/fp32 values fit fp32
        return dequant_rows(q, s)
    return xf


def _swiglu_then_requant(gu: np.ndarray, I: int, fp8: bool, gate: str = "silu", parts=None) -> np.ndarray:
    """gu [..., 2I] fp64 -> the activation fed to the down projection: gate(g) * u with the
    gate function silu (SwiGLU, the default), gelu (GeGLU) or relu (ReGLU).

    With e4m3 activations the result, rounded to fp32, is quantised per row and 128 columns
    and dequantised.  If `parts` is a list, (gu, a rounded to fp32, codes, scales) of these
    rows is appended to it (the intermediate values, for inspection; nothing else changes).
    """
    a = GATES[gate](gu[..., :I]) * gu[..., I:]
    if fp8:
        a2 = np.atleast_2d(f64_to_f32(a))
        q, s = quant_rows(a2)
        if parts is not None:
            parts.append((np.atleast_2d(gu), a2, q, s))
        a = dequant_rows(q, s).reshape(a.shape)
    return a


def round_out(acc: np.ndarray, act: str) -> np.ndarray:
    """fp64 accumulator -> output storage (fp32 values or bf16 bit patterns)."""
    return f64_to_f32(acc) if act == "f32" else f64_to_bf16_bits(acc)


def out_as_f64(out: np.ndarray, act: str) -> np.ndarray:
    return hidden_f64(out, act)


def forward(x: np.ndarray, idx: np.ndarray, w: np.ndarray, weights: ExpertWeights, *,
            act: str, E: Optional[int] = None, mode: str = "fast",
            tokens: Optional[Sequence[int]] = None, gate: str = "silu",
            capture: Optional[dict] = None):
    """Routed top-k experts forward.

    x: [T, H] (fp32 values or bf16 bits); idx: int [T, k]; w: float32 [T, k].
    E: number of experts (taken from the weight arrays when they are arrays).
    tokens: optional subset of token rows to evaluate (each token is independent).
    gate: the gated activation, "silu" (SwiGLU), "gelu" (GeGLU, exact erf form) or "relu"
    (ReGLU).
    capture: with e4m3 activations (fp8 / fp4 experts), an optional dict that receives, for
    every evaluated slot (token t, slot j), capture[(t, j)] = (gu fp64 [2I], a as fp32 [I],
    e4m3 codes [I], float32 scales [I/128]): the SwiGLU intermediates of the definition.
    Returns (acc fp64 [n, H], out [n, H] in the output storage) for the chosen
    rows (all T rows when tokens is None), in the order of `tokens`.
    """
    idx = np.asarray(idx)
    T, k = idx.shape
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    fp8 = weights.quantised          # e4m3 activations (fp8 and fp4 experts)
    if E is None and not callable(weights.gate_up):
        E = len(weights.gate_up)
    chosen = idx[rows]
    if chosen.size and (chosen.min() < 0 or (E is not None and chosen.max() >= E)):
        raise IndexError("expert id outside [0, E)")
    xs = _prepare_x(np.asarray(x)[rows], act, fp8)          # [n, H] fp64
    ws = np.asarray(w, dtype=np.float32)[rows].astype(np.float64)
    ids = idx[rows]
    n, H = xs.shape
    acc = np.zeros((n, H), dtype=np.float64)
    if mode == "literal":
        cache: dict = {}
        for r in range(n):
            for j in range(k):
                e = int(ids[r, j])
                if e not in cache:
                    cache.clear()
                    cache[e] = (weights.gate_up_f64(e), weights.down_f64(e))
                wgu, wd = cache[e]
                I = wd.shape[1]
                parts = [] if (capture is not None and fp8) else None
                a = _swiglu_then_requant(wgu @ xs[r], I, fp8, gate, parts)
                if parts:
                    gu_, a32_, q_, s_ = parts[0]
                    capture[(int(rows[r]), j)] = (gu_[0], a32_[0], q_[0], s_[0])
                acc[r] += ws[r, j] * (wd @ a)
    elif mode == "fast":
        flat = ids.reshape(-1)
        for e in np.unique(flat):
            sl = np.nonzero(flat == e)[0]          # slots (r*k + j) choosing e
            r_of, j_of = sl // k, sl % k
            wgu, wd = weights.gate_up_f64(int(e)), weights.down_f64(int(e))
            I = wd.shape[1]
            parts = [] if (capture is not None and fp8) else None
            a = _swiglu_then_requant(xs[r_of] @ wgu.T, I, fp8, gate, parts)
            if parts:
                gu_, a32_, q_, s_ = parts[0]
                for n_, (r_, j_) in enumerate(zip(r_of, j_of)):
                    capture[(int(rows[r_]), int(j_))] = (gu_[n_], a32_[n_], q_[n_], s_[n_])
            y = a @ wd.T
            np.add.at(acc, r_of, ws[r_of, j_of][:, None] * y)
    else:
        raise ValueError(f"unknown mode {mode!r}")
    return acc, round_out(acc, act)
