"""Routed top-k MoE experts forward on MI355X (gfx950): Python binding.

A thin ctypes layer over libmoe_experts.so (declared in include/moe_experts.h).
It only marshals arguments: torch tensors provide device pointers, the current
HIP stream and workspace memory; every step of the forward runs in the library's
HIP kernels.  There is no fallback: if the library is not built, or a tensor is
not on the GPU, the call raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "experts_forward", "experts_forward_noalloc", "check_scales", "check_mfma_blocks", "route", "route_logits", "quantize_rows_fp8", "workspace_size", "plan_describe",
    "Problem", "MoeError", "lib", "FLAG_CHECK_INDICES", "FLAG_DETERMINISTIC", "FLAG_ATOMIC_COMBINE", "FLAG_ACT_GELU", "FLAG_ACT_RELU",
    "FLAG_FORCE_GROUPED", "FLAG_FORCE_DECODE", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_experts.so")

# moe_status
OK, ERR_NULL_ARG, ERR_BAD_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_BAD_INDEX, ERR_HIP = range(7)
# moe_dtype
F32, BF16, FP8_E4M3, FP4_E2M1 = 0, 1, 2, 3
# moe_scale_fmt
SCALE_NONE, SCALE_F32, SCALE_UE8M0 = 0, 1, 2
# flags
FLAG_CHECK_INDICES = 1
FLAG_DETERMINISTIC = 2
FLAG_FORCE_GROUPED = 4
FLAG_FORCE_DECODE = 8
FLAG_ATOMIC_COMBINE = 16
FLAG_ACT_GELU = 32
FLAG_ACT_RELU = 64

EXPORTS = ["moe_abi_version", "moe_status_str", "moe_workspace_size", "moe_experts_forward",
           "moe_route", "moe_route_logits", "moe_quantize_rows_fp8", "moe_plan_describe",
           "moe_set_stage_events", "moe_check_mfma_blocks", "moe_experts_forward_noalloc",
           "moe_noalloc_scratch_bytes"]

# stage ids (moe_set_stage_events)
STAGES = ["zero", "route", "quant_x", "gate_up", "quant_act", "down", "finalize"]


class Problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("scale_fmt", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"moe status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                           "`python -m mixture_experts_routed_topk_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(Problem)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    L.moe_abi_version.restype = ctypes.c_int
    L.moe_abi_version.argtypes = []
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_workspace_size.restype = ctypes.c_int
    L.moe_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    L.moe_experts_forward.restype = ctypes.c_int
    L.moe_experts_forward.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_experts_forward_noalloc.restype = ctypes.c_int
    L.moe_experts_forward_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_noalloc_scratch_bytes.restype = ctypes.c_size_t
    L.moe_noalloc_scratch_bytes.argtypes = []
    L.moe_route.restype = ctypes.c_int
    L.moe_route.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_route_logits.restype = ctypes.c_int
    L.moe_route_logits.argtypes = [P, vp, ctypes.c_int, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_quantize_rows_fp8.restype = ctypes.c_int
    L.moe_quantize_rows_fp8.argtypes = [vp, ctypes.c_int64, ctypes.c_int32, vp, vp, vp]
    L.moe_plan_describe.restype = ctypes.c_int
    L.moe_plan_describe.argtypes = [P, ctypes.c_char_p, sz]
    L.moe_check_mfma_blocks.restype = ctypes.c_int
    L.moe_check_mfma_blocks.argtypes = [ctypes.c_int, vp, vp, vp, vp, ctypes.c_int, vp]
    L.moe_set_stage_events.restype = ctypes.c_int
    L.moe_set_stage_events.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int]
    _lib = L
    return L


def _check(status: int):
    if status == OK:
        return
    msg = lib().moe_status_str(status).decode()
    if status in (ERR_NULL_ARG, ERR_BAD_SHAPE, ERR_UNSUPPORTED, ERR_WORKSPACE):
        raise ValueError(f"moe status {status}: {msg}")
    if status == ERR_BAD_INDEX:
        raise IndexError(f"moe status {status}: {msg}")
    raise MoeError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


_ACT = {torch.float32: F32, torch.bfloat16: BF16}
_WGT = {torch.float32: F32, torch.bfloat16: BF16, torch.float8_e4m3fn: FP8_E4M3, torch.uint8: FP8_E4M3}
_FP4_DTYPES = (torch.float4_e2m1fn_x2,) if hasattr(torch, "float4_e2m1fn_x2") else ()


def make_problem(T, H, I, E, k, act, weight, scale=SCALE_NONE, flags=0) -> Problem:
    return Problem(T, H, I, E, k, act, weight, scale, flags)


def workspace_size(problem: Problem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().moe_workspace_size(ctypes.byref(problem), ctypes.byref(n)))
    return n.value


def plan_describe(problem: Problem) -> str:
    buf = ctypes.create_string_buffer(512)
    _check(lib().moe_plan_describe(ctypes.byref(problem), buf, len(buf)))
    return buf.value.decode()


def _need_gpu(name: str, t: torch.Tensor):
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def problem_for(hidden, topk_idx, w_gate_up, w_down, w_gate_up_scale=None, flags=0) -> Problem:
    T, H = hidden.shape
    E, twoI, H2 = w_gate_up.shape
    k = topk_idx.shape[1]
    # fp4 weights: packed bytes (uint8 or float4_e2m1fn_x2) with half as many columns
    fp4 = (w_gate_up.dtype in _FP4_DTYPES or w_gate_up.dtype == torch.uint8) and 2 * H2 == H
    cols = 2 if fp4 else 1
    if (H2 * cols != H or twoI % 2 or tuple(w_down.shape) != (E, H, twoI // 2 // cols)
            or topk_idx.shape[0] != T):
        raise ValueError("inconsistent shapes: hidden [T,H], topk_idx [T,k], "
                         "w_gate_up [E,2I,H], w_down [E,H,I] (fp4: [E,2I,H/2], [E,H,I/2])")
    if hidden.dtype not in _ACT or w_down.dtype != w_gate_up.dtype or not (fp4 or w_gate_up.dtype in _WGT):
        raise ValueError("unsupported dtypes")
    weight = FP4_E2M1 if fp4 else _WGT[w_gate_up.dtype]
    scale = SCALE_NONE
    if weight in (FP8_E4M3, FP4_E2M1):
        if w_gate_up_scale is None:
            raise ValueError("fp8 and fp4 weights need scales")
        scale = SCALE_UE8M0 if w_gate_up_scale.dtype == torch.uint8 else SCALE_F32
    return Problem(T, H, twoI // 2, E, k, _ACT[hidden.dtype], weight, scale, flags)


def check_scales(prob: Problem, w_gate_up_scale: Optional[torch.Tensor],
                 w_down_scale: Optional[torch.Tensor]) -> None:
    """Block scales must match the weight format exactly, since the kernels read them by index.

    e4m3 weights: [E, 2I/128, H/128] and [E, H/128, I/128], both float32 or both uint8 (UE8M0);
    fp4 weights: [E, 2I, H/32] and [E, H, I/32] uint8 (UE8M0); other weights take none.
    Raises ValueError on a missing, extra, mismatched or wrongly shaped scale tensor.
    """
    E, H, I = prob.E, prob.H, prob.I
    if prob.weight_dtype not in (FP8_E4M3, FP4_E2M1):
        if w_gate_up_scale is not None or w_down_scale is not None:
            raise ValueError("block scales are only taken with e4m3 or fp4 weights")
        return
    if w_gate_up_scale is None or w_down_scale is None:
        raise ValueError("e4m3 and fp4 weights need both w_gate_up_scale and w_down_scale")
    if w_gate_up_scale.dtype != w_down_scale.dtype:
        raise ValueError(f"scale dtypes differ: {w_gate_up_scale.dtype} and {w_down_scale.dtype}")
    if prob.weight_dtype == FP4_E2M1:
        if w_gate_up_scale.dtype != torch.uint8:
            raise ValueError("fp4 weights take UE8M0 (uint8) scales")
        want = ((E, 2 * I, H // 32), (E, H, I // 32))
    else:
        if w_gate_up_scale.dtype not in (torch.float32, torch.uint8):
            raise ValueError("e4m3 block scales must be float32 or uint8 (UE8M0)")
        want = ((E, 2 * I // 128, H // 128), (E, H // 128, I // 128))
    for name, t, shape in (("w_gate_up_scale", w_gate_up_scale, want[0]),
                           ("w_down_scale", w_down_scale, want[1])):
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {shape}")


def experts_forward(hidden: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                    w_gate_up: torch.Tensor, w_down: torch.Tensor,
                    w_gate_up_scale: Optional[torch.Tensor] = None,
                    w_down_scale: Optional[torch.Tensor] = None,
                    out: Optional[torch.Tensor] = None, flags: int = 0,
                    workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """out[T,H] = sum_j topk_w[:,j] * SwiGLU-MLP_{topk_idx[:,j]}(hidden) on the GPU.

    hidden [T,H] f32|bf16; topk_idx [T,k] int32; topk_w [T,k] f32;
    w_gate_up [E,2I,H] and w_down [E,H,I] in f32 | bf16 | e4m3 (float8_e4m3fn or
    uint8 codes) with block scales [E,2I/128,H/128] / [E,H/128,I/128]
    (float32, or uint8 UE8M0 exponents); or fp4: w_gate_up [E,2I,H/2] and
    w_down [E,H,I/2] packed e2m1 bytes (uint8 or float4_e2m1fn_x2, element 2j in the low
    nibble of byte j) with UE8M0 scales [E,2I,H/32] / [E,H,I/32] (uint8).
    """
    for name, t in (("hidden", hidden), ("topk_idx", topk_idx), ("topk_w", topk_w),
                    ("w_gate_up", w_gate_up), ("w_down", w_down)):
        _need_gpu(name, t)
    if topk_idx.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("topk_idx must be int32 and topk_w float32")
    if topk_w.shape != topk_idx.shape:
        raise ValueError("topk_w and topk_idx shapes differ")
    prob = problem_for(hidden, topk_idx, w_gate_up, w_down, w_gate_up_scale, flags)
    check_scales(prob, w_gate_up_scale, w_down_scale)
    for name, t in (("w_gate_up_scale", w_gate_up_scale), ("w_down_scale", w_down_scale)):
        if t is not None:
            _need_gpu(name, t)
    if out is None:
        out = torch.empty_like(hidden)
    else:
        _need_gpu("out", out)
        if out.shape != hidden.shape or out.dtype != hidden.dtype:
            raise ValueError("out must match hidden in shape and dtype")
    nbytes = workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=hidden.device)
    else:
        _need_gpu("workspace", workspace)
    _check(lib().moe_experts_forward(
        ctypes.byref(prob), _ptr(hidden), _ptr(topk_idx), _ptr(topk_w), _ptr(w_gate_up),
        _ptr(w_down), _ptr(w_gate_up_scale), _ptr(w_down_scale), _ptr(out), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(hidden.device)))
    return out


def experts_forward_noalloc(hidden: torch.Tensor, topk_idx: torch.Tensor, topk_w: torch.Tensor,
                            w_gate_up: torch.Tensor, w_down: torch.Tensor,
                            w_gate_up_scale: Optional[torch.Tensor] = None,
                            w_down_scale: Optional[torch.Tensor] = None,
                            out: Optional[torch.Tensor] = None, flags: int = 0) -> torch.Tensor:
    """experts_forward on the library's own device array instead of a workspace
    (moe_experts_forward_noalloc): allocates nothing when `out` is given."""
    for name, t in (("hidden", hidden), ("topk_idx", topk_idx), ("topk_w", topk_w),
                    ("w_gate_up", w_gate_up), ("w_down", w_down)):
        _need_gpu(name, t)
    if topk_idx.dtype != torch.int32 or topk_w.dtype != torch.float32:
        raise ValueError("topk_idx must be int32 and topk_w float32")
    if topk_w.shape != topk_idx.shape:
        raise ValueError("topk_w and topk_idx shapes differ")
    prob = problem_for(hidden, topk_idx, w_gate_up, w_down, w_gate_up_scale, flags)
    check_scales(prob, w_gate_up_scale, w_down_scale)
    for name, t in (("w_gate_up_scale", w_gate_up_scale), ("w_down_scale", w_down_scale)):
        if t is not None:
            _need_gpu(name, t)
    if out is None:
        out = torch.empty_like(hidden)
    else:
        _need_gpu("out", out)
        if out.shape != hidden.shape or out.dtype != hidden.dtype:
            raise ValueError("out must match hidden in shape and dtype")
    _check(lib().moe_experts_forward_noalloc(
        ctypes.byref(prob), _ptr(hidden), _ptr(topk_idx), _ptr(topk_w), _ptr(w_gate_up), _ptr(w_down),
        _ptr(w_gate_up_scale), _ptr(w_down_scale), _ptr(out), _stream(hidden.device)))
    return out


def route(topk_idx: torch.Tensor, E: int, flags: int = 0, workspace=None):
    """(counts[E], offsets[E+1], perm[T*k], inv[T*k]) int32: the stable sort of slots by expert."""
    _need_gpu("topk_idx", topk_idx)
    if topk_idx.dtype != torch.int32 or topk_idx.dim() != 2:
        raise ValueError("topk_idx must be a 2-D int32 tensor")
    T, k = topk_idx.shape
    dev = topk_idx.device
    # the bookkeeping does not depend on H, I or the dtypes; any valid problem sizes it
    prob = Problem(T, 128, 128, E, k, BF16, BF16, SCALE_NONE, flags)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_size(prob), dtype=torch.uint8, device=dev)
    _check(lib().moe_route(ctypes.byref(prob), _ptr(topk_idx), _ptr(counts), _ptr(offsets),
                           _ptr(perm), _ptr(inv), _ptr(workspace), workspace.numel(), _stream(dev)))
    return counts, offsets, perm[: T * k], inv[: T * k]


def route_logits(logits: torch.Tensor, k: int, renorm: bool = False, workspace=None):
    """Router + bookkeeping from float32 logits [T, E]: (topk_idx[T,k] int32, topk_w[T,k] float32,
    counts[E], offsets[E+1], perm[T*k], inv[T*k]); see moe_route_logits."""
    _need_gpu("logits", logits)
    if logits.dtype != torch.float32 or logits.dim() != 2 or not logits.is_contiguous():
        raise ValueError("logits must be a contiguous 2-D float32 tensor")
    T, E = logits.shape
    dev = logits.device
    prob = Problem(T, 128, 128, E, k, BF16, BF16, SCALE_NONE, 0)
    idx = torch.empty((max(T, 1), k), dtype=torch.int32, device=dev)
    w = torch.empty((max(T, 1), k), dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    inv = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(workspace_size(prob), dtype=torch.uint8, device=dev)
    _check(lib().moe_route_logits(ctypes.byref(prob), _ptr(logits), int(bool(renorm)), _ptr(idx), _ptr(w),
                                  _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(inv), _ptr(workspace),
                                  workspace.numel(), _stream(dev)))
    return idx[:T], w[:T], counts, offsets, perm[: T * k], inv[: T * k]


def set_stage_events(handles):
    """Install per-stage hipEvent_t handles (a list of 2*len(STAGES) ints or None) on this thread;
    None clears the hook."""
    if handles is None:
        _check(lib().moe_set_stage_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(handles))(*[h or None for h in handles])
    _check(lib().moe_set_stage_events(arr, len(handles)))


def quantize_rows_fp8(x: torch.Tensor):
    """Per-row, per-128-column e4m3 quantisation of a bf16 matrix -> (codes uint8, scales f32)."""
    _need_gpu("x", x)
    if x.dtype != torch.bfloat16 or x.dim() != 2:
        raise ValueError("x must be a 2-D bf16 tensor")
    R, C = x.shape
    if C % 128:
        raise ValueError("columns must be a multiple of 128")
    q = torch.empty((R, C), dtype=torch.uint8, device=x.device)
    s = torch.empty((R, C // 128), dtype=torch.float32, device=x.device)
    _check(lib().moe_quantize_rows_fp8(_ptr(x), R, C, _ptr(q), _ptr(s), _stream(x.device)))
    return q, s


def check_mfma_blocks(a: torch.Tensor, b: torch.Tensor, b_scale: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Block products on the kernels' block-scaled MFMA (moe_check_mfma_blocks): a uint8
    [n,16,128] e4m3 codes; b uint8 [n,16,128] e4m3 codes (with an optional b_scale), or
    [n,16,64] packed e2m1 with b_scale; b_scale uint8 [n,16,4] UE8M0.  Returns float32
    [n,16,16]."""
    fmt = 0 if b_scale is None else (2 if b.dim() == 3 and b.shape[-1] == 128 else 1)
    for name, t in (("a", a), ("b", b)) + ((("b_scale", b_scale),) if fmt else ()):
        _need_gpu(name, t)
        if t.dtype != torch.uint8:
            raise ValueError(f"{name} must be uint8")
    n = a.shape[0]
    want_b = (n, 16, 64) if fmt == 1 else (n, 16, 128)
    if tuple(a.shape) != (n, 16, 128) or tuple(b.shape) != want_b or (fmt and tuple(b_scale.shape) != (n, 16, 4)):
        raise ValueError("shapes: a [n,16,128], b [n,16,128] (e4m3, b_scale optional) or [n,16,64] with "
                         "b_scale [n,16,4] (e2m1)")
    d = torch.empty((n, 16, 16), dtype=torch.float32, device=a.device)
    _check(lib().moe_check_mfma_blocks(fmt, _ptr(a), _ptr(b), _ptr(b_scale), _ptr(d), n, _stream(a.device)))
    return d
