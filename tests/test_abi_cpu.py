"""The C-ABI library loads without a GPU, exports what the header declares, and
rejects bad arguments on the host before any HIP call."""

import ctypes
import os
import re

import pytest

import mixture_experts_routed_topk_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_experts.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def test_header_and_binding_agree():
    assert _declared() == sorted(m.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = m.lib()
    for name in _declared():
        assert hasattr(L, name), name
    assert L.moe_abi_version() == 1
    for s in range(7):
        assert L.moe_status_str(s)


def P(**kw):
    d = dict(T=32, H=128, I=256, E=8, k=2, act=m.F32, weight=m.F32, scale=m.SCALE_NONE, flags=0)
    d.update(kw)
    return m.Problem(d["T"], d["H"], d["I"], d["E"], d["k"], d["act"], d["weight"], d["scale"],
                     d["flags"])


def _ws(p):
    n = ctypes.c_size_t(0)
    return m.lib().moe_workspace_size(ctypes.byref(p), ctypes.byref(n)), n.value


@pytest.mark.parametrize("kw,status", [
    (dict(), m.OK),
    (dict(act=m.BF16, weight=m.BF16), m.OK),
    (dict(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32), m.OK),
    (dict(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_UE8M0), m.OK),
    (dict(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0), m.OK),
    (dict(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_F32), m.ERR_UNSUPPORTED),   # fp4: UE8M0 only
    (dict(act=m.BF16, weight=m.FP4_E2M1), m.ERR_UNSUPPORTED),
    (dict(act=m.F32, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0), m.ERR_UNSUPPORTED),
    (dict(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0, I=192), m.ERR_BAD_SHAPE),
    (dict(act=m.BF16, weight=4, scale=m.SCALE_UE8M0), m.ERR_UNSUPPORTED),
    (dict(T=0), m.OK),
    (dict(k=9), m.ERR_BAD_SHAPE),
    (dict(k=0), m.ERR_BAD_SHAPE),
    (dict(E=0), m.ERR_BAD_SHAPE),
    (dict(E=1025, k=1), m.ERR_BAD_SHAPE),
    (dict(T=-1), m.ERR_BAD_SHAPE),
    (dict(H=96), m.ERR_BAD_SHAPE),
    (dict(I=96), m.ERR_BAD_SHAPE),
    (dict(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32, I=192), m.ERR_BAD_SHAPE),
    (dict(T=2**30, k=2), m.ERR_BAD_SHAPE),
    (dict(act=m.F32, weight=m.BF16), m.ERR_UNSUPPORTED),
    (dict(act=m.BF16, weight=m.FP8_E4M3), m.ERR_UNSUPPORTED),          # fp8 without scales
    (dict(act=m.BF16, weight=m.BF16, scale=m.SCALE_F32), m.ERR_UNSUPPORTED),
    (dict(act=m.F32, weight=m.FP8_E4M3, scale=m.SCALE_F32), m.ERR_UNSUPPORTED),
    (dict(flags=m.FLAG_FORCE_DECODE | m.FLAG_FORCE_GROUPED), m.ERR_UNSUPPORTED),
    (dict(flags=128), m.ERR_UNSUPPORTED),
    (dict(flags=m.FLAG_ACT_GELU | m.FLAG_ACT_RELU), m.ERR_UNSUPPORTED),
    (dict(flags=m.FLAG_ACT_GELU), m.OK),
    (dict(flags=m.FLAG_ACT_RELU), m.OK),
])
def test_problem_validation(kw, status):
    st, n = _ws(P(**kw))
    assert st == status
    if status == m.OK:
        assert n > 0


def test_workspace_by_combine():
    # per-slot rows [T*k, H] f32 (deterministic, and the default while they are <= 512 MiB)
    # against the [T, H] f32 accumulator of the atomic combine
    p = P(act=m.BF16, weight=m.BF16, T=4096, H=2048, I=1408, E=60, k=4)
    _, n_default = _ws(p)
    p.flags = m.FLAG_ATOMIC_COMBINE
    _, n_atomic = _ws(p)
    p.flags = m.FLAG_DETERMINISTIC
    _, n_det = _ws(p)
    A, H, T = 4096 * 4, 2048, 4096
    assert n_det - n_default == 2 * A * H        # default: bf16 slot rows; deterministic: float32
    assert n_det - n_atomic == 4 * A * H - 4 * T * H
    # bf16 layers keep bf16 slot rows up to 1 GiB of them (the DeepSeek-shaped layer: 0.94 GB) ...
    big = P(act=m.BF16, weight=m.BF16, T=8192, H=7168, I=2048, E=256, k=8)
    _, nb_default = _ws(big)
    big.flags = m.FLAG_ATOMIC_COMBINE
    _, nb_atomic = _ws(big)
    Ab, Hb, Tb = 8192 * 8, 7168, 8192
    assert nb_default - nb_atomic == 2 * Ab * Hb - 4 * Tb * Hb
    assert "combine=slot_rows_bf16" in m.plan_describe(P(act=m.BF16, weight=m.BF16, T=8192, H=7168, I=2048,
                                                         E=256, k=8))
    # ... as do fp8 and fp4 layers (their down kernels share the bf16 slot-row epilogue) ...
    fp8 = P(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32, T=4096, H=7168, I=2048, E=256, k=8)
    assert "combine=slot_rows_bf16" in m.plan_describe(fp8)
    fp4 = P(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0, T=4096, H=7168, I=2048, E=256, k=8)
    assert "combine=slot_rows_bf16" in m.plan_describe(fp4)
    # ... and above that, or for float32 rows above 512 MiB, the default is the atomic combine
    bigger = P(act=m.BF16, weight=m.BF16, T=9363, H=7168, I=2048, E=256, k=8)   # 2*T*k*H > 1 GiB
    assert "combine=atomic_f32" in m.plan_describe(bigger)
    fp8.T = 9363
    assert "combine=atomic_f32" in m.plan_describe(fp8)
    f32 = P(act=m.F32, weight=m.F32, T=2341, H=7168, I=2048, E=256, k=8)        # 4*T*k*H > 512 MiB
    assert "combine=atomic_f32" in m.plan_describe(f32)
    p.flags = m.FLAG_DETERMINISTIC | m.FLAG_ATOMIC_COMBINE
    assert _ws(p)[0] == m.ERR_UNSUPPORTED


def test_forward_rejects_before_any_hip_call():
    L = m.lib()
    p = P()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    # null hidden
    st = L.moe_experts_forward(ctypes.byref(p), None, fake, fake, fake, fake, None, None, fake,
                               fake, 1 << 40, None)
    assert st == m.ERR_NULL_ARG
    # workspace too small
    st = L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, None, None, fake,
                               fake, 16, None)
    assert st == m.ERR_WORKSPACE
    # misaligned hidden
    st = L.moe_experts_forward(ctypes.byref(p), ctypes.c_void_p(0x10004), fake, fake, fake, fake,
                               None, None, fake, fake, 1 << 40, None)
    assert st == m.ERR_BAD_SHAPE
    # fp8 without scale pointers
    p8 = P(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32)
    st = L.moe_experts_forward(ctypes.byref(p8), fake, fake, fake, fake, fake, None, None, fake,
                               fake, 1 << 40, None)
    assert st == m.ERR_NULL_ARG
    # fp4 without scale pointers; fp4 has no decode path
    p4 = P(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0)
    st = L.moe_experts_forward(ctypes.byref(p4), fake, fake, fake, fake, fake, None, None, fake,
                               fake, 1 << 40, None)
    assert st == m.ERR_NULL_ARG
    p4.flags = m.FLAG_FORCE_DECODE
    st = L.moe_experts_forward(ctypes.byref(p4), fake, fake, fake, fake, fake, fake, fake, fake,
                               fake, 1 << 40, None)
    assert st == m.ERR_UNSUPPORTED
    # the decode path holds its routing tables in LDS: at most 2048 slots
    pd = P(act=m.BF16, weight=m.BF16, T=64, k=33, E=64, I=128, flags=m.FLAG_FORCE_DECODE)
    st = L.moe_experts_forward(ctypes.byref(pd), fake, fake, fake, fake, fake, None, None, fake,
                               fake, 1 << 40, None)
    assert st == m.ERR_UNSUPPORTED
    pd.k = 32
    s = ctypes.create_string_buffer(512)
    assert L.moe_plan_describe(ctypes.byref(pd), s, 512) == m.OK
    assert b"path=decode" in s.value
    # null problem
    assert L.moe_experts_forward(None, fake, fake, fake, fake, fake, None, None, fake, fake,
                                 1 << 40, None) == m.ERR_NULL_ARG
    # T == 0 is a no-op that touches nothing
    p0 = P(T=0)
    assert L.moe_experts_forward(ctypes.byref(p0), None, None, None, None, None, None, None, None,
                                 None, 0, None) == m.OK


def test_quantize_rows_validation():
    L = m.lib()
    fake = ctypes.c_void_p(0x10000)
    assert L.moe_quantize_rows_fp8(fake, 4, 100, fake, fake, None) == m.ERR_BAD_SHAPE
    assert L.moe_quantize_rows_fp8(fake, -1, 128, fake, fake, None) == m.ERR_BAD_SHAPE
    assert L.moe_quantize_rows_fp8(None, 4, 128, fake, fake, None) == m.ERR_NULL_ARG
    assert L.moe_quantize_rows_fp8(None, 0, 128, None, None, None) == m.OK


def test_plan_describe():
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=4096, H=2048, I=1408, E=60, k=4))
    assert "path=grouped" in s and "weights=bf16" in s
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=16, H=2048, I=1408, E=60, k=4))
    assert "path=decode" in s
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=16, H=2048, I=1408, E=60, k=4,
                          flags=m.FLAG_FORCE_GROUPED))
    assert "path=grouped" in s
    # the default switch: decode while T * k <= min(16 * E, 512)
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=128, H=2048, I=1408, E=60, k=4))
    assert "path=decode" in s
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=129, H=2048, I=1408, E=60, k=4))
    assert "path=grouped" in s
    s = m.plan_describe(P(act=m.BF16, weight=m.BF16, T=33, H=256, I=128, E=2, k=1))   # > 16 E
    assert "path=grouped" in s
    s = m.plan_describe(P(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0, T=16, H=7168, I=2048,
                          E=256, k=8))
    assert "path=grouped" in s and "weights=fp4_e2m1" in s and "scales=ue8m0" in s


def test_python_problem_infers_fp4_from_packed_shape():
    import torch
    x = torch.zeros(4, 256, dtype=torch.bfloat16)
    idx = torch.zeros(4, 2, dtype=torch.int32)
    gu4 = torch.zeros(3, 256, 128, dtype=torch.uint8)
    dn4 = torch.zeros(3, 256, 64, dtype=torch.uint8)
    p = m.problem_for(x, idx, gu4, dn4, torch.zeros(3, 256, 8, dtype=torch.uint8))
    assert (p.weight_dtype, p.scale_fmt, p.I) == (m.FP4_E2M1, m.SCALE_UE8M0, 128)
    gu8 = torch.zeros(3, 256, 256, dtype=torch.uint8)
    dn8 = torch.zeros(3, 256, 128, dtype=torch.uint8)
    p = m.problem_for(x, idx, gu8, dn8, torch.zeros(3, 2, 2, dtype=torch.float32))
    assert (p.weight_dtype, p.scale_fmt, p.I) == (m.FP8_E4M3, m.SCALE_F32, 128)
    with pytest.raises(ValueError):
        m.problem_for(x, idx, gu4, dn4, None)


def test_python_wrapper_rejects_cpu_tensors():
    import torch
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError):
        m.experts_forward(x, torch.zeros(4, 2, dtype=torch.int32), torch.zeros(4, 2),
                          torch.zeros(8, 512, 128), torch.zeros(8, 128, 256))


def test_route_logits_rejects_before_any_hip_call():
    L = m.lib()
    fake = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first
    p = P(act=m.BF16, weight=m.BF16, T=4, H=128, I=128, E=100, k=65)
    st = L.moe_route_logits(ctypes.byref(p), fake, 0, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == m.ERR_UNSUPPORTED      # k > 64
    p.k = 4
    st = L.moe_route_logits(ctypes.byref(p), None, 0, fake, fake, fake, fake, fake, fake, fake, 1 << 40, None)
    assert st == m.ERR_NULL_ARG         # no logits
    st = L.moe_route_logits(ctypes.byref(p), fake, 0, fake, fake, fake, fake, fake, fake, fake, 16, None)
    assert st == m.ERR_WORKSPACE


# ----------------------------------------------------------------------------- scale tensors

def _scales(shape_gu, shape_dn, dtype_gu, dtype_dn=None):
    import torch
    return torch.zeros(shape_gu, dtype=dtype_gu), torch.zeros(shape_dn, dtype=dtype_dn or dtype_gu)


def test_check_scales_accepts_the_exact_shapes():
    import torch
    E, H, I = 4, 256, 384
    p8 = P(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32, E=E, H=H, I=I)
    for dt in (torch.float32, torch.uint8):
        m.check_scales(p8, *_scales((E, 2 * I // 128, H // 128), (E, H // 128, I // 128), dt))
    p4 = P(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0, E=E, H=H, I=I)
    m.check_scales(p4, *_scales((E, 2 * I, H // 32), (E, H, I // 32), torch.uint8))
    m.check_scales(P(act=m.BF16, weight=m.BF16), None, None)


@pytest.mark.parametrize("case", ["mixed_dtypes", "short_gate_up", "short_down", "missing_down",
                                  "fp4_float_scales", "fp4_short", "scales_on_bf16", "float64"])
def test_check_scales_rejects(case):
    import torch
    E, H, I = 4, 256, 384
    p8 = P(act=m.BF16, weight=m.FP8_E4M3, scale=m.SCALE_F32, E=E, H=H, I=I)
    p4 = P(act=m.BF16, weight=m.FP4_E2M1, scale=m.SCALE_UE8M0, E=E, H=H, I=I)
    gu8, dn8 = (E, 2 * I // 128, H // 128), (E, H // 128, I // 128)
    gu4, dn4 = (E, 2 * I, H // 32), (E, H, I // 32)
    args = {
        # a float32 w_down_scale beside UE8M0 gate_up scales would be read as bytes
        "mixed_dtypes": (p8, *_scales(gu8, dn8, torch.uint8, torch.float32)),
        "short_gate_up": (p8, *_scales((E, 2 * I // 128 - 1, H // 128), dn8, torch.float32)),
        "short_down": (p8, *_scales(gu8, (E - 1, H // 128, I // 128), torch.float32)),
        "missing_down": (p8, _scales(gu8, dn8, torch.float32)[0], None),
        "fp4_float_scales": (p4, *_scales(gu4, dn4, torch.float32)),
        "fp4_short": (p4, *_scales(gu4, (E, H, I // 64), torch.uint8)),
        "scales_on_bf16": (P(act=m.BF16, weight=m.BF16), *_scales(gu8, dn8, torch.float32)),
        "float64": (p8, *_scales(gu8, dn8, torch.float64)),
    }[case]
    with pytest.raises(ValueError):
        m.check_scales(*args)


# ----------------------------------------------------------------------------- allocation-free forward

def test_noalloc_rejects_problems_beyond_its_array_before_any_hip_call():
    L = m.lib()
    cap = L.moe_noalloc_scratch_bytes()
    assert cap == 128 << 20
    fake = ctypes.c_void_p(1 << 20)     # aligned stand-ins: the size check comes before any HIP call
    big = P(act=m.BF16, weight=m.BF16, T=8192, H=7168, I=2048, E=256, k=8)
    assert m.workspace_size(big) > cap
    st = L.moe_experts_forward_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, None, None, fake, None)
    assert st == m.ERR_WORKSPACE
    # the Qwen-shaped prefill layer fits
    qwen = P(act=m.BF16, weight=m.BF16, T=4096, H=2048, I=1408, E=60, k=4)
    assert m.workspace_size(qwen) <= cap
    # argument errors as for the forward
    assert L.moe_experts_forward_noalloc(None, fake, fake, fake, fake, fake, None, None, fake, None) == m.ERR_NULL_ARG
    assert L.moe_experts_forward_noalloc(ctypes.byref(qwen), None, fake, fake, fake, fake, None, None, fake,
                                         None) == m.ERR_NULL_ARG
    t0 = P(act=m.BF16, weight=m.BF16, T=0)
    assert L.moe_experts_forward_noalloc(ctypes.byref(t0), None, None, None, None, None, None, None, None, None) == m.OK


def test_check_mfma_blocks_rejects_before_any_hip_call():
    L = m.lib()
    a, b, s, d = ctypes.c_void_p(4096), ctypes.c_void_p(8192), ctypes.c_void_p(12288), ctypes.c_void_p(16384)
    assert L.moe_check_mfma_blocks(3, a, b, s, d, 4, None) == m.ERR_UNSUPPORTED
    assert L.moe_check_mfma_blocks(-1, a, b, s, d, 4, None) == m.ERR_UNSUPPORTED
    assert L.moe_check_mfma_blocks(0, a, b, None, d, -1, None) == m.ERR_BAD_SHAPE
    assert L.moe_check_mfma_blocks(2, a, b, None, d, 4, None) == m.ERR_NULL_ARG    # fmt 2 needs exponents
    assert L.moe_check_mfma_blocks(1, a, b, None, d, 4, None) == m.ERR_NULL_ARG
    assert L.moe_check_mfma_blocks(2, ctypes.c_void_p(4100), b, s, d, 4, None) == m.ERR_BAD_SHAPE   # a not 16-byte aligned
    assert L.moe_check_mfma_blocks(2, a, b, s, d, 0, None) == m.OK                # nothing to do, no launch
