"""The accumulation bound of the block-scaled 16x16x128 MFMA, checked on the instruction itself.

The e4m3 and FP4 grouped kernels compute every 128-long block of their dot products with
one such MFMA (zero accumulator) and fold the result into float32 ("FP8 and FP4 quantized
experts" section of the Experts backends page: fp8 / fp4 expert GEMMs with per-block
scales).  The parity check of the requantised SwiGLU rows (moe_helpers.check_requantised)
takes |MFMA block result - exact block sum| <= MFMA_BLOCK_BOUND * max_k |a_k b_k| as the
instruction's accumulation model.  This test runs the instruction, through the library's
moe_check_mfma_blocks, on blocks built to stress it -- values with the spread of real
quantised rows, codes drawn over the whole e4m3 range, cancelling pairs with small
residues, one dominant product among tiny ones, and e2m1 weights with widely spread
UE8M0 exponents -- and compares each result with the fp64 sum of the exact products
(exact for e4m3 operands; for e2m1 its rounding is far below the bound).
"""

import numpy as np
import pytest
import torch

import mixture_experts_routed_topk_amd as m
from moe_helpers import MFMA_BLOCK_BOUND
from oracle.numerics import e2m1_decode, e4m3_decode, fp4_unpack, ue8m0_decode

pytestmark = pytest.mark.gpu

N = 2048      # blocks per operand set


def _e4m3(v):
    return torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_codes(rng, shape):
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    return rng.choice(finite, shape)


def _rows_like_quantised(rng, shape):
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.float32(448.0) / np.abs(x).max(axis=-1, keepdims=True)
    return _e4m3(x)


def _cancelling(rng):
    a = np.zeros((N, 16, 128), np.float32)
    for i in range(N):
        for r in range(16):
            npair = rng.integers(1, 24)
            ks = rng.choice(128, 2 * npair + rng.integers(1, 40), replace=False)
            v = 2.0 ** rng.integers(0, 8, npair) * rng.choice([1.0, 1.5, 1.75], npair)
            a[i, r, ks[:npair]] = v
            a[i, r, ks[npair:2 * npair]] = -v
            rest = ks[2 * npair:]
            a[i, r, rest] = 2.0 ** rng.integers(-9, 3, len(rest)) * rng.choice([1.0, -1.125, 1.625], len(rest))
    return _e4m3(a)


def _dominant(rng):
    a = np.zeros((N, 16, 128), np.float32)
    for i in range(N):
        for r in range(16):
            ks = rng.permutation(128)
            a[i, r, ks[0]] = 2.0 ** rng.integers(2, 8) * rng.choice([1.0, -1.25, 1.875])
            m_ = rng.integers(1, 128)
            a[i, r, ks[1:1 + m_]] = 2.0 ** rng.integers(-9, 0, m_) * rng.choice([1.0, -1.0, 1.5, -1.75], m_)
    return _e4m3(a)


def _worst_ratio(d, prod):
    exact = prod.sum(axis=-1)
    pmax = np.abs(prod).max(axis=-1)
    ok = pmax > 0
    assert np.isfinite(d).all()
    assert np.all(d[~ok] == 0)
    return float((np.abs(d.astype(np.float64) - exact)[ok] / pmax[ok]).max())


CASES = ["quantised_rows", "all_codes", "cancelling", "dominant"]


@pytest.mark.parametrize("case", CASES)
def test_e4m3_block_bound(case):
    rng = np.random.default_rng(CASES.index(case))
    if case == "quantised_rows":
        a, b = _rows_like_quantised(rng, (N, 16, 128)), _rows_like_quantised(rng, (N, 16, 128))
    elif case == "all_codes":
        a, b = _finite_codes(rng, (N, 16, 128)), _finite_codes(rng, (N, 16, 128))
    elif case == "cancelling":
        a, b = _cancelling(rng), np.full((N, 16, 128), 0x38, np.uint8)           # b = 1.0
    else:
        a, b = _dominant(rng), _rows_like_quantised(rng, (N, 16, 128))
    d = m.check_mfma_blocks(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()).cpu().numpy()
    av = e4m3_decode(a).reshape(a.shape)
    bv = e4m3_decode(b).reshape(b.shape)
    prod = av[:, :, None, :] * bv[:, None, :, :]              # exact in fp64
    r = _worst_ratio(d, prod)
    print(f"e4m3 {case}: max |mfma - exact| / max|product| = 2^{np.log2(max(r, 1e-300)):.2f}")
    assert r <= MFMA_BLOCK_BOUND


@pytest.mark.parametrize("spread", [(120, 135), (100, 150)])
def test_e4m3_e2m1_block_bound(spread):
    rng = np.random.default_rng(spread[1])
    a = _rows_like_quantised(rng, (N, 16, 128)) if spread[1] < 140 else _finite_codes(rng, (N, 16, 128))
    b = rng.integers(0, 256, (N, 16, 64), dtype=np.uint8)
    sb = rng.integers(spread[0], spread[1], (N, 16, 4)).astype(np.uint8)
    d = m.check_mfma_blocks(torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda(),
                            torch.from_numpy(sb).cuda()).cpu().numpy()
    av = e4m3_decode(a).reshape(a.shape)
    bv = e2m1_decode(fp4_unpack(b.reshape(-1, 64))).reshape(N, 16, 128) * np.repeat(ue8m0_decode(sb), 32, axis=2)
    prod = av[:, :, None, :] * bv[:, None, :, :]
    r = _worst_ratio(d, prod)
    print(f"e4m3 x e2m1 exponents {spread}: max |mfma - exact| / max|product| = 2^{np.log2(max(r, 1e-300)):.2f}")
    assert r <= MFMA_BLOCK_BOUND



@pytest.mark.parametrize("spread", [(120, 135), (100, 150)])
def test_e4m3_scaled_block_bound(spread):
    """e4m3 x e4m3 with one UE8M0 exponent on B for the whole block, passed by every lane:
    how the e4m3 kernels apply UE8M0 weight scales (a 128 x 128 weight block is one exponent).
    The result is the exact sum times 2^(s - 127) within the block bound, and bit for bit the
    unit-scale result times that power of two.  (Which lane's byte scales which column and
    32-block differs between the operand formats; with one exponent for the block it does not
    matter, and the kernels rely on nothing else.)"""
    rng = np.random.default_rng(spread[1] + 7)
    a = _rows_like_quantised(rng, (N, 16, 128))
    b = _rows_like_quantised(rng, (N, 16, 128)) if spread[1] < 140 else _finite_codes(rng, (N, 16, 128))
    s_blk = rng.integers(spread[0], spread[1], N).astype(np.uint8)
    sb = np.ascontiguousarray(np.broadcast_to(s_blk[:, None, None], (N, 16, 4)))
    ta, tb = torch.from_numpy(a).cuda(), torch.from_numpy(b).cuda()
    d = m.check_mfma_blocks(ta, tb, torch.from_numpy(sb).cuda()).cpu().numpy()
    d0 = m.check_mfma_blocks(ta, tb).cpu().numpy()
    scale = ue8m0_decode(s_blk).astype(np.float64)[:, None, None]
    av = e4m3_decode(a).reshape(a.shape)
    bv = e4m3_decode(b).reshape(b.shape)
    prod = av[:, :, None, :] * bv[:, None, :, :] * scale[..., None]   # exact in fp64
    r = _worst_ratio(d, prod)
    print(f"e4m3 x e4m3, block exponents {spread}: max |mfma - exact| / max|product| = 2^{np.log2(max(r, 1e-300)):.2f}")
    assert r <= MFMA_BLOCK_BOUND
    assert np.array_equal(d.astype(np.float64), d0.astype(np.float64) * scale)
