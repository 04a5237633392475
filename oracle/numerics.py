"""Number formats used by the oracle, written from their definitions.

bf16  : IEEE-754 binary32 with the low 16 significand bits dropped (8 significant
        bits, same exponent range as fp32).
e4m3  : OCP 8-bit floating point, E4M3 ("e4m3fn"): bias 7, 3 fraction bits,
        subnormals below 2^-6 with quantum 2^-9, largest finite 448 (0x7E),
        0x7F / 0xFF are NaN, no infinities.
UE8M0 : unsigned 8-bit exponent-only scale, value 2^(b - 127), 0xFF is NaN.
e2m1  : OCP 4-bit floating point (the MX element type FP4): 1 sign, 2 exponent bits
        with bias 1, 1 fraction bit; exponent field 0 is subnormal (value m / 2);
        no infinities or NaN, largest magnitude 6.  Two codes per byte.

The Experts backends page ("FP8 and FP4 quantized experts" section and note) says
fp8 experts come with float32 or UE8M0 block scales and FP4 experts come packed two
codes per int8 with UE8M0 scales; these helpers decode all of them.
Rounding is round-to-nearest-even throughout, done with np.rint on values scaled
to an integer quantum (exact in fp64 for every case used here).
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bit patterns, one round-to-nearest-even step (no fp32 detour)."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    out = np.zeros(v.shape, dtype=np.float64)
    finite = np.isfinite(a) & (a > 0)
    af = a[finite]
    _, ex = np.frexp(af)                     # af = m * 2**ex, m in [0.5, 1)
    e = ex - 1                               # floor(log2 af)
    qe = np.maximum(e - 7, -133)             # quantum exponent (subnormal floor 2^-133)
    r = np.rint(np.ldexp(af, -qe))           # ties to even
    out[finite] = np.ldexp(r, qe)
    out[np.isinf(a)] = np.inf
    out[out >= 2.0 ** 128] = np.inf          # rounded past the largest finite bf16
    signed = np.where(np.signbit(v), -out, out)
    bits = (signed.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    bits[np.isnan(v)] = np.uint16(0x7FC0)
    return bits


def e4m3_value_table() -> np.ndarray:
    """fp64 value of each of the 256 e4m3 codes (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        ef = (code >> 3) & 0xF
        m = code & 0x7
        if ef == 0xF and m == 0x7:
            vals[code] = np.nan
        elif ef == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (ef - 7)
    return vals


_E4M3 = e4m3_value_table()


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


def f32_to_e4m3(v: np.ndarray) -> np.ndarray:
    """fp32 values -> e4m3 codes: round to nearest even, saturate at +-448, NaN -> 0x7F."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    mag = np.zeros(v.shape, dtype=np.float64)
    nz = (a > 0) & np.isfinite(a)
    _, ex = np.frexp(a[nz])
    qe = np.maximum(ex - 1 - 3, -9)          # 3 fraction bits; subnormal quantum 2^-9
    mag[nz] = np.ldexp(np.rint(np.ldexp(a[nz], -qe)), qe)
    mag = np.minimum(mag, E4M3_MAX)          # saturate (also catches +inf)
    mag[np.isinf(a)] = E4M3_MAX
    codes = np.zeros(v.shape, dtype=np.uint8)
    sub = mag < 2.0 ** -6
    codes[sub] = np.rint(mag[sub] / 2.0 ** -9).astype(np.uint8)  # 0..7
    nrm = ~sub
    _, ex = np.frexp(mag[nrm])
    e = ex - 1
    m = np.rint(np.ldexp(mag[nrm], -(e - 3))).astype(np.int64) - 8
    codes[nrm] = (((e + 7) << 3) | m).astype(np.uint8)
    codes |= np.where(np.signbit(v), np.uint8(0x80), np.uint8(0))
    codes[np.isnan(v)] = np.uint8(0x7F)
    return codes


def e2m1_value_table() -> np.ndarray:
    """fp64 value of each of the 16 e2m1 codes, from the bit fields."""
    vals = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        ef = (code >> 1) & 0x3
        m = code & 0x1
        if ef == 0:
            vals[code] = sign * (m / 2.0)                      # subnormal: 2^(1-1) * 0.m
        else:
            vals[code] = sign * (1.0 + m / 2.0) * 2.0 ** (ef - 1)
    return vals


_E2M1 = e2m1_value_table()


def fp4_unpack(packed: np.ndarray) -> np.ndarray:
    """Packed e2m1 bytes [..., C/2] -> codes [..., C]: byte j holds element 2j in its low
    nibble and element 2j + 1 in its high nibble."""
    b = np.asarray(packed, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = b & 0x0F
    out[..., 1::2] = b >> 4
    return out


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return _E2M1[np.asarray(codes, dtype=np.uint8) & 0x0F]


def ue8m0_decode(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.ldexp(1.0, b.astype(np.int64) - 127)
    return np.where(b == 0xFF, np.nan, out)


def f64_to_f32(v: np.ndarray) -> np.ndarray:
    """fp64 -> fp32, round to nearest even (IEEE conversion)."""
    return np.asarray(v, dtype=np.float64).astype(np.float32)
