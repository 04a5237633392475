// Device-side helpers shared by the HIP kernels of the experts forward (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16 bits, round to nearest even (gfx950's v_cvt_pk_bf16_f32; a NaN stays a
// quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// ---------------------------------------------------------------------------- e4m3
// OCP E4M3 ("e4m3fn"): bias 7, 3 fraction bits, subnormal quantum 2^-9, largest
// finite 448 (0x7E), 0x7F NaN, no infinity.  Round to nearest even, saturating.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;                  // NaN
  if (a >= 0x43e80000u) return sign | 0x7eu;          // |v| >= 464 (or inf): saturate
  if (a < 0x3c800000u) {                              // |v| < 2^-6: subnormal range
    const float f = __uint_as_float(a) * 512.0f;      // exact power-of-two scaling
    return sign | (uint32_t)__builtin_rintf(f);       // 0..8 (8 is the smallest normal)
  }
  const uint32_t r = a + 0x7ffffu + ((a >> 20) & 1u); // RNE at fraction bit 20
  const uint32_t e = (r >> 23) - 127u + 7u;           // biased e4m3 exponent, 1..15
  return sign | (e << 3) | ((r >> 20) & 7u);
}

// ---------------------------------------------------------------------------- math

__device__ __forceinline__ float silu_fast(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_exact(float z) { return z / (1.0f + expf(-z)); }
// GELU in its exact form z * Phi(z) = z / 2 * erfc(-z / sqrt 2) (erfc keeps the far negative
// tail accurate), and ReLU: the gates of GeGLU and ReGLU
__device__ __forceinline__ float gelu_exact(float z) { return 0.5f * z * erfcf(-0.70710678118654752f * z); }
__device__ __forceinline__ float relu_gate(float z) { return z > 0.0f ? z : 0.0f; }

// The gate function of the gated activation a = gate(g) * u: SwiGLU (silu, the default),
// GeGLU (gelu) or ReGLU (relu).  FAST: silu on the hardware exp and reciprocal (a few float32
// ulps from the exact quotient, where the libm exp and an IEEE division cost about three times
// the instructions): for bf16 results and for the e4m3 requantization of the SwiGLU rows,
// whose float32 input already carries the block-scaled MFMA's accumulation error.
enum { kGateSilu = 0, kGateGelu = 1, kGateRelu = 2 };
template <bool FAST>
__device__ __forceinline__ float gate_fn(int gate, float z) {
  if (gate == kGateGelu) return gelu_exact(z);
  if (gate == kGateRelu) return relu_gate(z);
  return FAST ? silu_fast(z) : silu_exact(z);
}

// ---------------------------------------------------------------------------- MFMA

// C[16x16] += A[16x32] * B[32x16]; lane l holds A row (l & 15) and B column (l & 15),
// eight consecutive k of group (l >> 4); C: column (l & 15), rows 4*(l >> 4) + i.
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C[32x32] += A[32x16] * B[16x32]; lane l holds A row (l & 31) and B column (l & 31),
// eight consecutive k of group (l >> 5); C element r of lane l sits at column (l & 31),
// row 8*(r/4) + 4*(l >> 5) + (r % 4).
__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// C[16x16] += A[16x128] * B[128x16] with e4m3 operands (32 bytes per lane), unit
// block scales (E8M0 exponent 127 = 2^0 on both sides).
__device__ __forceinline__ f32x4 mfma_16x16x128_e4m3(i32x8 a, i32x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// C[16x16] = A[16x128] * B[128x16], A in e4m3 (32 bytes per lane, unit scale) and B in
// e2m1 (16 bytes per lane).  With g = l >> 4, lane l holds B column (l & 15) and k 32 g ..
// 32 g + 31 in nibble order (element 2j in the low nibble of byte j), and A row (l & 15)
// with k 16 g .. 16 g + 15 in its first 16 bytes and k 64 + 16 g .. 64 + 16 g + 15 in its
// last 16 (measured on gfx950 by one-hot operands; the two formats split k differently).
// B is scaled per 32-k block by 2^(s - 127), s = the low byte of `scale_b` of the lane
// holding that column and block.
__device__ __forceinline__ f32x4 mfma_16x16x128_e4m3_e2m1(i32x8 a, i32x4 b, int scale_b) {
  const i32x8 b8 = {b[0], b[1], b[2], b[3], 0, 0, 0, 0};   // (only the low four are read)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b8, f32x4{}, 0, 4, 0, 127, 0, scale_b);
}

// C[32x32] += A[32x64] * B[64x32] with e4m3 operands (32 bytes per lane: lane l holds
// A row / B column (l & 31) and 32 k of group (l >> 5)), unit block scales.
__device__ __forceinline__ f32x16 mfma_32x32x64_e4m3(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// ---------------------------------------------------------------------------- LDS DMA
// Global -> LDS loads that bypass the registers.  One instruction per wave: lane L
// reads `base + off` and its data lands at LDS byte address m0 + 16 L (dwordx4) or
// m0 + 4 L (dword; ubyte zero-extended to a dword).  `base` and `m0` are wave-uniform.
// The compiler does not count these loads: every reader of the data waits for them
// with wait_vmcnt<N>() (at most N vector-memory operations of this wave outstanding,
// which retire in issue order) followed by a workgroup barrier.
//
// The compiler's hazard checks do not look inside inline asm, so each load carries its
// own wait states: on the gfx9 family a VMEM instruction that reads an SGPR written by
// a VALU instruction (v_readlane / v_readfirstlane, as when the compiler restores a
// spilled SGPR) needs 5 wait states, and an LDS DMA needs 1 after an SALU write of M0.
// Without them the load can use a stale base address.  s_nop 4 provides 5.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}
__device__ __forceinline__ void dma_lds_x4(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma_lds_x1(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma_lds_u8(const void* base, uint32_t off, uint32_t m0) {
  asm volatile("s_nop 4\n\tglobal_load_lds_ubyte %0, %1" ::"v"(off), "s"(base), "{m0}"(m0) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// ---------------------------------------------------------------------------- misc

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Work item `local` of one expert's mt_e x NT tiles -> (N tile nt, M tile m).  The items go
// in blocks of mb M tiles x nb N tiles (nb = 32 / mb, the workgroups of one XCD in one
// round), M fastest inside a block, the blocks of a group of mb M tiles in N order, the
// groups in M order; the last group and block may be smaller.  The tiles that run together
// on one XCD then share mb row tiles and nb weight tiles in its L2 instead of one weight
// tile and 32 row tiles.  mb <= 0: M fastest over the whole expert (nt = local / mt_e).
__host__ __device__ __forceinline__ void blocked_tile(int local, int mt_e, int NT, int mb, int& nt, int& m) {
  if (mb <= 0) {
    nt = local / mt_e;
    m = local - nt * mt_e;
    return;
  }
  const int nb = mb >= 32 ? 1 : 32 / mb;
  const int full = mt_e / mb;                  // groups of exactly mb M tiles
  int mg = local / (mb * NT);
  const int msz = mg < full ? mb : mt_e - full * mb;
  if (mg > full) mg = full;
  const int l2 = local - mg * mb * NT;         // index inside the group, [0, msz * NT)
  const int nbk = l2 / (msz * nb);             // block of nb N tiles (the last may be short)
  const int l3 = l2 - nbk * msz * nb;
  nt = nbk * nb + l3 / msz;
  m = mg * mb + l3 % msz;
}

// Largest e in [0, E) with start[e] * nt <= w (start is non-decreasing, start[E] * nt > w).
__device__ __forceinline__ int find_group(const int32_t* __restrict__ start, int E, int nt, int w) {
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (start[mid] * nt <= w) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace moe
