// Instruction check: single 16x16x128 block products on the block-scaled MFMA the e4m3 and
// e2m1 grouped kernels use, with the operand layout those kernels use and a zero
// accumulator, so the instruction's accumulation can be compared with exact sums.
//
// One wave per block.  Block b of `a` is [16][128] e4m3 codes (row r, k contiguous).
// fmt 0: block b of `b` is [16][128] e4m3 codes (row = output column n, k contiguous);
// fmt 1: [16][64] bytes of e2m1 codes (element k in the low nibble of byte k / 2 when k is
// even) with one UE8M0 exponent per column and 32-long k block in b_scale [16][4];
// fmt 2: e4m3 codes as for fmt 0 with the UE8M0 exponent byte b_scale[16][4] of lane
// (column, k block) passed as that lane's B scale (the e4m3 kernels with UE8M0 weight
// scales pass one exponent for the whole block; which lane's byte scales which column and
// block is the instruction's, and only a uniform exponent has a format-independent meaning).
// d[b][r][n] = sum_k a[r][k] * b[n][k] (fmt 1: times 2^(s - 127) per 32-block; fmt 2 with
// one exponent s for the block: times 2^(s - 127)).
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

__global__ __launch_bounds__(64) void mfma_block_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                        const uint8_t* __restrict__ b_scale, float* __restrict__ d,
                                                        int nblocks, int fmt) {
  const int blk = blockIdx.x;
  if (blk >= nblocks) return;
  const int l = threadIdx.x, l16 = l & 15, g = l >> 4;
  const uint8_t* arow = a + (int64_t)blk * 2048 + l16 * 128;
  f32x4 r;
  if (fmt == 0 || fmt == 2) {
    // e4m3 x e4m3: both lanes hold k 32 g .. 32 g + 31 of their row
    const i32x4 a0 = *reinterpret_cast<const i32x4*>(arow + 32 * g);
    const i32x4 a1 = *reinterpret_cast<const i32x4*>(arow + 32 * g + 16);
    const uint8_t* brow = b + (int64_t)blk * 2048 + l16 * 128;
    const i32x4 b0 = *reinterpret_cast<const i32x4*>(brow + 32 * g);
    const i32x4 b1 = *reinterpret_cast<const i32x4*>(brow + 32 * g + 16);
    const i32x8 av = i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const i32x8 bv = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
    if (fmt == 0) r = mfma_16x16x128_e4m3(av, bv, f32x4{});
    else   // the lane's UE8M0 byte as its B scale
      r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, f32x4{}, 0, 0, 0, 127, 0,
                                                           (int)b_scale[(int64_t)blk * 64 + l16 * 4 + g]);
  } else {
    // e4m3 x e2m1: A lane holds k 16 g .. 16 g + 15 and 64 + 16 g .. 64 + 16 g + 15, B lane
    // k 32 g .. 32 g + 31 (the pairing the hardware uses for the two formats)
    const i32x4 a0 = *reinterpret_cast<const i32x4*>(arow + 16 * g);
    const i32x4 a1 = *reinterpret_cast<const i32x4*>(arow + 64 + 16 * g);
    const i32x4 bb = *reinterpret_cast<const i32x4*>(b + (int64_t)blk * 1024 + l16 * 64 + 16 * g);
    const int sb = b_scale[(int64_t)blk * 64 + l16 * 4 + g];
    r = mfma_16x16x128_e4m3_e2m1(i32x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]}, bb, sb);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) d[(int64_t)blk * 256 + (4 * g + q) * 16 + l16] = r[q];
}

}  // namespace

hipError_t launch_mfma_block_check(const uint8_t* a, const uint8_t* b, const uint8_t* b_scale, float* d, int nblocks,
                                   int fmt, hipStream_t s) {
  hipLaunchKernelGGL(mfma_block_kernel, dim3(nblocks), dim3(64), 0, s, a, b, b_scale, d, nblocks, fmt);
  return hipGetLastError();
}

}  // namespace moe
