// Epilogue of the e4m3 and e2m1 gate_up kernels: the gated activation of a tile's 128
// columns, quantised to e4m3 per row in registers.
//
// With fp8 and FP4 experts the activation rows entering the down projection carry dynamic
// per-row scales ("FP8 and FP4 quantized experts" section of the Experts backends page).
// Per row and per group of 128 consecutive columns: amax = max |a| over the group (float32),
// s = amax / 448 (float32, correctly rounded; 1 when the group is all zero), and each
// element becomes e4m3(a / s) (float32 division, round to nearest even, saturating).  A
// gate_up tile holds exactly one such group per row (128 SwiGLU columns, I % 128 == 0), so
// the group never leaves the workgroup: each wave reduces its 32 columns of a row across
// its 16 lanes and the four column waves meet in LDS; then each lane stores its codes
// straight from registers (the 16 lanes of a group write 16 consecutive bytes of a row of
// the [rows][I] code matrix; staging them in LDS for 16-byte stores measured 1-3% slower),
// with one float32 scale per row and tile in the [rows][I / 128] scale matrix.  The values
// quantised are the same float32 values a separate pass would read back, so the codes and
// scales are those of the row quantiser applied to them.  The gate runs on the hardware exp
// and reciprocal (gate_fn<true>): a few float32 ulps, far inside the accumulation error the
// block-scaled MFMA leaves in its input (2-3% faster gate_up than the libm exp and an IEEE
// division).
//
// Tile layout (shared by both kernels): 128 rows; wave (wm, wn) of the 2 x 4 grid holds,
// for row fragment i, rows (2 i + wm) * 16 + 4 g4 + q (q < 4, g4 = lane >> 4) and, in
// acc[i][j] (j < 2), gate columns 32 wn + 16 j + (lane & 15) with the matching up columns
// in acc[i][j + 2].
#pragma once

#include "device_common.h"

namespace moe {

constexpr int kActQRows = 128;          // tile rows
constexpr int kActQCols = 128;          // SwiGLU columns per tile (one scale group)
// LDS bytes the epilogue needs: the per-wave row maxima
constexpr int kActQLdsBytes = kActQRows * 4 * 4;

// Every wave of the 512-thread workgroup must call this (it holds a barrier), after a
// barrier that ends all reads of `lds`.  rows: valid tile rows; row0: the tile's first row
// in the code matrix; nt: the tile's column group; I: columns of the code matrix.
template <int MFRAG>
__device__ __forceinline__ void gateup_requant_epilogue(const f32x4 (&acc)[MFRAG][4], int gate, int wm, int wn,
                                                        int l16, int g4, int rows, int row0, int nt, int I,
                                                        char* lds, uint8_t* __restrict__ codes,
                                                        float* __restrict__ scales) {
  static_assert(2 * 16 * MFRAG == kActQRows, "two row waves of MFRAG 16-row fragments");
  float* sAmax = reinterpret_cast<float*>(lds);   // [row][wn]
  float v[MFRAG][4][2];
#pragma unroll
  for (int i = 0; i < MFRAG; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int j = 0; j < 2; ++j) v[i][q][j] = gate_fn<true>(gate, acc[i][j][q]) * acc[i][j + 2][q];
#pragma unroll
  for (int i = 0; i < MFRAG; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float m = fmaxf(fabsf(v[i][q][0]), fabsf(v[i][q][1]));
#pragma unroll
      for (int d = 1; d < 16; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
      const int r = (2 * i + wm) * 16 + 4 * g4 + q;
      if (l16 == 0) sAmax[r * 4 + wn] = m;
    }
  __syncthreads();
  const int gpr = I / kActQCols;
#pragma unroll
  for (int i = 0; i < MFRAG; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = (2 * i + wm) * 16 + 4 * g4 + q;
      const f32x4 mm = *reinterpret_cast<const f32x4*>(&sAmax[r * 4]);
      const float amax = fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3]));
      const float s = amax > 0.f ? amax / 448.0f : 1.0f;   // correctly rounded division
      if (r < rows) {
        uint8_t* o = codes + (int64_t)(row0 + r) * I + nt * kActQCols + 32 * wn + l16;
#pragma unroll
        for (int j = 0; j < 2; ++j) o[16 * j] = (uint8_t)f32_to_e4m3(v[i][q][j] / s);
        if (wn == 0 && l16 == 0) scales[(int64_t)(row0 + r) * gpr + nt] = s;
      }
    }
}

}  // namespace moe
