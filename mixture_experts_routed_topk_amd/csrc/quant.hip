// Dynamic per-row e4m3 quantisation of the hidden states (fp8 and fp4 experts; the SwiGLU
// rows are quantised the same way inside the gate_up kernels, act_quant_epilogue.h).
//
// The Experts backends page ("FP8 and FP4 quantized experts" section) requires
// dynamic activation scales per row and rejects static per-tensor scales.  Here each
// row is split into groups of 128 consecutive columns; a group's scale is
// amax / 448 (float32, correctly rounded; 1 when the group is all zero) and every
// element becomes e4m3(x / scale) (float32 division, round to nearest even,
// saturating).  The largest element of a group therefore lands on +-448.
//
// 16 lanes cover one group (8 elements each); the group maximum is reduced with
// lane shuffles inside those 16 lanes.  Memory-bound: one read of the input, one
// write of the codes and of one float per group.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void quant_rows_kernel(const void* __restrict__ x, int64_t groups, int cols,
                                                              uint8_t* __restrict__ q, float* __restrict__ scales) {
  const int sub = threadIdx.x & 15;                       // lane within the group
  const int64_t gpb = kThreads / 16;                      // groups per block pass
  const int gpr = cols / 128;                             // groups per row
  for (int64_t grp = (int64_t)blockIdx.x * gpb + (threadIdx.x >> 4); grp < groups;
       grp += (int64_t)gridDim.x * gpb) {
    // all 16 lanes of a group share grp, so the loop exit is uniform per group
    const int64_t row = grp / gpr;
    const int64_t col = (grp - row * gpr) * 128 + sub * 8;
    const int64_t at = row * cols + col;
    float v[8];
    const i32x4 raw = *reinterpret_cast<const i32x4*>(static_cast<const uint16_t*>(x) + at);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = bf16_lo((uint32_t)raw[i]);
      v[2 * i + 1] = bf16_hi((uint32_t)raw[i]);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 16));
    const float s = amax > 0.f ? amax / 448.0f : 1.0f;    // correctly rounded division
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      lo |= f32_to_e4m3(v[i] / s) << (8 * i);
      hi |= f32_to_e4m3(v[4 + i] / s) << (8 * i);
    }
    *reinterpret_cast<uint2*>(q + at) = make_uint2(lo, hi);
    if (sub == 0) scales[grp] = s;
  }
}

int grid_for(int64_t groups) {
  const int64_t b = (groups + 15) / 16;
  return (int)(b < 1 ? 1 : (b > 16384 ? 16384 : b));
}

}  // namespace

hipError_t launch_quant_rows_bf16(const void* x, int64_t rows, int cols, uint8_t* q, float* scales, hipStream_t s) {
  const int64_t groups = rows * (cols / 128);
  hipLaunchKernelGGL(quant_rows_kernel, dim3(grid_for(groups)), dim3(kThreads), 0, s, x, groups, cols, q,
                     scales);
  return hipGetLastError();
}

}  // namespace moe
