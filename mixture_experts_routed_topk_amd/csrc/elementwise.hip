// Small bandwidth-bound kernels around the grouped GEMMs: clearing the float32
// accumulator and writing the final output (the weighted sum of the k expert
// outputs of each token, rounded once to the output type).
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void zero_f32_kernel(float4* p, int64_t n4, float* tail, int ntail) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n4; i += stride)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0.f;
}

// 8 consecutive elements per thread-iteration; H % 8 == 0.
__global__ __launch_bounds__(kThreads) void finalize_acc_kernel(const float4* __restrict__ acc, void* out,
                                                                int64_t n8, int out_bf16) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    const float4 a = acc[2 * i], b = acc[2 * i + 1];
    if (out_bf16) {
      uint4 o;
      o.x = pack_bf16x2(a.x, a.y);
      o.y = pack_bf16x2(a.z, a.w);
      o.z = pack_bf16x2(b.x, b.y);
      o.w = pack_bf16x2(b.z, b.w);
      static_cast<uint4*>(out)[i] = o;
    } else {
      static_cast<float4*>(out)[2 * i] = a;
      static_cast<float4*>(out)[2 * i + 1] = b;
    }
  }
}

// 8 consecutive values of a slot row (float32 or bf16 bits) as float32
__device__ __forceinline__ void load8(const float* rows, int64_t at, float* v) {
  const float4* r = reinterpret_cast<const float4*>(rows + at);
  const float4 a = r[0], b = r[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* rows, int64_t at, float* v) {
  const uint4 q = *reinterpret_cast<const uint4*>(rows + at);
  v[0] = bf16_lo(q.x); v[1] = bf16_hi(q.x); v[2] = bf16_lo(q.y); v[3] = bf16_hi(q.y);
  v[4] = bf16_lo(q.z); v[5] = bf16_hi(q.z); v[6] = bf16_lo(q.w); v[7] = bf16_hi(q.w);
}

template <typename R>
__global__ __launch_bounds__(kThreads) void finalize_slots_kernel(const R* __restrict__ rows,
                                                                  const int32_t* __restrict__ inv, void* out,
                                                                  int64_t T, int k, int H, int out_bf16) {
  const int h8 = H / 8;
  const int64_t n8 = T * h8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n8; i += stride) {
    const int64_t t = i / h8;
    const int c = (int)(i - t * h8) * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // four slots at a time: their rows are loaded together (a dropped slot's row too, and
    // then not added), and added in slot order
    for (int j0 = 0; j0 < k; j0 += 4) {
      bool use[4];
      float v[4][8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) use[jj] = j0 + jj < k && inv[t * k + j0 + jj] >= 0;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) load8(rows, (t * k + min(j0 + jj, k - 1)) * H + c, v[jj]);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        if (use[jj]) {
#pragma unroll
          for (int q = 0; q < 8; ++q) s[q] += v[jj][q];
        }
    }
    if (out_bf16) {
      uint4 o;
      o.x = pack_bf16x2(s[0], s[1]);
      o.y = pack_bf16x2(s[2], s[3]);
      o.z = pack_bf16x2(s[4], s[5]);
      o.w = pack_bf16x2(s[6], s[7]);
      reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + t * H + c)[0] = o;
    } else {
      float4* o = reinterpret_cast<float4*>(static_cast<float*>(out) + t * H + c);
      o[0] = make_float4(s[0], s[1], s[2], s[3]);
      o[1] = make_float4(s[4], s[5], s[6], s[7]);
    }
  }
}

int grid_for(int64_t n) {
  const int64_t b = (n + kThreads - 1) / kThreads;
  return (int)(b < 1 ? 1 : (b > 8192 ? 8192 : b));
}

}  // namespace

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL(zero_f32_kernel, dim3(grid_for(n4)), dim3(kThreads), 0, s, reinterpret_cast<float4*>(p), n4,
                     p + n4 * 4, (int)(n - n4 * 4));
  return hipGetLastError();
}

hipError_t launch_finalize_acc(const float* acc, void* out, int64_t T, int H, int out_bf16, hipStream_t s) {
  const int64_t n8 = T * H / 8;
  hipLaunchKernelGGL(finalize_acc_kernel, dim3(grid_for(n8)), dim3(kThreads), 0, s,
                     reinterpret_cast<const float4*>(acc), out, n8, out_bf16);
  return hipGetLastError();
}

hipError_t launch_finalize_slots(const float* slot_rows, const int32_t* inv, void* out, int64_t T, int k, int H,
                                 int out_bf16, hipStream_t s) {
  const int64_t n8 = T * (H / 8);
  hipLaunchKernelGGL(finalize_slots_kernel<float>, dim3(grid_for(n8)), dim3(kThreads), 0, s, slot_rows, inv, out, T,
                     k, H, out_bf16);
  return hipGetLastError();
}

hipError_t launch_finalize_slots_bf16(const uint16_t* slot_rows, const int32_t* inv, void* out, int64_t T, int k,
                                      int H, int out_bf16, hipStream_t s) {
  const int64_t n8 = T * (H / 8);
  hipLaunchKernelGGL(finalize_slots_kernel<uint16_t>, dim3(grid_for(n8)), dim3(kThreads), 0, s, slot_rows, inv, out,
                     T, k, H, out_bf16);
  return hipGetLastError();
}

}  // namespace moe
