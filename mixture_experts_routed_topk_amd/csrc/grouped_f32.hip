// fp32 grouped GEMMs of the experts forward (fp32 hidden states and weights).
//
// Same two steps as the bf16 kernels -- gate/up projection with the SwiGLU fused
// into the epilogue, then the down projection with the routing-weight scale and
// the scatter-add into the token rows -- computed with plain fp32 FMAs (no lower
// precision anywhere), in 64-row tiles staged through LDS.  This path serves small
// fp32 layers, where the call is launch-latency bound.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 64, BK = 32, kThreads = 256;
constexpr int BNG = 32;   // gate_up: SwiGLU columns per tile (32 gate + 32 up weight rows)
constexpr int BND = 64;   // down: output columns per tile

struct Item {
  int e, nt, row0, rows;
};

__device__ __forceinline__ bool decode_item(const GroupedArgs& g, int w, Item& it) {
  if (w >= g.mt[g.E] * g.NT) return false;
  it.e = find_group(g.mt, g.E, g.NT, w);
  const int mt_e = g.mt[it.e + 1] - g.mt[it.e];
  const int local = w - g.mt[it.e] * g.NT;
  it.nt = local / mt_e;
  const int mloc = local - it.nt * mt_e;
  it.row0 = g.offsets[it.e] + mloc * BM;
  it.rows = min(BM, g.offsets[it.e + 1] - it.row0);
  return true;
}

__global__ __launch_bounds__(kThreads) void gateup_f32_kernel(GroupedArgs g) {
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[2 * BNG][BK + 1];
  Item it;
  if (!decode_item(g, blockIdx.x, it)) return;
  const float* __restrict__ A = static_cast<const float*>(g.a);
  const float* __restrict__ Bw = static_cast<const float*>(g.b) + (int64_t)it.e * g.b_expert_stride;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float gt[4][2] = {}, up[4][2] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    for (int i = threadIdx.x; i < BM * BK; i += kThreads) {
      const int r = i / BK, c = i % BK;
      const int p = it.row0 + min(r, it.rows - 1);
      const int64_t src = g.a_rows ? (int64_t)(g.a_rows[p] / g.a_row_div) : (int64_t)p;
      sA[r][c] = A[src * g.lda + k0 + c];
    }
    for (int i = threadIdx.x; i < 2 * BNG * BK; i += kThreads) {
      const int r = i / BK, c = i % BK;
      const int grow = r < BNG ? it.nt * BNG + r : g.I + it.nt * BNG + (r - BNG);
      sB[r][c] = Bw[(int64_t)grow * g.K + k0 + c];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = sA[ty + 16 * i][kk];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          gt[i][j] = fmaf(a, sB[tx + 16 * j][kk], gt[i][j]);
          up[i][j] = fmaf(a, sB[BNG + tx + 16 * j][kk], up[i][j]);
        }
      }
    }
    __syncthreads();
  }
  float* out = static_cast<float*>(g.act_out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    if (r < it.rows) {
#pragma unroll
      for (int j = 0; j < 2; ++j)
        out[(int64_t)(it.row0 + r) * g.I + it.nt * BNG + tx + 16 * j] = gate_fn<false>(g.gate, gt[i][j]) * up[i][j];
    }
  }
}

template <bool SLOTS>
__global__ __launch_bounds__(kThreads) void down_f32_kernel(GroupedArgs g) {
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BND][BK + 1];
  Item it;
  if (!decode_item(g, blockIdx.x, it)) return;
  const float* __restrict__ A = static_cast<const float*>(g.a);
  const float* __restrict__ Bw = static_cast<const float*>(g.b) + (int64_t)it.e * g.b_expert_stride;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < g.K; k0 += BK) {
    for (int i = threadIdx.x; i < BM * BK; i += kThreads) {
      const int r = i / BK, c = i % BK;
      const int p = it.row0 + min(r, it.rows - 1);
      sA[r][c] = A[(int64_t)p * g.lda + k0 + c];
    }
    for (int i = threadIdx.x; i < BND * BK; i += kThreads) {
      const int r = i / BK, c = i % BK;
      sB[r][c] = Bw[(int64_t)(it.nt * BND + r) * g.K + k0 + c];
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < BK; ++kk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = sA[ty + 16 * i][kk];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a, sB[tx + 16 * j][kk], acc[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    if (r < it.rows) {
      const int slot = g.perm[it.row0 + r];
      const float wt = g.topk_w[slot];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = (int64_t)it.nt * BND + tx + 16 * j;
        if (SLOTS) g.slot_out[(int64_t)slot * g.H + col] = wt * acc[i][j];
        else unsafeAtomicAdd(g.acc_out + (int64_t)(slot / g.k) * g.H + col, wt * acc[i][j]);
      }
    }
  }
}

}  // namespace

int gateup_f32_bm() { return BM; }
int down_f32_bm() { return BM; }

hipError_t launch_gateup_f32(const GroupedArgs& g, int64_t max_items, hipStream_t s) {
  hipLaunchKernelGGL(gateup_f32_kernel, dim3((unsigned)max_items), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_down_f32(const GroupedArgs& g, int64_t max_items, hipStream_t s) {
  if (g.slot_out) hipLaunchKernelGGL(down_f32_kernel<true>, dim3((unsigned)max_items), dim3(kThreads), 0, s, g);
  else hipLaunchKernelGGL(down_f32_kernel<false>, dim3((unsigned)max_items), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
