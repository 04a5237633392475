// fp32 grouped GEMMs of the experts forward (fp32 hidden states and weights).
//
// Same two steps as the bf16 kernels -- gate/up projection with the SwiGLU fused
// into the epilogue, then the down projection with the routing-weight scale and
// the scatter-add into the token rows -- computed with plain fp32 FMAs (no lower
// precision anywhere), in 64-row tiles staged through LDS.  This path serves small
// fp32 layers, where the call is bound by memory latency and launches.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 64, BK = 64, kThreads = 256;
constexpr int BNG = 32;   // gate_up: SwiGLU columns per tile (32 gate + 32 up weight rows)
constexpr int BND = 64;   // down: output columns per tile
constexpr int BR = 64;    // weight rows per tile (gate_up: 2 BNG; down: BND)
constexpr int LPT = BM * BK / kThreads;   // elements of each operand tile a thread loads (16)

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

// C[BM x 64] = A_tile . W_tile^T over K, both tiles staged through LDS.  Source rows of
// the A tile are looked up once per item; the next K tile's loads are issued into
// registers before the current one is multiplied, so each K tile costs one memory
// latency at most.  Thread (tx, ty) accumulates rows ty + 16 i and columns tx + 16 j.
template <typename WRow>
__device__ __forceinline__ void tile_gemm(const GroupedArgs& g, const Item& it, WRow wrow, float (*sA)[BK + 1],
                                          float (*sB)[BK + 1], int64_t* sSrc, float acc[4][4]) {
  const float* __restrict__ A = static_cast<const float*>(g.a);
  const float* __restrict__ Bw = static_cast<const float*>(g.b) + (int64_t)it.e * g.b_expert_stride;
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  if (tid < BM) {
    const int p = it.row0 + min(tid, it.rows - 1);
    sSrc[tid] = (g.a_rows ? (int64_t)(g.a_rows[p] / g.a_row_div) : (int64_t)p) * g.lda;
  }
  __syncthreads();
  // element i of a thread: tile row (tid + kThreads i) / BK, column (tid + kThreads i) % BK
  int64_t aoff[LPT], boff[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    const int e = tid + kThreads * i, r = e / BK, c = e % BK;
    aoff[i] = sSrc[r] + c;
    boff[i] = (int64_t)wrow(r) * g.K + c;
  }
  float ra[LPT], rb[LPT];
#pragma unroll
  for (int i = 0; i < LPT; ++i) {
    ra[i] = A[aoff[i]];
    rb[i] = Bw[boff[i]];
  }
  for (int k0 = 0; k0 < g.K; k0 += BK) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int e = tid + kThreads * i;
      sA[e / BK][e % BK] = ra[i];
      sB[e / BK][e % BK] = rb[i];
    }
    __syncthreads();
    if (k0 + BK < g.K) {
#pragma unroll
      for (int i = 0; i < LPT; ++i) {
        ra[i] = A[aoff[i] + k0 + BK];
        rb[i] = Bw[boff[i] + k0 + BK];
      }
    }
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
}

__global__ __launch_bounds__(kThreads) void gateup_f32_kernel(GroupedArgs g) {
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BR][BK + 1];
  __shared__ int64_t sSrc[BM];
  Item it;
  if (!decode_item(g, blockIdx.x, it)) return;
  // tile rows 0..31: gate rows of SwiGLU columns nt BNG + 0..31; rows 32..63: their up rows
  auto wrow = [&](int r) { return r < BNG ? it.nt * BNG + r : g.I + it.nt * BNG + (r - BNG); };
  float acc[4][4] = {};
  tile_gemm(g, it, wrow, sA, sB, sSrc, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float* out = static_cast<float*>(g.act_out);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty + 16 * i;
    if (r < it.rows) {
      // columns tx + 16 j: j = 0, 1 gate rows, j = 2, 3 the matching up rows
#pragma unroll
      for (int j = 0; j < 2; ++j)
        out[(int64_t)(it.row0 + r) * g.I + it.nt * BNG + tx + 16 * j] = gate_fn<false>(g.gate, acc[i][j]) * acc[i][j + 2];
    }
  }
}

template <bool SLOTS>
__global__ __launch_bounds__(kThreads) void down_f32_kernel(GroupedArgs g) {
  __shared__ float sA[BM][BK + 1];
  __shared__ float sB[BR][BK + 1];
  __shared__ int64_t sSrc[BM];
  Item it;
  if (!decode_item(g, blockIdx.x, it)) return;
  auto wrow = [&](int r) { return it.nt * BND + r; };
  float acc[4][4] = {};
  tile_gemm(g, it, wrow, sA, sB, sSrc, acc);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
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
