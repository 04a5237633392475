// Grouped GEMMs of the experts forward on bf16 MFMA (gfx950 v_mfma_f32_16x16x32_bf16).
//
// The Experts backends page (backend table, "grouped_mm" row) sorts the tokens by
// selected expert and projects them in one grouped GEMM; the expert is the gated
// MLP of the "deepgemm_megamoe" row and the "SonicMoE" section (up projection,
// SwiGLU, down projection).  Two kernels share one main loop:
//
//   gate_up : rows = hidden rows gathered through the sorted permutation,
//             B = W_gate_up[e] ([2I, H], K = H contiguous).  A 128-row B tile holds
//             64 gate rows and the 64 matching up rows, so the SwiGLU
//             a = silu(gate) * up is formed in registers and stored as bf16.
//   down    : rows = the SwiGLU rows (already in sorted order), B = W_down[e]
//             ([H, I], K = I contiguous).  The epilogue scales each row by its
//             routing weight and adds it into the token's float32 output row
//             (hardware float atomics), or stores it to the slot's own row for the
//             deterministic combine.
//
// Tiles: 128 x 128 x 64, 256 threads = 4 waves in a 2 x 2 grid, 64 x 64 per wave
// (4 x 4 MFMA fragments).  Operands are staged through LDS, double buffered, rows of
// 128 bytes with the 16-byte chunks XOR-swizzled by (row & 7) so that the fragment
// reads of 8 consecutive rows hit distinct banks.  The grid is persistent; work
// items are (expert, N tile, M tile) with M fastest, and each round hands every
// XCD (blockIdx % 8) a contiguous run of items, so the M tiles that share one
// weight tile run together on one XCD and meet in its L2.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kTileElems = 128 * BK;  // one operand tile in bf16 elements (16 KB)

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return row * BK + ((chunk ^ (row & 7)) << 3); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void grouped_bf16_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][kTileElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int n_items = g.mt[g.E] * g.NT;
  const int KT = g.K / BK;
  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.a);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(g.b);

  // loader mapping: chunk c of rows lr + 32 i
  const int lc = tid & 7, lr = tid >> 3;

  for (int base = 0; base < n_items; base += gridDim.x) {
    const int w = base + xcd * gx + xslot;
    if (w >= n_items) continue;
    const int e = find_group(g.mt, g.E, g.NT, w);
    const int mt_e = g.mt[e + 1] - g.mt[e];
    const int local = w - g.mt[e] * g.NT;
    const int nt = local / mt_e;
    const int mloc = local - nt * mt_e;
    const int row0 = g.offsets[e] + mloc * BM;
    const int rows = min(BM, g.offsets[e + 1] - row0);

    // global source pointers for this thread's 4 A rows and 4 B rows
    const uint16_t* pa[4];
    const uint16_t* pb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lr + 32 * i;
      const int p = row0 + min(r, rows - 1);  // rows past the tile end re-read the last row
      const int64_t src = g.a_rows ? (int64_t)(g.a_rows[p] / g.a_row_div) : (int64_t)p;
      pa[i] = A + src * g.lda + lc * 8;
      int grow;
      if (MODE == kGateUp) grow = (r < 64) ? nt * 64 + r : g.I + nt * 64 + (r - 64);
      else grow = nt * BN + r;
      pb[i] = B + (int64_t)e * g.b_expert_stride + (int64_t)grow * g.K + lc * 8;
    }

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    uint4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ra[i] = *reinterpret_cast<const uint4*>(pa[i]);
      rb[i] = *reinterpret_cast<const uint4*>(pb[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *reinterpret_cast<uint4*>(&sA[0][swz(lr + 32 * i, lc)]) = ra[i];
      *reinterpret_cast<uint4*>(&sB[0][swz(lr + 32 * i, lc)]) = rb[i];
    }
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ra[i] = *reinterpret_cast<const uint4*>(pa[i] + (kt + 1) * BK);
          rb[i] = *reinterpret_cast<const uint4*>(pb[i] + (kt + 1) * BK);
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 fa[4], fb[4];
        const int ch = s * 4 + (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 64 + i * 16 + (lane & 15);
          fa[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][swz(r, ch)]);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          int r;
          if (MODE == kGateUp) r = (j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16) + (lane & 15);
          else r = wn * 64 + j * 16 + (lane & 15);
          fb[j] = *reinterpret_cast<const bf16x8*>(&sB[cur][swz(r, ch)]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_16x16x32_bf16(fa[i], fb[j], acc[i][j]);
      }
      if (kt + 1 < KT) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          *reinterpret_cast<uint4*>(&sA[cur ^ 1][swz(lr + 32 * i, lc)]) = ra[i];
          *reinterpret_cast<uint4*>(&sB[cur ^ 1][swz(lr + 32 * i, lc)]) = rb[i];
        }
      }
      __syncthreads();
    }

    // epilogue; fragment (i, j) element q sits at tile row wm*64 + i*16 + 4*(lane>>4) + q,
    // tile column (lane & 15) of fragment j
    const int col_in = lane & 15;
    if (MODE == kGateUp) {
      uint16_t* out = static_cast<uint16_t*>(g.act_out);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + q;
          if (r < rows) {
            uint16_t* orow = out + (int64_t)(row0 + r) * g.I + nt * 64 + wn * 32 + col_in;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float gt = acc[i][j][q], up = acc[i][j + 2][q];
              orow[j * 16] = (uint16_t)f32_to_bf16_bits(silu_fast(gt) * up);
            }
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + q;
          if (r < rows) {
            const int slot = g.perm[row0 + r];
            const float wt = g.topk_w[slot];
            const int64_t colbase = (int64_t)nt * BN + wn * 64 + col_in;
            if (MODE == kDownAtomic) {
              float* orow = g.acc_out + (int64_t)(slot / g.k) * g.H + colbase;
#pragma unroll
              for (int j = 0; j < 4; ++j) unsafeAtomicAdd(orow + j * 16, wt * acc[i][j][q]);
            } else {
              float* orow = g.slot_out + (int64_t)slot * g.H + colbase;
#pragma unroll
              for (int j = 0; j < 4; ++j) orow[j * 16] = wt * acc[i][j][q];
            }
          }
        }
      }
    }
  }
}

}  // namespace

int gateup_bf16_bm() { return BM; }
int down_bf16_bm() { return BM; }

hipError_t launch_gateup_bf16(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL(grouped_bf16_kernel<kGateUp>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_down_bf16(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.slot_out) hipLaunchKernelGGL(grouped_bf16_kernel<kDownSlots>, dim3(grid), dim3(kThreads), 0, s, g);
  else hipLaunchKernelGGL(grouped_bf16_kernel<kDownAtomic>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
