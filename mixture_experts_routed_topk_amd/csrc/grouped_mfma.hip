// Grouped GEMMs of the experts forward on MFMA (gfx950).
//
// The Experts backends page (backend table, "grouped_mm" row) sorts the tokens by
// selected expert and projects them in one grouped GEMM; the expert is the gated
// MLP of the "deepgemm_megamoe" row and the "SonicMoE" section (up projection,
// SwiGLU, down projection).  Two kernels share one main loop:
//
//   gate_up : rows = hidden rows gathered through the sorted permutation, weights
//             W_gate_up[e] ([2I, H], K = H contiguous).  The weight tile holds gate
//             rows and the matching up rows, and every wave owns both halves of its
//             columns, so a = silu(gate) * up is formed in registers and stored as bf16.
//   down    : rows = the SwiGLU rows (already in sorted order), weights W_down[e]
//             ([H, I], K = I contiguous).  The epilogue scales each row by its
//             routing weight and adds it into the token's float32 output row
//             (hardware float atomics), or stores it to the slot's own row for the
//             deterministic combine.
//
// Tiling: one 512-thread block per CU (8 waves, two per SIMD, so one wave's LDS waits are
// covered by the other's MFMAs) computes a 256-row x BN-column tile; the waves form a
// 2 x 4 grid of 128 x BN/4 wave tiles built from 32 x 32 MFMA fragments.  The K loop
// runs over 64-byte slices of both operands (32 bf16 elements) held in a
// 4-stage LDS ring that is filled by global->LDS DMA (no staging registers): three
// slices are in flight while the fourth is multiplied, and one barrier per slice both
// publishes the oldest slice and frees the slot the next DMA writes.  In each slot a
// tile row is 64 bytes whose four 16-byte chunks are XOR-permuted by (row >> 1) & 3, so
// the 8 rows read by each 8-lane group of a fragment load cover all 32 banks.  Per CU
// this moves (256 + BN) * 64 bytes of operands per slice.  An expert's rows are split
// evenly over its M tiles (multiples of 32 rows, at most 256) and row fragments past the
// end of a tile are not multiplied.  The grid is persistent; work items are (expert,
// N tile, M tile) with M fastest, and each round hands every XCD (blockIdx % 8) a
// contiguous run of items, so the M tiles sharing a weight tile run at the same pace on
// one XCD and meet in its L2.
//
// Operands are bf16 on the 32x32x16 MFMA (measured on MI355X: v_mfma_f32_32x32x16_bf16
// sustains 89% of the bf16 peak, the 16x16x32 form half of it), BN = 256 (wave tile
// 128 x 64: 4 x 2 fragments).  The e4m3 experts have their own kernels.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;   // 8 waves: 2 (rows) x 4 (columns)
constexpr int BM = 256;         // tile rows
constexpr int BN = 256;         // tile columns (= weight rows)
constexpr int WM = 128;         // wave tile rows (4 fragments of 32)
constexpr int WN = BN / 4;      // wave tile columns (2 fragments of 32)
constexpr int MFRAG = WM / 32;
constexpr int NFRAG = WN / 32;
constexpr int KS = 32;          // K elements per slice
constexpr int ROWB = KS * 2;    // LDS bytes of one tile row in one ring slot
constexpr int NSTAGE = 4;       // ring depth
constexpr int STAGE = (BM + BN) * ROWB;  // bytes of one ring slot: A rows, then B rows
constexpr int ALD = BM / 16 / 8;         // A DMA instructions per wave per slice (16 rows each)
constexpr int BLD = BN / 16 / 8;         // B DMA instructions per wave per slice
constexpr int NLD = ALD + BLD;           // vector-memory instructions per wave per slice

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_mfma_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char ring[NSTAGE][STAGE];
  __shared__ int sTok[BM];    // epilogue: token (atomic combine) or slot (per-slot rows)
  __shared__ float sWt[BM];   // epilogue: routing weight

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int hgrp = lane >> 5, r32 = lane & 31;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int n_items = g.mt[g.E] * g.NT;
  const int KT = g.K / KS;
  const int ncols = MODE == kGateUp ? g.I : g.H;     // output columns of the whole GEMM
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const uint32_t a_row_bytes = (uint32_t)(g.lda * 2);
  const uint32_t b_row_bytes = (uint32_t)(g.K * 2);

  // DMA lane L fills LDS chunk slot (L & 3) of tile row 16 b + (L >> 2) with the row's
  // global chunk (L & 3) ^ ((row >> 1) & 3); (row >> 1) & 3 == (L >> 3) & 3 here
  const int ld_row = lane >> 2;
  const uint32_t ld_chunk = (uint32_t)((((lane & 3) ^ ((lane >> 3) & 3))) << 4);
  const uint32_t ring0 = lds_addr(&ring[0][0]);

  // fragment reads (32x32x16, k step s): lane reads tile row base + r32 (base a multiple
  // of 32), chunk c = 2 s + hgrp (8 bf16), at row * ROWB + ((c ^ ((row >> 1) & 3)) << 4),
  // and (row >> 1) & 3 == (lane >> 1) & 3
  uint32_t foff[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) foff[s] = (uint32_t)(r32 * ROWB + (((2 * s + hgrp) ^ ((lane >> 1) & 3)) << 4));

  // first tile row of this wave's fragment j inside the weight tile (gate/up: fragment 0
  // holds gate rows, fragment 1 the matching up rows)
  auto b_frag_row = [&](int j) __attribute__((always_inline)) -> int {
    if (MODE == kGateUp) return (j == 0 ? 0 : BN / 2) + wn * (WN / 2);
    return wn * WN + j * 32;
  };

  for (int base = 0; base < n_items; base += gridDim.x) {
    const int w = base + xcd * gx + xslot;
    if (w >= n_items) continue;
    const int e = find_group(g.mt, g.E, g.NT, w);
    const int mt_e = g.mt[e + 1] - g.mt[e];
    const int local = w - g.mt[e] * g.NT;
    const int nt = local / mt_e;
    const int mloc = local - nt * mt_e;
    // the expert's rows split evenly over its M tiles (multiples of 32 rows), so tiles that
    // share a weight tile advance at the same pace and meet in L2
    const int cnt = g.offsets[e + 1] - g.offsets[e];
    const int per = min(BM, ((cnt + mt_e - 1) / mt_e + 31) & ~31);
    const int row0 = g.offsets[e] + mloc * per;
    const int rows = min(per, g.offsets[e + 1] - row0);
    if (rows <= 0) continue;
    const char* __restrict__ Bexp = static_cast<const char*>(g.b) + (int64_t)e * g.b_expert_stride * 2;

    // global weight row of tile row r; rows past the matrix repeat its last valid row
    auto b_row = [&](int r) __attribute__((always_inline)) -> int {
      if (MODE == kGateUp) {
        const int c = min(nt * (BN / 2) + (r % (BN / 2)), g.I - 1);
        return r < BN / 2 ? c : g.I + c;
      }
      return min(nt * BN + r, g.H - 1);
    };
    auto a_src = [&](int r) __attribute__((always_inline)) -> int {   // source row of tile row r
      const int p = row0 + min(r, rows - 1);                          // (rows past the end repeat the last)
      return g.a_rows ? g.a_rows[p] / g.a_row_div : p;
    };

    // 32-bit byte offsets of this lane's DMA sources (operands are < 4 GiB, checked on the host)
    uint32_t aoff[ALD], boff[BLD];
#pragma unroll
    for (int i = 0; i < ALD; ++i)
      aoff[i] = (uint32_t)a_src(16 * (wave + 8 * i) + ld_row) * a_row_bytes + ld_chunk;
#pragma unroll
    for (int i = 0; i < BLD; ++i)
      boff[i] = (uint32_t)b_row(16 * (wave + 8 * i) + ld_row) * b_row_bytes + ld_chunk;
    if (MODE != kGateUp && tid < rows) {
      const int slot = g.perm[row0 + tid];
      sTok[tid] = MODE == kDownAtomic ? slot / g.k : slot;
      sWt[tid] = g.topk_w[slot];
    }

    // DMA of K slice kt into ring slot kt % NSTAGE
    auto issue = [&](int kt) __attribute__((always_inline)) {
      const uint32_t st = ring0 + (uint32_t)((kt & (NSTAGE - 1)) * STAGE);
      const char* ab = Abase + (int64_t)kt * ROWB;
      const char* bb = Bexp + (int64_t)kt * ROWB;
#pragma unroll
      for (int i = 0; i < ALD; ++i) dma_lds_x4(ab, aoff[i], st + (uint32_t)((wave + 8 * i) * 1024));
#pragma unroll
      for (int i = 0; i < BLD; ++i) dma_lds_x4(bb, boff[i], st + (uint32_t)(BM * ROWB + (wave + 8 * i) * 1024));
    };

    f32x16 acc[MFRAG][NFRAG];
#pragma unroll
    for (int i = 0; i < MFRAG; ++i) {
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x16{};
    }

    // multiply K slice kt (ring slot kt % NSTAGE); NI = active row fragments of this wave
    auto compute = [&](auto NI_, int kt) __attribute__((always_inline)) {
      constexpr int NI = decltype(NI_)::value;
      const char* As = &ring[kt & (NSTAGE - 1)][wm * WM * ROWB];
      const char* Bs = &ring[kt & (NSTAGE - 1)][BM * ROWB];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 bfr[NFRAG];
#pragma unroll
        for (int j = 0; j < NFRAG; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + foff[s] + b_frag_row(j) * ROWB);
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const bf16x8 afr = *reinterpret_cast<const bf16x8*>(As + foff[s] + i * 32 * ROWB);
#pragma unroll
          for (int j = 0; j < NFRAG; ++j) acc[i][j] = mfma_32x32x16_bf16(afr, bfr[j], acc[i][j]);
        }
      }
    };

    // the K loop for a wave with NI active row fragments: slice kt is waited for (the
    // two younger slices may still be in flight), published by the barrier, and the slot
    // that slice kt - 1 used (every wave is past it) is refilled with slice kt + 3
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < KT) issue(s);
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 2 < KT) wait_vmcnt<2 * NLD>();
        else if (kt + 1 < KT) wait_vmcnt<NLD>();
        else wait_vmcnt<0>();
        __syncthreads();
        if (kt + NSTAGE - 1 < KT) issue(kt + NSTAGE - 1);
        compute(NI_, kt);
      }
    };
    // row fragments of this wave that hold rows of the tile
    const int groups = min(MFRAG, max(0, (rows - wm * WM + 31) / 32));
    switch (groups) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // epilogue. 32x32 fragment (i, j): element v at row i*32 + 8*(v/4) + 4*hgrp + (v%4),
    // column r32
#pragma unroll
    for (int i = 0; i < MFRAG; ++i) {
      if (wm * WM + i * 32 >= rows) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * hgrp + (v & 3);
        if (r >= rows) continue;
        if constexpr (MODE == kGateUp) {
          const int col = nt * (BN / 2) + wn * (WN / 2) + r32;
          if (col < ncols) {
            const float a = silu_fast(acc[i][0][v]) * acc[i][1][v];
            static_cast<uint16_t*>(g.act_out)[(int64_t)(row0 + r) * g.I + col] = (uint16_t)f32_to_bf16_bits(a);
          }
        } else {
          const float wt = sWt[r];
          const int64_t tok = sTok[r];
#pragma unroll
          for (int j = 0; j < NFRAG; ++j) {
            const int col = nt * BN + b_frag_row(j) + r32;
            if (col < ncols) {
              if (MODE == kDownAtomic) unsafeAtomicAdd(g.acc_out + tok * g.H + col, wt * acc[i][j][v]);
              else g.slot_out[tok * g.H + col] = wt * acc[i][j][v];
            }
          }
        }
      }
    }
    __syncthreads();  // sTok / sWt / ring slots are reused by the next item
  }
}

template <int MODE>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_mfma_kernel<MODE>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_mfma_bm() { return BM; }
int gateup_bf16_cols() { return BN / 2; }
int down_bf16_cols() { return BN; }

hipError_t launch_gateup_bf16(const GroupedArgs& g, int grid, hipStream_t s) { return launch<kGateUp>(g, grid, s); }

hipError_t launch_down_bf16(const GroupedArgs& g, int grid, hipStream_t s) {
  return g.slot_out ? launch<kDownSlots>(g, grid, s) : launch<kDownAtomic>(g, grid, s);
}

}  // namespace moe
