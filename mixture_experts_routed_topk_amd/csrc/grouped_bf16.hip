// bf16 grouped GEMMs of the experts forward on MFMA (gfx950).
//
// The Experts backends page (backend table, "grouped_mm" row) sorts the tokens by
// selected expert and projects them in one grouped GEMM; the expert is the gated
// MLP of the "deepgemm_megamoe" row and the "SonicMoE" section (up projection,
// SwiGLU, down projection).  Two kernels share one main loop:
//
//   gate_up : rows = hidden rows gathered through the sorted permutation, weights
//             W_gate_up[e] ([2I, H], K = H contiguous).  The weight tile holds 128 gate
//             rows and the matching 128 up rows, and every wave owns both halves of
//             its output columns, so a = silu(gate) * up is formed in registers and
//             stored once as bf16.
//   down    : rows = the SwiGLU rows (already in sorted order), weights W_down[e]
//             ([H, I], K = I contiguous).  The epilogue scales each row by its routing
//             weight and adds it into the token's float32 output row (hardware float
//             atomics), or stores it to the slot's own row: float32 for the deterministic
//             combine, or bf16 rows staged through LDS and written in 16-byte pieces (the
//             default combine of bf16 layers).
//
// A workgroup of eight waves (two per SIMD, so one wave's LDS and barrier waits are
// covered by the other's MFMAs) computes a tile of up to 160 rows x 256 columns with
// 32x32x16 MFMA.  The waves form a 2 x 4 grid of wave tiles of up to three 32-row x two
// 32-column fragments; the rows of wave (wm, wn) are the 32-row fragments wm, wm + 2,
// wm + 4 of the tile, so a partly filled tile spreads its work over both waves of every
// SIMD.
//
// K advances in slices of 64 elements (one 128-byte L2 line of every operand row) held
// in a three-slot LDS ring (52 KB per slot) filled by global->LDS DMA.  Slices kt + 1 and
// kt + 2 stream in while slice kt is multiplied: the DMA of slice kt + 2 is spread over
// the four k steps of slice kt, one A and one B block per step, into the slot that
// slice kt - 1 used.  One barrier per slice publishes a slice and frees that slot.  In a
// slot a tile row is 128 bytes whose eight 16-byte chunks are XOR-permuted by
// (row >> 1) & 7, so the 16 rows read by each 16-lane group of a fragment load hit
// distinct banks.  A rows past the tile's last 32-row fragment are neither loaded nor
// multiplied.
//
// Work items are (expert, N tile, M tile), an expert's items in blocks of 8 M tiles x 4 N
// tiles (blocked_tile); an expert's rows are split evenly over its M tiles (multiples of 32
// rows, at most 160).  The grid is persistent and each round hands every XCD (blockIdx % 8)
// a contiguous run of items, so the tiles of a block run at the same pace on one XCD and
// share their row and weight tiles in its L2.  The M-tile
// table lives in LDS as 16-bit entries (read from global memory when it does not fit).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;             // eight waves, two per SIMD, in a 2 x 4 grid
constexpr int NW = 8;
constexpr int BM = 160;                   // tile rows (five 32-row fragments)
constexpr int BN = 256;                   // tile columns (= weight rows)
constexpr int MFRAG = 3;                  // 32-row fragments per wave (2 i + wm < 5)
constexpr int NFRAG = 2;                  // 32-column fragments per wave
constexpr int KS = 64;                    // K elements per slice
constexpr int ROWB = KS * 2;              // bytes of one tile row in one slice
constexpr int KSTEPS = KS / 16;           // 32x32x16 k steps per slice
constexpr int NSTAGE = 3;                 // ring slots
constexpr int STAGE = (BM + BN) * ROWB;   // 52 KB: A rows, then B rows
constexpr int RPI = 1024 / ROWB;          // tile rows per DMA instruction (1 KB)
constexpr int ALD = (BM / RPI + NW - 1) / NW;   // most A DMA instructions per wave per slice
constexpr int BLD = BN / RPI / NW;        // B DMA instructions per wave per slice
constexpr int kMaxE = 1024;
static_assert(ALD <= KSTEPS && BLD == KSTEPS, "the DMA of a slice is spread one A and one B block per k step");

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2, kDownSlotsBf16 = 3 };

// LDS chunk slot of logical 16-byte chunk c of tile row `row`: the 16 rows of a 16-lane
// fragment-read group land in 16 distinct 16-byte bank groups of a 256-byte window
__device__ __forceinline__ int chunk_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_bf16_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char ring[NSTAGE][STAGE];
  __shared__ uint16_t sMt[kMaxE + 1];   // M-tile starts (when they fit in 16 bits)
  __shared__ int sTok[BM];    // epilogue: token (atomic combine) or slot (per-slot rows)
  __shared__ float sWt[BM];   // epilogue: routing weight

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int hgrp = lane >> 5, r32 = lane & 31;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int E = g.E;
  const int KT = g.K / KS;
  const int ncols = MODE == kGateUp ? g.I : g.H;     // output columns of the whole GEMM
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const uint32_t a_row_bytes = (uint32_t)(g.lda * 2);
  const uint32_t b_row_bytes = (uint32_t)(g.K * 2);

  const int n_mt = g.mt[E];
  const bool mt_lds = n_mt < 65536;
  if (mt_lds)
    for (int i = tid; i <= E; i += kThreads) sMt[i] = (uint16_t)g.mt[i];
  __syncthreads();
  const int n_items = n_mt * g.NT;
  // as few workgroups take items as still finish them in the least number of rounds, the
  // same number on every XCD (fewer tiles in flight at once shorten each tile's operand
  // stream); workgroup b takes items (b & 7) gx + (b >> 3) + 8 gx j when (b >> 3) < gx
  const int rounds = max(1, (n_items + (int)gridDim.x - 1) / (int)gridDim.x);
  const int gx = ((n_items + rounds - 1) / rounds + 7) >> 3;
  auto mt_at = [&](int i) __attribute__((always_inline)) -> int { return mt_lds ? (int)sMt[i] : g.mt[i]; };

  // DMA lane L of the instruction for row block b (RPI rows) fills chunk slot (L & 7) of
  // tile row RPI b + (L >> 3) with the global chunk chunk_slot maps there
  const int ld_row = lane >> 3, ld_slot = lane & 7;
  const uint32_t ring0 = lds_addr(&ring[0][0]);
  // fragment reads (k step s): tile row base + r32 (base a multiple of 32), logical
  // chunk 2 s + hgrp, at row * ROWB + (chunk_slot(row, 2 s + hgrp) << 4)
  uint32_t foff[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s) foff[s] = (uint32_t)(r32 * ROWB + (chunk_slot(r32, 2 * s + hgrp) << 4));

  // tile column of this wave's fragment j (gate/up: fragment 0 holds the gate columns,
  // fragment 1 the matching up columns, of output columns 32 wn .. 32 wn + 31)
  auto tile_col0 = [&](int j) __attribute__((always_inline)) -> int {
    if (MODE == kGateUp) return (j == 0 ? 0 : BN / 2) + wn * 32;
    return wn * 64 + j * 32;
  };

  f32x16 acc[MFRAG][NFRAG];

  for (int w = xslot < gx ? xcd * gx + xslot : n_items; w < n_items; w += 8 * gx) {
    // ---- the tile of work item w
    int e;
    {
      int lo = 0, hi = E - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (mt_at(mid) * g.NT <= w) lo = mid; else hi = mid - 1;
      }
      e = lo;
    }
    const int mt0 = mt_at(e);
    const int mt_e = mt_at(e + 1) - mt0;
    const int local = w - mt0 * g.NT;
    int nt, mloc;
    blocked_tile(local, mt_e, g.NT, g.item_mb, nt, mloc);
    const int off0 = g.offsets[e], off1 = g.offsets[e + 1];
    const int cnt = off1 - off0;
    const int per = min(BM, ((cnt + mt_e - 1) / mt_e + 31) & ~31);
    const int row0 = off0 + mloc * per;
    const int rows = min(per, off1 - row0);
    if (rows <= 0) continue;   // (never: the even split leaves every M tile some rows)
    const char* __restrict__ Bexp = static_cast<const char*>(g.b) + (int64_t)e * g.b_expert_stride * 2;

    // global weight row of tile column c; columns past the matrix repeat its last row
    auto b_row = [&](int c) __attribute__((always_inline)) -> int {
      if (MODE == kGateUp) {
        const int i = min(nt * (BN / 2) + (c % (BN / 2)), g.I - 1);
        return c < BN / 2 ? i : g.I + i;
      }
      return min(nt * BN + c, g.H - 1);
    };
    auto a_src = [&](int r) __attribute__((always_inline)) -> int {   // source row of tile row r
      const int p = row0 + min(r, rows - 1);                          // (rows past the end repeat the last)
      return g.a_rows ? g.a_rows[p] / g.a_row_div : p;
    };

    // epilogue inputs of the down projection (consumed after the K loop)
    int my_tok = 0;
    float my_wt = 0.f;
    if (MODE != kGateUp && tid < rows) {
      const int slot = g.perm[row0 + tid];
      my_tok = MODE == kDownAtomic ? slot / g.k : slot;
      my_wt = g.topk_w[slot];
    }

    // DMA: wave w loads row blocks w, w + 8, ... of A (those covering the tile's 32-row
    // fragments) and of B.  32-bit byte offsets: operands are < 4 GiB (checked on the host).
    const int nfr = (rows + 31) / 32;           // 32-row fragments with rows
    const int nblk = nfr * (32 / RPI);          // A row blocks to load
    uint32_t aoff[ALD], boff[BLD];
#pragma unroll
    for (int q = 0; q < ALD; ++q) {
      const int r = RPI * (wave + NW * q) + ld_row;
      aoff[q] = (uint32_t)a_src(r) * a_row_bytes + (uint32_t)(chunk_slot(r, ld_slot) << 4);
    }
#pragma unroll
    for (int q = 0; q < BLD; ++q) {
      const int c = RPI * (wave + NW * q) + ld_row;
      boff[q] = (uint32_t)b_row(c) * b_row_bytes + (uint32_t)(chunk_slot(c, ld_slot) << 4);
    }
    // DMA of this wave's part p of K slice kt into ring slot `slot`: A block q = p (if it
    // covers rows of the tile) and B block q = p
    auto issue_part = [&](int kt, int slot, int p) __attribute__((always_inline)) {
      const uint32_t st = ring0 + (uint32_t)(slot * STAGE);
      if (p < ALD && wave + NW * p < nblk)
        dma_lds_x4(Abase + (int64_t)kt * ROWB, aoff[p < ALD ? p : 0], st + (uint32_t)((wave + NW * p) * 1024));
      dma_lds_x4(Bexp + (int64_t)kt * ROWB, boff[p], st + (uint32_t)(BM * ROWB + (wave + NW * p) * 1024));
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < KSTEPS; ++p) issue_part(kt, slot, p);
    };
    // vector-memory instructions this wave issues per slice
    int na = 0;
#pragma unroll
    for (int q = 0; q < ALD; ++q) na += wave + NW * q < nblk ? 1 : 0;
    const int nld = __builtin_amdgcn_readfirstlane(na + BLD);
    // wait until this wave has at most one slice (nld instructions) in flight
    auto wait_one_slice = [&]() __attribute__((always_inline)) {
      switch (nld) {
        case BLD: wait_vmcnt<BLD>(); break;
        case BLD + 1: wait_vmcnt<BLD + 1>(); break;
        case BLD + 2: wait_vmcnt<BLD + 2>(); break;
        default: wait_vmcnt<BLD + 3>(); break;
      }
    };
    static_assert(ALD <= 3, "wait_one_slice covers at most three A blocks per wave");

#pragma unroll
    for (int i = 0; i < MFRAG; ++i) {
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x16{};
    }

    // multiply slice kt (ring slot `slot`) on the NI active fragments of this wave; with
    // `next`, slice kt + 2 is issued into slot `nslot` one part per k step
    auto compute = [&](auto NI_, int slot, bool next, int kt2, int nslot) __attribute__((always_inline)) {
      constexpr int NI = decltype(NI_)::value;
      const char* As = &ring[slot][0];
      const char* Bs = As + BM * ROWB;
      bf16x8 fa[2][NI > 0 ? NI : 1], fb[2][NFRAG];
      auto load_frags = [&](int s, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i)
          fa[buf][i] = *reinterpret_cast<const bf16x8*>(As + (2 * i + wm) * 32 * ROWB + foff[s]);
#pragma unroll
        for (int j = 0; j < NFRAG; ++j)
          fb[buf][j] = *reinterpret_cast<const bf16x8*>(Bs + tile_col0(j) * ROWB + foff[s]);
      };
      if constexpr (NI > 0) load_frags(0, 0);
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) {
        if (next) issue_part(kt2, nslot, s);
        if constexpr (NI > 0) {
          if (s + 1 < KSTEPS) load_frags(s + 1, (s + 1) & 1);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
#pragma unroll
            for (int j = 0; j < NFRAG; ++j) acc[i][j] = mfma_32x32x16_bf16(fa[s & 1][i], fb[s & 1][j], acc[i][j]);
          }
        }
      }
    };
    // three-slot ring: slices kt + 1 and kt + 2 stream in while slice kt is multiplied
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
      issue(0, 0);
      if (1 < KT) issue(1, 1);
      int slot = 0;
      for (int kt = 0; kt + 1 < KT; ++kt) {
        wait_one_slice();                    // slice kt has landed (kt + 1 may not) ...
        __syncthreads();                     // ... for every wave; slot (kt + 2) % 3 is free
        const int nslot = slot == 0 ? 2 : slot - 1;
        compute(NI_, slot, kt + 2 < KT, kt + 2, nslot);
        slot = slot == 2 ? 0 : slot + 1;
      }
      wait_vmcnt<0>();                       // the last slice
      __syncthreads();
      compute(NI_, slot, false, 0, 0);
    };
    // this wave's fragments 2 i + wm with rows: i < NI
    switch ((nfr - wm + 1) / 2) {
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }
    __syncthreads();   // every wave is done with the ring

    // ---- epilogue.  32x32 fragment (i, j): element v at tile row (2 i + wm) * 32 +
    // 8 (v / 4) + 4 hgrp + (v % 4), tile column tile_col0(j) + r32
    if constexpr (MODE == kGateUp) {
      // a = silu(gate) * up as bf16, staged through LDS as [BM rows][128 columns] and
      // written to HBM in 16-byte row pieces
      uint16_t* stage = reinterpret_cast<uint16_t*>(&ring[0][0]);
#pragma unroll
      for (int i = 0; i < MFRAG; ++i) {
        if ((2 * i + wm) * 32 >= rows) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (2 * i + wm) * 32 + 8 * (v >> 2) + 4 * hgrp + (v & 3);
          const float a = gate_fn<true>(g.gate, acc[i][0][v]) * acc[i][1][v];
          stage[r * 128 + wn * 32 + r32] = (uint16_t)f32_to_bf16_bits(a);
        }
      }
      __syncthreads();
      // every lane stores in every round (lanes past the end repeat the last piece inside
      // the matrix), so the loop has no divergent branch
      uint16_t* out = static_cast<uint16_t*>(g.act_out);
      const int npieces = rows * 16;
      const int last_col = min(16, (ncols - nt * 128) / 8) - 1;
      const int nround = (npieces + kThreads - 1) / kThreads;
      for (int q = 0; q < nround; ++q) {
        const int c = min(q * kThreads + tid, npieces - 1);
        const int r = c >> 4, piece = min(c & 15, last_col);
        const int col = nt * 128 + piece * 8;
        *reinterpret_cast<i32x4*>(out + (int64_t)(row0 + r) * g.I + col) =
            *reinterpret_cast<const i32x4*>(stage + r * 128 + piece * 8);
      }
    } else if constexpr (MODE == kDownSlotsBf16) {
      // weighted rows as bf16, staged through LDS as [BM rows][256 columns] and written to
      // the slots' rows in 16-byte pieces
      if (tid < BM) {
        sTok[tid] = my_tok;
        sWt[tid] = my_wt;
      }
      __syncthreads();
      uint16_t* stage = reinterpret_cast<uint16_t*>(&ring[0][0]);
#pragma unroll
      for (int i = 0; i < MFRAG; ++i) {
        if ((2 * i + wm) * 32 >= rows) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (2 * i + wm) * 32 + 8 * (v >> 2) + 4 * hgrp + (v & 3);
          const float wt = sWt[r];
#pragma unroll
          for (int j = 0; j < NFRAG; ++j)
            stage[r * BN + tile_col0(j) + r32] = (uint16_t)f32_to_bf16_bits(wt * acc[i][j][v]);
        }
      }
      __syncthreads();
      uint16_t* out = reinterpret_cast<uint16_t*>(g.slot_out);
      const int npieces = rows * (BN / 8);
      const int last_piece = min(BN / 8, (ncols - nt * BN) / 8) - 1;
      const int nround = (npieces + kThreads - 1) / kThreads;
      for (int q = 0; q < nround; ++q) {
        const int c = min(q * kThreads + tid, npieces - 1);
        const int r = c / (BN / 8), piece = min(c % (BN / 8), last_piece);
        const int col = nt * BN + piece * 8;
        *reinterpret_cast<i32x4*>(out + (int64_t)sTok[r] * g.H + col) =
            *reinterpret_cast<const i32x4*>(stage + r * BN + piece * 8);
      }
    } else {
      if (tid < BM) {
        sTok[tid] = my_tok;
        sWt[tid] = my_wt;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < MFRAG; ++i) {
        if ((2 * i + wm) * 32 >= rows) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = (2 * i + wm) * 32 + 8 * (v >> 2) + 4 * hgrp + (v & 3);
          if (r >= rows) continue;
          const float wt = sWt[r];
          const int64_t tok = sTok[r];
#pragma unroll
          for (int j = 0; j < NFRAG; ++j) {
            const int col = nt * BN + tile_col0(j) + r32;
            if (col < ncols) {
              if (MODE == kDownAtomic) unsafeAtomicAdd(g.acc_out + tok * g.H + col, wt * acc[i][j][v]);
              else if (MODE == kDownSlotsBf16)
                reinterpret_cast<uint16_t*>(g.slot_out)[tok * g.H + col] = (uint16_t)f32_to_bf16_bits(wt * acc[i][j][v]);
              else g.slot_out[tok * g.H + col] = wt * acc[i][j][v];
            }
          }
        }
      }
    }
    __syncthreads();   // the staging area and sTok / sWt are reused by the next item
  }
  // gate_up also clears the float32 accumulator of the down kernel's combine: each
  // workgroup a contiguous share, after its last tile (workgroups with one tile fewer
  // do it while the others finish)
  if constexpr (MODE == kGateUp) {
    if (g.zero_out != nullptr) {
      const int64_t per = (g.zero_n4 + gridDim.x - 1) / gridDim.x;
      const int64_t z0 = per * blockIdx.x;
      const int64_t z1 = min(g.zero_n4, z0 + per);
      f32x4* z = reinterpret_cast<f32x4*>(g.zero_out);
      for (int64_t i = z0 + tid; i < z1; i += kThreads) z[i] = f32x4{};
    }
  }
}

template <int MODE>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_bf16_kernel<MODE>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_mfma_bm() { return BM; }
int gateup_bf16_cols() { return BN / 2; }
int down_bf16_cols() { return BN; }

hipError_t launch_gateup_bf16(const GroupedArgs& g, int grid, hipStream_t s) { return launch<kGateUp>(g, grid, s); }

hipError_t launch_down_bf16(const GroupedArgs& g, int grid, hipStream_t s) {
  if (!g.slot_out) return launch<kDownAtomic>(g, grid, s);
  return g.slot_bf16 ? launch<kDownSlotsBf16>(g, grid, s) : launch<kDownSlots>(g, grid, s);
}

}  // namespace moe
