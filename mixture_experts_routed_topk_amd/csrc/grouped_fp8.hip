// e4m3 grouped GEMMs of the expert MLP on MFMA (gfx950): gate_up + SwiGLU, and down +
// routing weight + combine.
//
// The "FP8 and FP4 quantized experts" section of the Experts backends page (and its
// note): e4m3 weights ([2I, H] gate_up, [H, I] down; K contiguous) with 128x128 block
// scales (float32 or UE8M0, used directly) and e4m3 activation rows (the hidden states,
// then the SwiGLU rows) with dynamic per-row scales over 128-column blocks.  For sorted
// row m and weight row n
//     y[m, n] = sum over 128-blocks kb of  sa[m, kb] * sw[n, kb] * sum_{k in kb} a[m, k] w[n, k]
// The inner sum of one block is one 16x16x128 e4m3 MFMA; its result is folded into the
// float32 accumulator times the two scales.  With UE8M0 weight scales the MFMA applies sw
// itself (its block-scale operand: a power of two, exact), so the fold multiplies by sa
// alone -- the same value, one multiplication fewer per row and block.
//
// gate_up: a tile's 256 weight rows are 128 gate rows and the matching 128 up rows, so the
// epilogue forms gate(g) * u for 128 SwiGLU columns in registers -- one activation scale
// group per row -- and writes them as e4m3 codes with their per-row float32 scale, ready
// for the down projection (act_quant_epilogue.h).  down: 256 output
// columns; the epilogue multiplies by the routing weight and adds the row into the token's
// float32 output row (hardware float atomics) or stores it to the slot's own row
// (per-slot combine: float32 rows, or by default bf16 rows staged through LDS and written
// in 16-byte pieces).
//
// Tiles of up to 128 rows x 256 weight rows; eight waves in a 2 x 4 grid, wave (wm, wn)
// owning the 16-row fragments wm, wm + 2, .., wm + 6 and four 16-column fragments (down:
// columns 64 wn .. 64 wn + 63; gate_up: gate columns 32 wn .. 32 wn + 31 and the matching
// up columns).  K advances in slices of 128 codes (one
// scale block) held in a three-slot LDS ring filled by global->LDS DMA: slices kt + 1
// and kt + 2 stream in while slice kt is multiplied, the DMA of kt + 2 spread over the
// slice's work.  Slot rows are 128 bytes with 16-byte chunks XOR-permuted by
// (row >> 1) & 7; the row scales of the slice ride in the slot.  Work items (expert,
// N tile, M tile) in blocks of 8 M tiles x 4 N tiles (blocked_tile), an expert's rows split
// evenly over its M tiles (multiples of 32 rows, at most 128); persistent grid with
// XCD-contiguous runs of items.
#include <type_traits>

#include "act_quant_epilogue.h"
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int NW = 8;
constexpr int BM = 128;                    // tile rows (eight 16-row fragments)
constexpr int BN = 256;                    // output columns (weight rows)
constexpr int MFRAG = 4;                   // 16-row fragments per wave (2 i + wm)
constexpr int NFRAG = 4;                   // 16-column fragments per wave
constexpr int ROWB = 128;                  // bytes (= codes = K) of a tile row per slice
constexpr int NSTAGE = 3;
constexpr int SA_OFF = (BM + BN) * ROWB;   // per slot: A rows, B rows, then the row scales
constexpr int SA_N = 128;                  // row-scale entries per slot (two DMAs of 64)
constexpr int STAGE = SA_OFF + 4 * SA_N;   // 49664 bytes
constexpr int RPI = 1024 / ROWB;           // tile rows per DMA instruction
constexpr int ALD = BM / RPI / NW;         // A DMA instructions per wave per slice (2)
constexpr int BLD = BN / RPI / NW;         // B DMA instructions per wave per slice (4)
constexpr int kMaxE = 1024;
constexpr int kMaxKB = 512;                // K / 128 (K = I <= 65536)
static_assert(ALD <= 4 && BLD == 4, "the DMA of a slice is spread over four parts");
static_assert(BM == kActQRows && BN / 2 == kActQCols && NSTAGE * STAGE >= kActQLdsBytes, "epilogue tile");

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2, kDownSlotsBf16 = 3 };

__device__ __forceinline__ int chunk_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

// mfma_16x16x128_e4m3 with the whole B block scaled by 2^(s - 127): every lane passes the
// same UE8M0 byte s as the instruction's B scale.  (The instruction takes one scale per
// column and 32-long k block from the lanes; which lane feeds which differs between operand
// formats, and with one exponent for the block it does not matter.)  A power-of-two scale is
// exact, so the result is the unit-scale one times it.
__device__ __forceinline__ f32x4 mfma_16x16x128_e4m3_sb(i32x8 a, i32x8 b, int scale_b) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, f32x4{}, 0, 0, 0, 127, 0, scale_b);
}


template <int MODE, bool UE8>
__global__ __launch_bounds__(kThreads, 1) void grouped_fp8_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char ring[NSTAGE][STAGE];
  __shared__ float sSb[2][kMaxKB];          // the item's weight block scales (two row blocks)
  __shared__ uint16_t sMt[kMaxE + 1];
  __shared__ int sTok[BM];
  __shared__ float sWt[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int l16 = lane & 15, g4 = lane >> 4;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int E = g.E;
  const int KT = g.K / ROWB;
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const char* __restrict__ Sbase = reinterpret_cast<const char*>(g.a_scale);
  const uint32_t a_row_bytes = (uint32_t)g.lda;
  const uint32_t b_row_bytes = (uint32_t)g.K;
  const int ncols = MODE == kGateUp ? g.I : g.H;     // output columns of the whole GEMM

  const int n_mt = g.mt[E];
  const bool mt_lds = n_mt < 65536;
  if (mt_lds)
    for (int i = tid; i <= E; i += kThreads) sMt[i] = (uint16_t)g.mt[i];
  __syncthreads();
  const int n_items = n_mt * g.NT;
  auto mt_at = [&](int i) __attribute__((always_inline)) -> int { return mt_lds ? (int)sMt[i] : g.mt[i]; };

  const int ld_row = lane >> 3, ld_slot = lane & 7;
  const uint32_t ring0 = lds_addr(&ring[0][0]);
  // 16x16x128 operands: lane holds row (lane & 15) and codes 32 g4 .. 32 g4 + 31 of the
  // slice: logical chunks 2 g4 and 2 g4 + 1
  const uint32_t foff0 = (uint32_t)(l16 * ROWB + (chunk_slot(l16, 2 * g4) << 4));
  const uint32_t foff1 = (uint32_t)(l16 * ROWB + (chunk_slot(l16, 2 * g4 + 1) << 4));

  // tile column (weight row) of fragment j of this wave: gate_up pairs gate fragment j
  // with up fragment j + 2 (the same SwiGLU column)
  auto bcol0 = [&](int j) __attribute__((always_inline)) -> int {
    if (MODE == kGateUp) return j < 2 ? 32 * wn + 16 * j : BN / 2 + 32 * wn + 16 * (j - 2);
    return 64 * wn + 16 * j;
  };

  f32x4 acc[MFRAG][NFRAG];

  for (int w = xcd * gx + xslot; w < n_items; w += gridDim.x) {
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
    if (rows <= 0) continue;
    const char* __restrict__ Bexp = static_cast<const char*>(g.b) + (int64_t)e * g.b_expert_stride;

    // weight row of tile column c (columns past the matrix repeat its last row)
    auto b_row = [&](int c) __attribute__((always_inline)) -> int {
      if (MODE == kGateUp) {
        const int i = min(nt * (BN / 2) + (c % (BN / 2)), g.I - 1);
        return c < BN / 2 ? i : g.I + i;
      }
      return min(nt * BN + c, g.H - 1);
    };
    auto a_src = [&](int r) __attribute__((always_inline)) -> int {   // (rows past the end repeat the last)
      const int p = row0 + min(r, rows - 1);
      return g.a_rows ? g.a_rows[p] / g.a_row_div : p;
    };

    // the item's weight block scales: the 128-row blocks of tile columns 0 .. 127 and
    // 128 .. 255 (gate_up: the gate rows and the up rows of the tile)
    {
      const int KB = KT;
      const int64_t nblk_rows = g.b_rows / 128;
      for (int i = tid; i < 2 * KB; i += kThreads) {
        const int hb = i < KB ? 0 : 1;
        const int kb = i - hb * KB;
        const int64_t blk = (int64_t)e * nblk_rows + b_row(128 * hb) / 128;
        float v;   // UE8: the exponent byte itself (bits of the float), for the MFMA
        if (UE8) v = __int_as_float((int)static_cast<const uint8_t*>(g.b_scale)[blk * KB + kb]);
        else v = static_cast<const float*>(g.b_scale)[blk * KB + kb];
        sSb[hb][kb] = v;
      }
    }
    int my_tok = 0;
    float my_wt = 0.f;
    if (MODE != kGateUp && tid < rows) {
      const int slot = g.perm[row0 + tid];
      my_tok = MODE == kDownAtomic ? slot / g.k : slot;
      my_wt = g.topk_w[slot];
    }

    const int nfr16 = (rows + 15) / 16;
    const int nblk = nfr16 * (16 / RPI);   // A blocks covering the 16-row fragments with rows
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
    const bool sa_wave = wave < SA_N / 64;
    const uint32_t soff = (uint32_t)a_src(64 * (wave & 1) + lane) * (uint32_t)(KT * 4);

    auto issue_part = [&](int kt, int slot, int p) __attribute__((always_inline)) {
      const uint32_t st = ring0 + (uint32_t)(slot * STAGE);
      if (p < ALD && wave + NW * p < nblk)
        dma_lds_x4(Abase + (int64_t)kt * ROWB, aoff[p < ALD ? p : 0], st + (uint32_t)((wave + NW * p) * 1024));
      dma_lds_x4(Bexp + (int64_t)kt * ROWB, boff[p], st + (uint32_t)(BM * ROWB + (wave + NW * p) * 1024));
      if (p == 3 && sa_wave) dma_lds_x1(Sbase + (int64_t)kt * 4, soff, st + (uint32_t)(SA_OFF + wave * 256));
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) issue_part(kt, slot, p);
    };
    int na = 0;
#pragma unroll
    for (int q = 0; q < ALD; ++q) na += wave + NW * q < nblk ? 1 : 0;
    const int nld = __builtin_amdgcn_readfirstlane(na + BLD + (sa_wave ? 1 : 0));   // 4..7
    auto wait_one_slice = [&]() __attribute__((always_inline)) {
      switch (nld) {
        case 4: wait_vmcnt<4>(); break;
        case 5: wait_vmcnt<5>(); break;
        case 6: wait_vmcnt<6>(); break;
        default: wait_vmcnt<7>(); break;
      }
    };

#pragma unroll
    for (int i = 0; i < MFRAG; ++i)
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) acc[i][j] = f32x4{};

    // multiply slice kt (slot `slot`); with `next`, slice kt + 2 is issued into `nslot`,
    // one part per 16-row fragment step
    auto compute = [&](auto NI_, int kt, int slot, bool next, int nslot) __attribute__((always_inline)) {
      constexpr int NI = decltype(NI_)::value;
      const char* As = &ring[slot][0];
      const char* Bs = As + BM * ROWB;
      const float* Sa = reinterpret_cast<const float*>(As + SA_OFF);
      // weight block scale of fragment j: down, the wave's 64 columns lie in one 128-row
      // block; gate_up, fragments 0, 1 are gate rows and 2, 3 the matching up rows
      const float sb0 = sSb[MODE == kGateUp ? 0 : wn >> 1][kt];
      const float sb1 = sSb[MODE == kGateUp ? 1 : wn >> 1][kt];
      const int eb0 = __float_as_int(sb0), eb1 = __float_as_int(sb1);   // (UE8)
      i32x8 bf[NFRAG];
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) {
        const char* bp = Bs + bcol0(j) * ROWB;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(bp + foff0);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(bp + foff1);
        bf[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // four independent block products per row fragment (each MFMA writes its own
      // registers, so they issue back to back); those of fragment i are folded after the
      // MFMAs of fragment i + 1 are issued, so the folds never wait for the products they read
      f32x4 pr[2][NFRAG], sc[2][2];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        if (i < NI) {
          const char* ap = As + (2 * i + wm) * 16 * ROWB;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(ap + foff0);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(ap + foff1);
          const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&Sa[(2 * i + wm) * 16 + 4 * g4]);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            sc[i & 1][0][q] = UE8 ? sa[q] : sa[q] * sb0;
            sc[i & 1][1][q] = UE8 ? sa[q] : sa[q] * sb1;
          }
#pragma unroll
          for (int j = 0; j < NFRAG; ++j)
            pr[i & 1][j] = UE8 ? mfma_16x16x128_e4m3_sb(af, bf[j], j < 2 ? eb0 : eb1)
                               : mfma_16x16x128_e4m3(af, bf[j], f32x4{});
        }
        if (i >= 1 && i - 1 < NI) {
          const int ip = i - 1;
#pragma unroll
          for (int j = 0; j < NFRAG; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
              acc[ip][j][q] = fmaf(pr[ip & 1][j][q], sc[ip & 1][j < 2 ? 0 : 1][q], acc[ip][j][q]);
        }
        if (i < 4 && next) issue_part(kt + 2, nslot, i);
      }
    };
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
      issue(0, 0);
      if (1 < KT) issue(1, 1);
      int slot = 0;
      for (int kt = 0; kt + 1 < KT; ++kt) {
        wait_one_slice();
        __syncthreads();
        const int nslot = slot == 0 ? 2 : slot - 1;
        compute(NI_, kt, slot, kt + 2 < KT, nslot);
        slot = slot == 2 ? 0 : slot + 1;
      }
      wait_vmcnt<0>();   // the last slice
      __syncthreads();
      compute(NI_, KT - 1, slot, false, 0);
    };
    __syncthreads();   // sSb of this item is visible
    switch ((nfr16 - wm + 1) / 2) {
      case 4: kloop(std::integral_constant<int, 4>{}); break;
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // 16x16 fragment (i, j): element q at tile row (2 i + wm) * 16 + 4 g4 + q, tile column
    // bcol0(j) + l16
    if constexpr (MODE == kGateUp) {
      __syncthreads();   // every wave is done with the ring
      gateup_requant_epilogue<MFRAG>(acc, g.gate, wm, wn, l16, g4, rows, row0, nt, g.I, &ring[0][0],
                                     static_cast<uint8_t*>(g.act_out), g.act_scale_out);
    } else if constexpr (MODE == kDownSlotsBf16) {
      // weighted rows as bf16, staged through LDS as [BM rows][BN columns] and written to the
      // slots' rows in 16-byte pieces
      if (tid < BM) {
        sTok[tid] = my_tok;
        sWt[tid] = my_wt;
      }
      __syncthreads();
      uint16_t* stage = reinterpret_cast<uint16_t*>(&ring[0][0]);
#pragma unroll
      for (int i = 0; i < MFRAG; ++i) {
        if ((2 * i + wm) * 16 >= rows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = (2 * i + wm) * 16 + 4 * g4 + q;
          const float wt = sWt[r];
#pragma unroll
          for (int j = 0; j < NFRAG; ++j)
            stage[r * BN + bcol0(j) + l16] = (uint16_t)f32_to_bf16_bits(wt * acc[i][j][q]);
        }
      }
      __syncthreads();
      // every lane stores in every round (lanes past the end repeat the last piece inside
      // the matrix), so the loop has no divergent branch
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
        if ((2 * i + wm) * 16 >= rows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = (2 * i + wm) * 16 + 4 * g4 + q;
          if (r >= rows) continue;
          const float wt = sWt[r];
          const int64_t tok = sTok[r];
#pragma unroll
          for (int j = 0; j < NFRAG; ++j) {
            const int col = nt * BN + bcol0(j) + l16;
            if (col < ncols) {
              if (MODE == kDownAtomic) unsafeAtomicAdd(g.acc_out + tok * g.H + col, wt * acc[i][j][q]);
              else g.slot_out[tok * g.H + col] = wt * acc[i][j][q];
            }
          }
        }
      }
    }
    __syncthreads();   // ring, sSb, sTok / sWt are reused by the next item
  }
}

template <int MODE>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.K / ROWB > kMaxKB) return hipErrorInvalidValue;
  if (g.b_scale_ue8m0)
    hipLaunchKernelGGL((grouped_fp8_kernel<MODE, true>), dim3(grid), dim3(kThreads), 0, s, g);
  else
    hipLaunchKernelGGL((grouped_fp8_kernel<MODE, false>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_fp8_bm() { return BM; }
int gateup_fp8_cols() { return BN / 2; }
int down_fp8_cols() { return BN; }

hipError_t launch_gateup_fp8(const GroupedArgs& g, int grid, hipStream_t s) { return launch<kGateUp>(g, grid, s); }

hipError_t launch_down_fp8(const GroupedArgs& g, int grid, hipStream_t s) {
  if (!g.slot_out) return launch<kDownAtomic>(g, grid, s);
  return g.slot_bf16 ? launch<kDownSlotsBf16>(g, grid, s) : launch<kDownSlots>(g, grid, s);
}

}  // namespace moe
