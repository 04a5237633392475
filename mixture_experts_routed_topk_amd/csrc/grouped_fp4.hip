// FP4 experts: both grouped GEMMs of the expert MLP with e2m1 weights on MFMA (gfx950).
//
// The "FP8 and FP4 quantized experts" section of the Experts backends page: expert weights
// packed two 4-bit codes per int8 byte with UE8M0 weight scales, and dynamic per-row
// activation scales.  Weight row n of expert e holds K e2m1 codes (element 2j in the low
// nibble of byte j) with one UE8M0 exponent per 32 consecutive codes; the activation rows
// are e4m3 with one float32 scale per 128 columns.  For sorted row m and weight row n
//     y[m, n] = sum over 128-blocks kb of  sa[m, kb] * sum_{k in kb} a[m, k] * w[n, k] * 2^(s[n, k/32] - 127)
// One 16x16x128 MFMA takes e4m3 A against e2m1 B and applies the weight exponents of its
// four 32-blocks itself (the per-lane scale operand); its result is folded into the float32
// accumulator times the row scale sa.
//
// gate_up: a tile's 256 weight rows are 128 gate rows and the matching 128 up rows, so the
// epilogue forms gate(g) * u for 128 SwiGLU columns in registers -- one activation scale
// group per row -- and writes them as e4m3 codes with their per-row float32 scale
// (act_quant_epilogue.h).  down: 256 output
// columns; the epilogue multiplies by the routing weight and adds the row into the token's
// float32 output row (hardware float atomics) or stores it to the slot's own row
// (per-slot combine: float32 rows, or by default bf16 rows staged through LDS and written
// in 16-byte pieces).
//
// Tiles of up to 128 rows; eight waves in a 2 x 4 grid, wave (wm, wn) owning the 16-row
// fragments wm, wm + 2, .., wm + 6 and four 16-column fragments.  K advances in slices of
// 128 (one activation scale block): per slice, 128-byte A rows, 64-byte B rows, the A row
// scales and the B exponents (one dword per weight row) land in one slot of a three-slot
// LDS ring through global->LDS DMA; slices kt + 1 and kt + 2 stream in while slice kt is
// multiplied.  Rows are stored with their 16-byte chunks XOR-permuted (A: by (row >> 1) & 7
// over 8 chunks, B: by (row >> 2) & 3 over 4 chunks) so the fragment reads are free of bank
// conflicts.  Work items (expert, N tile, M tile) in blocks of 8 M tiles x 4 N tiles
// (blocked_tile), an expert's rows split evenly over its M tiles (multiples of 32 rows);
// persistent grid with XCD-contiguous runs of items.
#include <type_traits>

#include "act_quant_epilogue.h"
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int NW = 8;
constexpr int BM = 128;                    // tile rows (eight 16-row fragments)
constexpr int BN = 256;                    // weight rows per tile
constexpr int MFRAG = 4;                   // 16-row fragments per wave (2 i + wm)
constexpr int NFRAG = 4;                   // 16-column fragments per wave
constexpr int AROW = 128;                  // bytes of a tile A row per slice (128 e4m3)
constexpr int BROW = 64;                   // bytes of a tile B row per slice (128 e2m1)
constexpr int NSTAGE = 3;
constexpr int B_OFF = BM * AROW;           // per slot: A rows, B rows, A row scales, B exponents
constexpr int SA_OFF = B_OFF + BN * BROW;
constexpr int SA_N = 128;                  // A row-scale entries (two DMAs of 64)
constexpr int SB_OFF = SA_OFF + 4 * SA_N;
constexpr int STAGE = SB_OFF + 4 * BN;     // 34304 bytes
constexpr int ARPI = 1024 / AROW;          // tile A rows per DMA instruction (8)
constexpr int BRPI = 1024 / BROW;          // tile B rows per DMA instruction (16)
constexpr int ALD = BM / ARPI / NW;        // A DMA instructions per wave per slice (2)
constexpr int BLD = BN / BRPI / NW;        // B DMA instructions per wave per slice (2)
constexpr int kMaxE = 1024;
static_assert(ALD == 2 && BLD == 2, "the DMA of a slice is issued in parts 0 .. 2");
static_assert(BM == kActQRows && BN / 2 == kActQCols && NSTAGE * STAGE >= kActQLdsBytes, "epilogue tile");

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2, kDownSlotsBf16 = 3 };

__device__ __forceinline__ int a_chunk(int row, int c) { return c ^ ((row >> 1) & 7); }
__device__ __forceinline__ int b_chunk(int row, int c) { return c ^ ((row >> 2) & 3); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 1) void grouped_fp4_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char ring[NSTAGE][STAGE];
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
  const int KT = g.K / 128;
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const char* __restrict__ Sbase = reinterpret_cast<const char*>(g.a_scale);
  const uint32_t a_row_bytes = (uint32_t)g.lda;
  const uint32_t b_row_bytes = (uint32_t)(g.K / 2);
  const uint32_t sb_row_bytes = (uint32_t)(g.K / 32);
  const int ncols = MODE == kGateUp ? g.I : g.H;     // output columns of the whole GEMM

  const int n_mt = g.mt[E];
  const bool mt_lds = n_mt < 65536;
  if (mt_lds)
    for (int i = tid; i <= E; i += kThreads) sMt[i] = (uint16_t)g.mt[i];
  __syncthreads();
  const int n_items = n_mt * g.NT;
  auto mt_at = [&](int i) __attribute__((always_inline)) -> int { return mt_lds ? (int)sMt[i] : g.mt[i]; };

  const uint32_t ring0 = lds_addr(&ring[0][0]);
  // A operand (e4m3): lane holds row l16 and the slice's codes 16 g4 .. 16 g4 + 15 and
  // 64 + 16 g4 .. 64 + 16 g4 + 15, the logical chunks g4 and 4 + g4 (the k the hardware
  // pairs with the 32 e2m1 codes 32 g4' .. 32 g4' + 31 of the B lanes)
  const uint32_t foff0 = (uint32_t)(l16 * AROW + (a_chunk(l16, g4) << 4));
  const uint32_t foff1 = (uint32_t)(l16 * AROW + (a_chunk(l16, 4 + g4) << 4));
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
    const char* __restrict__ SBexp =
        static_cast<const char*>(g.b_scale) + (int64_t)e * g.b_rows * (int64_t)sb_row_bytes;

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

    int my_tok = 0;
    float my_wt = 0.f;
    if (MODE != kGateUp && tid < rows) {
      const int slot = g.perm[row0 + tid];
      my_tok = MODE == kDownAtomic ? slot / g.k : slot;
      my_wt = g.topk_w[slot];
    }

    const int nfr16 = (rows + 15) / 16;
    const int nblk = nfr16 * (16 / ARPI);   // A blocks covering the 16-row fragments with rows
    uint32_t aoff[ALD], boff[BLD];
#pragma unroll
    for (int q = 0; q < ALD; ++q) {
      const int r = ARPI * (wave + NW * q) + (lane >> 3);
      aoff[q] = (uint32_t)a_src(r) * a_row_bytes + (uint32_t)(a_chunk(r, lane & 7) << 4);
    }
#pragma unroll
    for (int q = 0; q < BLD; ++q) {
      const int c = BRPI * (wave + NW * q) + (lane >> 2);
      boff[q] = (uint32_t)b_row(c) * b_row_bytes + (uint32_t)(b_chunk(c, lane & 3) << 4);
    }
    // scale DMAs: waves 0, 1 the A row scales (rows 64 wave + lane), waves 4 .. 7 the B
    // exponents (tile columns 64 (wave - 4) + lane, one dword = four 32-blocks per slice)
    const bool sa_wave = wave < SA_N / 64;
    const bool sb_wave = wave >= 4;
    const uint32_t soff = sa_wave ? (uint32_t)a_src(64 * wave + lane) * (uint32_t)(KT * 4)
                                  : (uint32_t)b_row(64 * (wave & 3) + lane) * sb_row_bytes;

    auto issue_part = [&](int kt, int slot, int p) __attribute__((always_inline)) {
      const uint32_t st = ring0 + (uint32_t)(slot * STAGE);
      if (p < 2) {
        if (wave + NW * p < nblk)
          dma_lds_x4(Abase + (int64_t)kt * AROW, aoff[p], st + (uint32_t)((wave + NW * p) * 1024));
        dma_lds_x4(Bexp + (int64_t)kt * BROW, boff[p], st + (uint32_t)(B_OFF + (wave + NW * p) * 1024));
      } else if (p == 2) {
        if (sa_wave) dma_lds_x1(Sbase + (int64_t)kt * 4, soff, st + (uint32_t)(SA_OFF + wave * 256));
        else if (sb_wave) dma_lds_x1(SBexp + (int64_t)kt * 4, soff, st + (uint32_t)(SB_OFF + (wave & 3) * 256));
      }
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 3; ++p) issue_part(kt, slot, p);
    };
    int na = 0;
#pragma unroll
    for (int q = 0; q < ALD; ++q) na += wave + NW * q < nblk ? 1 : 0;
    const int nld = __builtin_amdgcn_readfirstlane(na + BLD + (sa_wave || sb_wave ? 1 : 0));   // 2..5
    auto wait_one_slice = [&]() __attribute__((always_inline)) {
      switch (nld) {
        case 2: wait_vmcnt<2>(); break;
        case 3: wait_vmcnt<3>(); break;
        case 4: wait_vmcnt<4>(); break;
        default: wait_vmcnt<5>(); break;
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
      const char* Bs = As + B_OFF;
      const float* Sa = reinterpret_cast<const float*>(As + SA_OFF);
      const uint8_t* Sb = reinterpret_cast<const uint8_t*>(As + SB_OFF);
      i32x4 bf[NFRAG];
      int sbv[NFRAG];
#pragma unroll
      for (int j = 0; j < NFRAG; ++j) {
        const int c = bcol0(j) + l16;
        bf[j] = *reinterpret_cast<const i32x4*>(Bs + c * BROW + (b_chunk(c, g4) << 4));
        sbv[j] = Sb[c * 4 + g4];
      }
      // four independent block products per row fragment (the MFMAs write distinct
      // registers and issue back to back); those of fragment i are folded after the MFMAs
      // of fragment i + 1 are issued, so the folds never wait for the products they read
      f32x4 pr[2][NFRAG], sc[2];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        if (i < NI) {
          const char* ap = As + (2 * i + wm) * 16 * AROW;
          const i32x4 lo = *reinterpret_cast<const i32x4*>(ap + foff0);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(ap + foff1);
          const i32x8 af = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          sc[i & 1] = *reinterpret_cast<const f32x4*>(&Sa[(2 * i + wm) * 16 + 4 * g4]);
#pragma unroll
          for (int j = 0; j < NFRAG; ++j) pr[i & 1][j] = mfma_16x16x128_e4m3_e2m1(af, bf[j], sbv[j]);
        }
        if (i >= 1 && i - 1 < NI) {
          const int ip = i - 1;
#pragma unroll
          for (int j = 0; j < NFRAG; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[ip][j][q] = fmaf(pr[ip & 1][j][q], sc[ip & 1][q], acc[ip][j][q]);
        }
        if (next && i < 3) issue_part(kt + 2, nslot, i);
      }
    };
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
      issue(0, 0);
      if (1 < KT) issue(1, 1);
      int slot = 0;
      for (int kt = 0; kt + 1 < KT; ++kt) {
        wait_one_slice();
        __syncthreads();   // slice kt has landed for every wave; slot (kt + 2) % 3 is free
        const int nslot = slot == 0 ? 2 : slot - 1;
        compute(NI_, kt, slot, kt + 2 < KT, nslot);
        slot = slot == 2 ? 0 : slot + 1;
      }
      wait_vmcnt<0>();   // the last slice
      __syncthreads();
      compute(NI_, KT - 1, slot, false, 0);
    };
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
    __syncthreads();   // the ring and sTok / sWt are reused by the next item
  }
}

template <int MODE>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.K % 128 != 0 || g.E > kMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_fp4_kernel<MODE>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_fp4_bm() { return BM; }
int gateup_fp4_cols() { return BN / 2; }
int down_fp4_cols() { return BN; }

hipError_t launch_gateup_fp4(const GroupedArgs& g, int grid, hipStream_t s) { return launch<kGateUp>(g, grid, s); }

hipError_t launch_down_fp4(const GroupedArgs& g, int grid, hipStream_t s) {
  if (!g.slot_out) return launch<kDownAtomic>(g, grid, s);
  return g.slot_bf16 ? launch<kDownSlotsBf16>(g, grid, s) : launch<kDownSlots>(g, grid, s);
}

}  // namespace moe
