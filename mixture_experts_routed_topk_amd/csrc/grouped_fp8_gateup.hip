// e4m3 gate/up grouped GEMM + SwiGLU on MFMA (gfx950).
//
// The "FP8 and FP4 quantized experts" section of the Experts backends page (and its
// note): e4m3 weights with 128x128 block scales (float32 or UE8M0, used directly) and
// e4m3 activations with dynamic per-row scales over 128-column blocks.  The gate/up
// projection of an expert is
//     g[m, n] = sum over 128-blocks kb of  sx[m, kb] * sw[n, kb] * sum_{k in kb} x[m, k] w[n, k]
// (x, w the e4m3 codes' values).  gfx950's e4m3 MFMAs sum their products with a
// precision of about 2^-13 of the sum of magnitudes (measured), which flips codes of
// the e4m3 quantisation of the SwiGLU output, so the inner sums run on the bf16 MFMA
// instead: every e4m3 code is exactly a bf16 value (v_cvt_scalef32_pk_bf16_fp8 at
// scale 1), and bf16 x bf16 products accumulate exactly enough in float32.
//
// The operands stay e4m3 in memory and in LDS (half the bytes of bf16): a four-slot LDS
// ring is filled by global->LDS DMA in K slices of 128 codes, one scale block, per
// operand row, and the codes are widened when a fragment is read.  Slices kt + 1 ..
// kt + 3 stream in while slice kt is multiplied (the DMA of kt + 3 is spread over slice
// kt's four k-step pairs).  A slice's products are summed in float32 partial
// accumulators and folded into the result times the two scales at the end of the slice.
//
// Tile: up to 160 rows x 128 weight rows = 64 output columns.  Eight waves in a 2 x 4
// grid; wave (wm, wn) owns the 32-row fragments wm, wm + 2, wm + 4 and one 32-column
// fragment whose columns 0..15 are gate rows and 16..31 the matching up rows of output
// columns 16 wn .. 16 wn + 15, so SwiGLU pairs lanes l and l ^ 16.  In a slot a tile row
// is 128 bytes whose 16-byte chunks are XOR-permuted by (row >> 1) & 7 (the 16 rows of a
// 16-lane fragment read hit distinct banks).  Work items are (expert, N tile, M tile)
// with M fastest, an expert's rows split evenly over its M tiles (multiples of 32 rows,
// at most 160); persistent grid, XCD-contiguous runs of items.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;
constexpr int NW = 8;
constexpr int BM = 160;                    // tile rows (five 32-row fragments)
constexpr int BN = 128;                    // weight rows: 64 gate + 64 up
constexpr int MFRAG = 3;                   // row fragments per wave (2 i + wm < 5)
constexpr int ROWB = 128;                  // bytes (= e4m3 codes = K) of a tile row per slice
constexpr int NSTAGE = 4;
constexpr int SA_OFF = (BM + BN) * ROWB;   // per slot: A rows, B rows, then the row scales
constexpr int SA_N = 192;                  // row-scale entries per slot (three DMAs of 64)
constexpr int STAGE = SA_OFF + 4 * SA_N;   // 37632 bytes
constexpr int RPI = 1024 / ROWB;           // tile rows per DMA instruction
constexpr int ALD = (BM / RPI + NW - 1) / NW;   // most A DMA instructions per wave per slice (3)
constexpr int BLD = BN / RPI / NW;         // B DMA instructions per wave per slice (2)
constexpr int kMaxE = 1024;
constexpr int kMaxKB = 512;                // K / 128 (K = H <= 65536)
static_assert(ALD <= 4 && BLD <= 4, "the DMA of a slice is spread over four k-step pairs");

__device__ __forceinline__ int chunk_slot(int row, int c) { return c ^ ((row >> 1) & 7); }

__device__ __forceinline__ float ue8m0_value(uint32_t b) {
  if (b == 0) return __uint_as_float(0x00400000u);   // 2^-127
  if (b == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(b << 23);
}

// 16 e4m3 codes -> two bf16x8 (codes 0..7, codes 8..15), exactly
__device__ __forceinline__ void widen16(const i32x4 raw, bf16x8& lo, bf16x8& hi) {
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, false));
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, true));
  }
  lo = __builtin_bit_cast(bf16x8, i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]});
  hi = __builtin_bit_cast(bf16x8, i32x4{(int)o[4], (int)o[5], (int)o[6], (int)o[7]});
}

__global__ __launch_bounds__(kThreads, 1) void grouped_fp8_gateup_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(1024))) char ring[NSTAGE][STAGE];
  __shared__ float sSb[2][kMaxKB];          // the item's weight block scales: gate, up
  __shared__ uint16_t sMt[kMaxE + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int hgrp = lane >> 5, r32 = lane & 31;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int E = g.E;
  const int KT = g.K / ROWB;               // slices = scale blocks along K
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const char* __restrict__ Sbase = reinterpret_cast<const char*>(g.a_scale);
  const uint32_t a_row_bytes = (uint32_t)g.lda;
  const uint32_t b_row_bytes = (uint32_t)g.K;

  const int n_mt = g.mt[E];
  const bool mt_lds = n_mt < 65536;
  if (mt_lds)
    for (int i = tid; i <= E; i += kThreads) sMt[i] = (uint16_t)g.mt[i];
  __syncthreads();
  const int n_items = n_mt * g.NT;
  auto mt_at = [&](int i) __attribute__((always_inline)) -> int { return mt_lds ? (int)sMt[i] : g.mt[i]; };

  const int ld_row = lane >> 3, ld_slot = lane & 7;
  const uint32_t ring0 = lds_addr(&ring[0][0]);
  // fragment reads: k-step pair p, lane group h reads logical chunk 2 p + h (16 codes) of
  // its row; the pair's two k steps take the chunk's first and last 8 codes
  uint32_t foff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) foff[p] = (uint32_t)(r32 * ROWB + (chunk_slot(r32, 2 * p + hgrp) << 4));

  f32x16 acc[MFRAG];

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
    const int nt = local / mt_e;
    const int mloc = local - nt * mt_e;
    const int off0 = g.offsets[e], off1 = g.offsets[e + 1];
    const int cnt = off1 - off0;
    const int per = min(BM, ((cnt + mt_e - 1) / mt_e + 31) & ~31);
    const int row0 = off0 + mloc * per;
    const int rows = min(per, off1 - row0);
    if (rows <= 0) continue;
    const char* __restrict__ Bexp = static_cast<const char*>(g.b) + (int64_t)e * g.b_expert_stride;

    // weight row of tile row c: 32-row groups of 16 gate rows and the matching 16 up rows
    auto b_row = [&](int c) __attribute__((always_inline)) -> int {
      const int i = nt * (BN / 2) + (c >> 5) * 16 + (c & 15);   // < I (I is a multiple of 128)
      return (c & 16) ? g.I + i : i;
    };
    auto a_src = [&](int r) __attribute__((always_inline)) -> int {
      const int p = row0 + min(r, rows - 1);
      return g.a_rows ? g.a_rows[p] / g.a_row_div : p;
    };

    // the item's weight block scales (gate block and up block of every K block)
    {
      const int KB = KT;
      const int64_t nblk_rows = g.b_rows / 128;
      const int64_t gblk = (int64_t)e * nblk_rows + (nt * (BN / 2)) / 128;
      const int64_t ublk = (int64_t)e * nblk_rows + (g.I + nt * (BN / 2)) / 128;
      for (int i = tid; i < 2 * KB; i += kThreads) {
        const int64_t blk = i < KB ? gblk : ublk;
        const int kb = i < KB ? i : i - KB;
        float v;
        if (g.b_scale_ue8m0) v = ue8m0_value(static_cast<const uint8_t*>(g.b_scale)[blk * KB + kb]);
        else v = static_cast<const float*>(g.b_scale)[blk * KB + kb];
        sSb[i < KB ? 0 : 1][kb] = v;
      }
    }

    const int nfr = (rows + 31) / 32;
    const int nblk = nfr * (32 / RPI);
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
    // row scales: waves 0..2 each bring 64 rows' scales of the slice (one dword per lane)
    const bool sa_wave = wave < SA_N / 64;
    const uint32_t soff = (uint32_t)a_src(64 * (wave % 3) + lane) * (uint32_t)(KT * 4);

    // this wave's part p of slice kt into ring slot `slot`
    auto issue_part = [&](int kt, int slot, int p) __attribute__((always_inline)) {
      const uint32_t st = ring0 + (uint32_t)(slot * STAGE);
      if (p < ALD && wave + NW * p < nblk)
        dma_lds_x4(Abase + (int64_t)kt * ROWB, aoff[p < ALD ? p : 0], st + (uint32_t)((wave + NW * p) * 1024));
      if (p < BLD)
        dma_lds_x4(Bexp + (int64_t)kt * ROWB, boff[p < BLD ? p : 0], st + (uint32_t)(BM * ROWB + (wave + NW * p) * 1024));
      if (p == 3 && sa_wave) dma_lds_x1(Sbase + (int64_t)kt * 4, soff, st + (uint32_t)(SA_OFF + wave * 256));
    };
    auto issue = [&](int kt, int slot) __attribute__((always_inline)) {
#pragma unroll
      for (int p = 0; p < 4; ++p) issue_part(kt, slot, p);
    };
    int na = 0;
#pragma unroll
    for (int q = 0; q < ALD; ++q) na += wave + NW * q < nblk ? 1 : 0;
    // vector-memory instructions of this wave per slice: 2..6
    const int nld = __builtin_amdgcn_readfirstlane(na + BLD + (sa_wave ? 1 : 0));
    // wait until at most `slices` slices of this wave (nld instructions each) are in flight
    auto wait_slices = [&](int slices) __attribute__((always_inline)) {
      switch (slices * 8 + nld) {
        case 8 + 2: wait_vmcnt<2>(); break;
        case 8 + 3: wait_vmcnt<3>(); break;
        case 8 + 4: wait_vmcnt<4>(); break;
        case 8 + 5: wait_vmcnt<5>(); break;
        case 8 + 6: wait_vmcnt<6>(); break;
        case 16 + 2: wait_vmcnt<4>(); break;
        case 16 + 3: wait_vmcnt<6>(); break;
        case 16 + 4: wait_vmcnt<8>(); break;
        case 16 + 5: wait_vmcnt<10>(); break;
        case 16 + 6: wait_vmcnt<12>(); break;
        default: wait_vmcnt<0>(); break;
      }
    };

#pragma unroll
    for (int i = 0; i < MFRAG; ++i) acc[i] = f32x16{};

    // multiply slice kt (slot `slot`); with `next`, slice kt + 3 is issued into `nslot`
    auto compute = [&](auto NI_, int kt, int slot, bool next, int nslot) __attribute__((always_inline)) {
      constexpr int NI = decltype(NI_)::value;
      const char* As = &ring[slot][0];
      const char* Bs = As + BM * ROWB;
      const float* Sa = reinterpret_cast<const float*>(As + SA_OFF);
      f32x16 part[NI > 0 ? NI : 1];
      i32x4 ra[2][NI > 0 ? NI : 1], rb[2];
      auto load = [&](int p, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) ra[buf][i] = *reinterpret_cast<const i32x4*>(As + (2 * i + wm) * 32 * ROWB + foff[p]);
        rb[buf] = *reinterpret_cast<const i32x4*>(Bs + wn * 32 * ROWB + foff[p]);
      };
      if constexpr (NI > 0) load(0, 0);
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (NI > 0) {
          if (p + 1 < 4) load(p + 1, (p + 1) & 1);
          bf16x8 blo, bhi;
          widen16(rb[p & 1], blo, bhi);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            bf16x8 alo, ahi;
            widen16(ra[p & 1][i], alo, ahi);
            part[i] = mfma_32x32x16_bf16(alo, blo, p == 0 ? f32x16{} : part[i]);
            part[i] = mfma_32x32x16_bf16(ahi, bhi, part[i]);
          }
        }
        if (next) issue_part(kt + 3, nslot, p);
      }
      if constexpr (NI > 0) {
        // fold: acc += part * (row scale) * (gate or up block scale of this lane's column)
        const float sb = sSb[(lane & 16) ? 1 : 0][kt];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const f32x4 sa = *reinterpret_cast<const f32x4*>(&Sa[(2 * i + wm) * 32 + 8 * q + 4 * hgrp]);
#pragma unroll
            for (int u = 0; u < 4; ++u) acc[i][4 * q + u] = fmaf(part[i][4 * q + u], sa[u] * sb, acc[i][4 * q + u]);
          }
        }
      }
    };
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
      issue(0, 0);
      if (1 < KT) issue(1, 1);
      if (2 < KT) issue(2, 2);
      int slot = 0;
      for (int kt = 0; kt < KT; ++kt) {
        wait_slices(kt + 2 < KT ? 2 : (kt + 1 < KT ? 1 : 0));   // slice kt has landed ...
        __syncthreads();   // ... for every wave, and slot (kt + 3) % 4 is free
        const int nslot = (slot + 3) & 3;
        compute(NI_, kt, slot, kt + 3 < KT, nslot);
        slot = (slot + 1) & 3;
      }
    };
    __syncthreads();   // sSb of this item is visible
    switch ((nfr - wm + 1) / 2) {
      case 3: kloop(std::integral_constant<int, 3>{}); break;
      case 2: kloop(std::integral_constant<int, 2>{}); break;
      case 1: kloop(std::integral_constant<int, 1>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // epilogue: element v of fragment i sits at tile row (2 i + wm) * 32 + 8 (v / 4) +
    // 4 hgrp + (v % 4), column r32 of the wave's fragment: gate (r32 < 16) or up
    float* out = static_cast<float*>(g.act_out);
    const int col = nt * (BN / 2) + wn * 16 + (lane & 15);
#pragma unroll
    for (int i = 0; i < MFRAG; ++i) {
      if ((2 * i + wm) * 32 >= rows) break;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float up = __shfl_xor(acc[i][v], 16);
        const int r = (2 * i + wm) * 32 + 8 * (v >> 2) + 4 * hgrp + (v & 3);
        if (!(lane & 16) && r < rows) out[(int64_t)(row0 + r) * g.I + col] = gate_fn<false>(g.gate, acc[i][v]) * up;
      }
    }
    __syncthreads();   // the ring and sSb are reused by the next item
  }
}

}  // namespace

int gateup_fp8_bm() { return BM; }
int gateup_fp8_cols() { return BN / 2; }

hipError_t launch_gateup_fp8(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.K / ROWB > kMaxKB) return hipErrorInvalidValue;
  hipLaunchKernelGGL(grouped_fp8_gateup_kernel, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
