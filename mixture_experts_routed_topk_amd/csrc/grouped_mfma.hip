// Grouped GEMMs of the experts forward on MFMA (gfx950).
//
// The Experts backends page (backend table, "grouped_mm" row) sorts the tokens by
// selected expert and projects them in one grouped GEMM; the expert is the gated
// MLP of the "deepgemm_megamoe" row and the "SonicMoE" section (up projection,
// SwiGLU, down projection).  Two kernels share one main loop:
//
//   gate_up : rows = hidden rows gathered through the sorted permutation,
//             B = W_gate_up[e] ([2I, H], K = H contiguous).  A 128-row B tile holds
//             64 gate rows and the 64 matching up rows, so the SwiGLU
//             a = silu(gate) * up is formed in registers (stored as bf16, or as
//             float32 for the fp8 path, which quantises it per 128 columns next).
//   down    : rows = the SwiGLU rows (already in sorted order), B = W_down[e]
//             ([H, I], K = I contiguous).  The epilogue scales each row by its
//             routing weight and adds it into the token's float32 output row
//             (hardware float atomics), or stores it to the slot's own row for the
//             deterministic combine.
//
// Operand kinds:
//   kOpBf16    bf16 operands, v_mfma_f32_16x16x32_bf16.
//   kOpFp8     OCP e4m3 operands with 128x128 block scales ("FP8 and FP4 quantized
//              experts" section and note of the same page: float32 or UE8M0 block
//              scales used directly, dynamic per-row activation scales), on
//              v_mfma_scale_f32_16x16x128_f8f6f4.  One K tile is one 128-wide scale
//              block, so each MFMA yields that block's partial product, added to the
//              float32 accumulator times (activation row scale) * (weight block scale).
//   kOpFp8Wide The same e4m3 operands widened exactly to bf16 on their way into LDS
//              (v_cvt_scalef32_pk_bf16_fp8 with scale 1) and multiplied on the bf16
//              MFMA.  gfx950's fp8 MFMAs sum their products with a precision of about
//              2^-13 of the sum of magnitudes (measured), while the bf16 MFMA sums
//              exact products in float32.  The gate/up projection feeds the e4m3
//              quantisation of the SwiGLU output, whose codes flip on such errors, so
//              it uses this kind; the down projection feeds nothing but the output
//              and uses kOpFp8.
//
// Tiles: 128 rows x 128 columns x 128 bytes of K in LDS, 256 threads = 4 waves in a
// 2 x 2 grid, 64 x 64 per wave (4 x 4 MFMA fragments).  Operands are staged through
// LDS, double buffered, in rows of 128 bytes whose 16-byte chunks are XOR-swizzled by
// (row & 7) so the fragment reads of 8 consecutive rows hit distinct banks.  The grid
// is persistent; work items are (expert, N tile, M tile) with M fastest, and each
// round hands every XCD (blockIdx % 8) a contiguous run of items, so the M tiles that
// share one weight tile run together on one XCD and meet in its L2.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, ROWB = 128;  // tile rows, tile columns, LDS bytes of K per row
constexpr int kThreads = 256;
constexpr int kTileBytes = 128 * ROWB;         // 16 KB per operand tile

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };
enum { kOpBf16 = 0, kOpFp8 = 1, kOpFp8Wide = 2 };

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ (row & 7)) << 4); }

__device__ __forceinline__ float ue8m0_to_f32(uint32_t b) {
  if (b == 0) return __uint_as_float(0x00400000u);  // 2^-127 (subnormal)
  if (b == 255) return __uint_as_float(0x7fc00000u);
  return __uint_as_float(b << 23);
}

// 16 e4m3 codes -> 16 bf16 values (exact), as two 16-byte chunks
__device__ __forceinline__ void widen_e4m3x16(const i32x4 raw, i32x4& lo, i32x4& hi) {
  uint32_t o[8];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    o[2 * w] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, false));
    o[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[w], 1.0f, true));
  }
  lo = i32x4{(int)o[0], (int)o[1], (int)o[2], (int)o[3]};
  hi = i32x4{(int)o[4], (int)o[5], (int)o[6], (int)o[7]};
}

template <int MODE, int OP>
__global__ __launch_bounds__(kThreads, 2) void grouped_mfma_kernel(GroupedArgs g) {
  constexpr bool SCALED = OP != kOpBf16;
  constexpr int ESZ = OP == kOpBf16 ? 2 : 1;          // bytes per element in global memory
  constexpr int KTILE = OP == kOpFp8 ? 128 : 64;      // K elements per LDS tile
  constexpr int TPB = 128 / KTILE;                    // K tiles per 128-wide scale block
  constexpr int GROWB = KTILE * ESZ;                  // global bytes per row per K tile
  constexpr int CPR = GROWB / 16;                     // 16-byte global chunks per row (8 or 4)
  constexpr int RPP = kThreads / CPR;                 // rows covered per loader pass (32 or 64)
  constexpr int NLD = 128 / RPP;                      // loader passes per operand (4 or 2)

  __shared__ __attribute__((aligned(16))) char sA[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) char sB[2][kTileBytes];
  __shared__ __attribute__((aligned(16))) float sSa[2][BM];  // activation row scales of the tile's block
  __shared__ float sSb[2][2];                                // weight block scales (tile rows <64, >=64)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int n_items = g.mt[g.E] * g.NT;
  const int KT = g.K / KTILE;
  const int KB = g.K / 128;                           // scale blocks along K
  const char* __restrict__ A = static_cast<const char*>(g.a);
  const char* __restrict__ B = static_cast<const char*>(g.b);

  const int lc = tid % CPR, lr = tid / CPR;           // loader: chunk lc of rows lr + RPP * i

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

    auto b_row = [&](int r) -> int {   // global weight row of tile row r
      if (MODE == kGateUp) return (r < 64) ? nt * 64 + r : g.I + nt * 64 + (r - 64);
      return nt * BN + r;
    };
    auto a_src = [&](int r) -> int64_t {  // source row of tile row r (rows past the end repeat the last)
      const int p = row0 + min(r, rows - 1);
      return g.a_rows ? (int64_t)(g.a_rows[p] / g.a_row_div) : (int64_t)p;
    };

    const char* pa[NLD];
    const char* pb[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      const int r = lr + RPP * i;
      pa[i] = A + a_src(r) * g.lda * ESZ + lc * 16;
      pb[i] = B + ((int64_t)e * g.b_expert_stride + (int64_t)b_row(r) * g.K) * ESZ + lc * 16;
    }
    // scale sources: threads 0..127 own one activation row, 128..129 one weight block
    const float* psa = nullptr;
    const void* psb = nullptr;
    if (SCALED) {
      if (tid < BM) psa = g.a_scale + a_src(tid) * KB;
      else if (tid < BM + 2) {
        const int64_t blk = (int64_t)e * (g.b_rows / 128) + b_row((tid - BM) * 64) / 128;
        psb = g.b_scale_ue8m0 ? (const void*)(static_cast<const uint8_t*>(g.b_scale) + blk * KB)
                              : (const void*)(static_cast<const float*>(g.b_scale) + blk * KB);
      }
    }
    auto load_scale = [&](int kt) -> float {
      if (!SCALED) return 0.f;
      const int kb = kt / TPB;
      if (psa) return psa[kb];
      if (psb) return g.b_scale_ue8m0 ? ue8m0_to_f32(static_cast<const uint8_t*>(psb)[kb])
                                      : static_cast<const float*>(psb)[kb];
      return 0.f;
    };
    auto store_scale = [&](int buf, float v) {
      if (!SCALED) return;
      if (tid < BM) sSa[buf][tid] = v;
      else if (tid < BM + 2) sSb[buf][tid - BM] = v;
    };
    auto store_tiles = [&](int buf, const i32x4* ra, const i32x4* rb) {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        const int r = lr + RPP * i;
        if (OP == kOpFp8Wide) {
          i32x4 lo, hi;
          widen_e4m3x16(ra[i], lo, hi);
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, 2 * lc)]) = lo;
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, 2 * lc + 1)]) = hi;
          widen_e4m3x16(rb[i], lo, hi);
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, 2 * lc)]) = lo;
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, 2 * lc + 1)]) = hi;
        } else {
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, lc)]) = ra[i];
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, lc)]) = rb[i];
        }
      }
    };

    f32x4 acc[4][4], part[4][4];   // part: running sum of the current scale block (kOpFp8Wide)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      }

    i32x4 ra[NLD], rb[NLD];
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      ra[i] = *reinterpret_cast<const i32x4*>(pa[i]);
      rb[i] = *reinterpret_cast<const i32x4*>(pb[i]);
    }
    rs = load_scale(0);
    store_tiles(0, ra, rb);
    store_scale(0, rs);
    __syncthreads();

    for (int kt = 0; kt < KT; ++kt) {
      const int cur = kt & 1;
      if (kt + 1 < KT) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          ra[i] = *reinterpret_cast<const i32x4*>(pa[i] + (kt + 1) * GROWB);
          rb[i] = *reinterpret_cast<const i32x4*>(pb[i] + (kt + 1) * GROWB);
        }
        rs = load_scale(kt + 1);
      }
      // keep the next tile's global loads in flight across the MFMA block: without
      // these fences the scheduler sinks the LDS stores (and the waits on the loads)
      // above the MFMAs, serialising every K step on memory latency
      __builtin_amdgcn_sched_barrier(0);
      if (OP != kOpFp8) {
        // bf16 MFMA over the two 32-wide K steps of this tile
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
            for (int j = 0; j < 4; ++j) {
              if (OP == kOpBf16) acc[i][j] = mfma_16x16x32_bf16(fa[i], fb[j], acc[i][j]);
              else part[i][j] = mfma_16x16x32_bf16(fa[i], fb[j], part[i][j]);
            }
        }
      } else {
        i32x8 fa[4], fb[4];
        const int c0 = 2 * (lane >> 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * 64 + i * 16 + (lane & 15);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&sA[cur][swz(r, c0)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&sA[cur][swz(r, c0 + 1)]);
          fa[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int r = wn * 64 + j * 16 + (lane & 15);
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&sB[cur][swz(r, c0)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&sB[cur][swz(r, c0 + 1)]);
          fb[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        // one MFMA covers the whole 128-wide scale block: scale its result right away
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        float sb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sb[j] = sSb[cur][wn];   // down tiles: rows of one 128-row block
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&sSa[cur][wm * 64 + i * 16 + 4 * (lane >> 4)]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 pr = mfma_16x16x128_e4m3(fa[i], fb[j], zero);
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(pr[q], sa[q] * sb[j], acc[i][j][q]);
          }
        }
      }
      if (OP == kOpFp8Wide && ((kt + 1) % TPB == 0)) {
        // end of a 128-wide scale block: acc += part * (row scale) * (block scale)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x4 sa = *reinterpret_cast<const f32x4*>(&sSa[cur][wm * 64 + i * 16 + 4 * (lane >> 4)]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            int rb0;
            if (MODE == kGateUp) rb0 = (j < 2 ? wn * 32 + j * 16 : 64 + wn * 32 + (j - 2) * 16);
            else rb0 = wn * 64 + j * 16;
            const float sb = sSb[cur][rb0 >= 64 ? 1 : 0];
#pragma unroll
            for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(part[i][j][q], sa[q] * sb, acc[i][j][q]);
            part[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (kt + 1 < KT) {
        store_tiles(cur ^ 1, ra, rb);
        store_scale(cur ^ 1, rs);
      }
      __syncthreads();
    }

    // epilogue; fragment (i, j) element q sits at tile row wm*64 + i*16 + 4*(lane>>4) + q,
    // tile column (lane & 15) of fragment j
    const int col_in = lane & 15;
    if (MODE == kGateUp) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * 64 + i * 16 + 4 * (lane >> 4) + q;
          if (r < rows) {
            const int64_t o = (int64_t)(row0 + r) * g.I + nt * 64 + wn * 32 + col_in;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const float gt = acc[i][j][q], up = acc[i][j + 2][q];
              if (SCALED) static_cast<float*>(g.act_out)[o + j * 16] = silu_exact(gt) * up;
              else static_cast<uint16_t*>(g.act_out)[o + j * 16] = (uint16_t)f32_to_bf16_bits(silu_fast(gt) * up);
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

template <int MODE, int OP>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_mfma_kernel<MODE, OP>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_mfma_bm() { return BM; }

hipError_t launch_gateup_mfma(const GroupedArgs& g, bool fp8, int grid, hipStream_t s) {
  return fp8 ? launch<kGateUp, kOpFp8Wide>(g, grid, s) : launch<kGateUp, kOpBf16>(g, grid, s);
}

hipError_t launch_down_mfma(const GroupedArgs& g, bool fp8, int grid, hipStream_t s) {
  if (g.slot_out) return fp8 ? launch<kDownSlots, kOpFp8>(g, grid, s) : launch<kDownSlots, kOpBf16>(g, grid, s);
  return fp8 ? launch<kDownAtomic, kOpFp8>(g, grid, s) : launch<kDownAtomic, kOpBf16>(g, grid, s);
}

}  // namespace moe
