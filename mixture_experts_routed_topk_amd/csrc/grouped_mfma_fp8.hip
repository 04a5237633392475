// Grouped GEMMs of the experts forward for e4m3 experts on MFMA (gfx950).
//
// The "FP8 and FP4 quantized experts" section of the Experts backends page (and its
// note): e4m3 weights with 128x128 block scales (float32 or UE8M0, used directly) and
// e4m3 activations with dynamic per-row scales over 128-column blocks.  The shapes are
// those of the bf16 grouped GEMMs (same work items, expert-sorted rows, gate/up pairing
// and combine epilogues); this file holds the two operand kinds of the e4m3 experts:
//
//   kOpFp8     16x16x128 block-scaled e4m3 MFMA (down projection), BN = 256 (wave
//              128 x 64: 8 x 4 fragments).  One MFMA spans one 128-wide scale block,
//              so its result is added to the float32 accumulator times
//              (activation row scale) * (weight block scale).
//   kOpFp8Wide The e4m3 operands widened exactly to bf16 while being written to LDS
//              (v_cvt_scalef32_pk_bf16_fp8, scale 1) and multiplied on the bf16
//              32x32x16 MFMA, the two scales applied at the end of each 128-wide block
//              (gate/up projection); BN = 128 (wave 128 x 32: 16 gate + 16 up columns
//              in one fragment, paired across lanes), since the per-block partial sums
//              need a second set of accumulators.  gfx950's fp8 MFMAs sum their
//              products with a precision of about 2^-13 of the sum of magnitudes
//              (measured); the gate/up projection feeds the e4m3 quantisation of the
//              SwiGLU output, whose codes flip on such errors, so it uses this kind.
//
// Tiling: one 512-thread block per CU, a 256-row x BN-column tile, 8 waves in a 2 x 4
// grid.  Both operands are staged through registers into two LDS buffers of 128-byte
// rows (one K tile) whose 16-byte chunks are XOR-swizzled by (row & 7); the global
// loads of tile kt+1 are in flight while tile kt is multiplied.  An expert's rows are
// split evenly over its M tiles (multiples of 32 rows, at most 256); the grid is
// persistent and XCD-aware (contiguous runs of (expert, N tile, M tile) items per XCD).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 512;          // 8 waves: 2 (rows) x 4 (columns)
constexpr int BM = 256;
constexpr int ROWB = 128;               // LDS bytes per tile row (one K tile)

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };
enum { kOpFp8 = 1, kOpFp8Wide = 2 };

template <int OP> struct Cfg;
template <> struct Cfg<kOpFp8> {        // 16x16x128 e4m3, wave 128 x 64
  static constexpr int FR = 16, MFRAG = 8, NFRAG = 4, BN = 256, KTILE = 128, GB = 128;
};
template <> struct Cfg<kOpFp8Wide> {    // 32x32x16 bf16 on widened e4m3, wave 128 x 32 (16 gate + 16 up)
  static constexpr int FR = 32, MFRAG = 4, NFRAG = 1, BN = 128, KTILE = 64, GB = 64;
};

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
__global__ __launch_bounds__(kThreads, 1) void grouped_fp8_kernel(GroupedArgs g) {
  using C = Cfg<OP>;
  constexpr bool F8 = OP == kOpFp8;
  constexpr bool WIDE = OP == kOpFp8Wide;
  constexpr bool SCALED = true;
  constexpr int BN = C::BN;
  constexpr int WM = 128, WN = BN / 4;               // wave tile
  constexpr int TPB = 128 / C::KTILE;                // K tiles per 128-wide scale block
  constexpr int CPR = C::GB / 16;                    // 16-byte global chunks per row per tile
  constexpr int RPP = kThreads / CPR;                // rows per loader pass
  constexpr int ANL = BM / RPP;                      // row loads per thread
  constexpr int BNL = BN / RPP;                      // weight loads per thread
  constexpr int ESZ = 1;                             // bytes per element in memory
  constexpr int MG = F8 ? 2 : 1;                     // row fragments per 32 rows
  using AccT = typename std::conditional<F8, f32x4, f32x16>::type;

  __shared__ __attribute__((aligned(16))) char sA[2][BM * ROWB];
  __shared__ __attribute__((aligned(16))) char sB[2][BN * ROWB];
  __shared__ __attribute__((aligned(16))) float sSa[2][BM];  // activation row scales of the stage's block
  __shared__ float sSb[2][2];                                // weight block scales: gate/first half, up/second half
  __shared__ int sTok[BM];                                   // epilogue: token (atomic) or slot (rows)
  __shared__ float sWt[BM];                                  // epilogue: routing weight

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int gx = gridDim.x >> 3;
  const int xcd = blockIdx.x & 7, xslot = blockIdx.x >> 3;
  const int n_items = g.mt[g.E] * g.NT;
  const int KT = g.K / C::KTILE;
  const int KB = g.K / 128;
  const char* __restrict__ Abase = static_cast<const char*>(g.a);
  const int lc = tid % CPR, lr = tid / CPR;          // loader: chunk lc of rows lr + RPP * i
  const int ncols = MODE == kGateUp ? g.I : g.H;     // output columns of the whole GEMM
  const int l7 = lane & 7;

  // column offset (in tile rows) of this wave's fragment j inside the weight tile
  // (gate/up, bf16: fragment 0 holds gate rows, fragment 1 the matching up rows;
  //  fp8 widened: the wave's single fragment holds 16 gate rows then the 16 up rows)
  auto b_frag_row = [&](int j) __attribute__((always_inline)) -> int {
    if (MODE == kGateUp && !WIDE) return (j == 0 ? 0 : BN / 2) + wn * (WN / 2);
    return wn * WN + j * C::FR;
  };

  // LDS byte offsets of this lane's fragment reads (swizzle term depends only on lane & 7,
  // since every fragment starts on a multiple of 8 rows)
  uint32_t a_lds[4], b_lds[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if constexpr (F8) {                              // s = 0, 1: the two 16-byte halves of 32 bytes
      const int ch = 2 * (lane >> 4) + (s & 1);
      a_lds[s] = (wm * WM + (lane & 15)) * ROWB + ((ch ^ l7) << 4);
      b_lds[s] = (lane & 15) * ROWB + ((ch ^ l7) << 4);
    } else {
      const int ch = 2 * s + (lane >> 5);
      a_lds[s] = (wm * WM + (lane & 31)) * ROWB + ((ch ^ l7) << 4);
      b_lds[s] = (lane & 31) * ROWB + ((ch ^ l7) << 4);
    }
  }

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
    const char* __restrict__ Bexp = static_cast<const char*>(g.b) + (int64_t)e * g.b_expert_stride * ESZ;

    // global weight row of tile row r; rows past the matrix repeat its last valid row
    auto b_row = [&](int r) __attribute__((always_inline)) -> int {
      if (MODE == kGateUp) {
        if (WIDE) {   // 32-row groups: 16 gate rows, then the matching 16 up rows
          const int c = min(nt * (BN / 2) + (r / 32) * 16 + (r % 16), g.I - 1);
          return (r % 32) < 16 ? c : g.I + c;
        }
        const int c = min(nt * (BN / 2) + (r % (BN / 2)), g.I - 1);
        return r < BN / 2 ? c : g.I + c;
      }
      return min(nt * BN + r, g.H - 1);
    };
    auto a_src = [&](int r) __attribute__((always_inline)) -> int {   // source row of tile row r
      const int p = row0 + min(r, rows - 1);                          // (rows past the end repeat the last)
      return g.a_rows ? g.a_rows[p] / g.a_row_div : p;
    };
    // 32-bit byte offsets of this thread's loader rows (operands are < 4 GiB, checked on the host)
    uint32_t aoff[ANL], boff[BNL];
#pragma unroll
    for (int i = 0; i < ANL; ++i) aoff[i] = (uint32_t)a_src(lr + RPP * i) * (uint32_t)(g.lda * ESZ) + lc * 16;
#pragma unroll
    for (int i = 0; i < BNL; ++i) boff[i] = (uint32_t)b_row(lr + RPP * i) * (uint32_t)(g.K * ESZ) + lc * 16;
    // scales: thread t owns activation row t; threads 0..1 also one weight block each
    const float* psa = (SCALED && tid < BM) ? g.a_scale + (int64_t)a_src(tid) * KB : nullptr;
    const char* psb = nullptr;
    if (SCALED && tid < 2) {
      // block of the first gate/down row (thread 0) and of the first up / second-half row (thread 1)
      const int64_t blk = (int64_t)e * (g.b_rows / 128) + b_row(tid == 0 ? 0 : (WIDE ? 16 : BN / 2)) / 128;
      psb = static_cast<const char*>(g.b_scale) + blk * KB * (g.b_scale_ue8m0 ? 1 : 4);
    }
    if (tid < rows) {
      const int slot = g.perm[row0 + tid];
      sTok[tid] = MODE == kDownAtomic ? slot / g.k : slot;
      sWt[tid] = g.topk_w[slot];
    }

    AccT acc[C::MFRAG][C::NFRAG], part[WIDE ? C::MFRAG : 1][WIDE ? C::NFRAG : 1];
#pragma unroll
    for (int i = 0; i < C::MFRAG; ++i)
#pragma unroll
      for (int j = 0; j < C::NFRAG; ++j) acc[i][j] = AccT{};
#pragma unroll
    for (int i = 0; i < (WIDE ? C::MFRAG : 1); ++i)
#pragma unroll
      for (int j = 0; j < (WIDE ? C::NFRAG : 1); ++j) part[i][j] = AccT{};

    i32x4 ra[ANL], rb[BNL];
    float rsa = 0.f, rsb = 0.f;

    auto load = [&](int kt) __attribute__((always_inline)) {   // global loads of tile kt into registers
      const uint32_t ko = (uint32_t)kt * C::GB;
#pragma unroll
      for (int i = 0; i < ANL; ++i) ra[i] = *reinterpret_cast<const i32x4*>(Abase + (aoff[i] + ko));
#pragma unroll
      for (int i = 0; i < BNL; ++i) rb[i] = *reinterpret_cast<const i32x4*>(Bexp + (boff[i] + ko));
      if (SCALED) {
        if (psa) rsa = psa[kt / TPB];
        if (psb) rsb = g.b_scale_ue8m0 ? ue8m0_to_f32(reinterpret_cast<const uint8_t*>(psb)[kt / TPB])
                                      : reinterpret_cast<const float*>(psb)[kt / TPB];
      }
    };
    auto store = [&](int buf) __attribute__((always_inline)) {  // registers -> LDS buffer buf
#pragma unroll
      for (int i = 0; i < ANL; ++i) {
        const int r = lr + RPP * i;
        if constexpr (WIDE) {
          i32x4 lo, hi;
          widen_e4m3x16(ra[i], lo, hi);
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, 2 * lc)]) = lo;
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, 2 * lc + 1)]) = hi;
        } else {
          *reinterpret_cast<i32x4*>(&sA[buf][swz(r, lc)]) = ra[i];
        }
      }
#pragma unroll
      for (int i = 0; i < BNL; ++i) {
        const int r = lr + RPP * i;
        if constexpr (WIDE) {
          i32x4 lo, hi;
          widen_e4m3x16(rb[i], lo, hi);
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, 2 * lc)]) = lo;
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, 2 * lc + 1)]) = hi;
        } else {
          *reinterpret_cast<i32x4*>(&sB[buf][swz(r, lc)]) = rb[i];
        }
      }
      if (SCALED) {
        if (tid < BM) sSa[buf][tid] = rsa;
        if (tid < 2) sSb[buf][tid] = rsb;
      }
    };

    // multiply the tile in LDS buffer cur; NI = active row fragments of this wave
    auto compute = [&](auto NI_, int kt) __attribute__((always_inline)) {
      constexpr int NI = decltype(NI_)::value;
      const int cur = kt & 1;
      const char* As = sA[cur];
      const char* Bs = sB[cur];
      if constexpr (!F8) {
        // 32x32x16: lane holds row (lane & 31), K chunk 2s + (lane >> 5) of the tile
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8 bfr[C::NFRAG];
#pragma unroll
          for (int j = 0; j < C::NFRAG; ++j)
            bfr[j] = *reinterpret_cast<const bf16x8*>(Bs + b_lds[s] + b_frag_row(j) * ROWB);
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const bf16x8 afr = *reinterpret_cast<const bf16x8*>(As + a_lds[s] + i * C::FR * ROWB);
#pragma unroll
            for (int j = 0; j < C::NFRAG; ++j) {
              if constexpr (WIDE) part[i][j] = mfma_32x32x16_bf16(afr, bfr[j], part[i][j]);
              else acc[i][j] = mfma_32x32x16_bf16(afr, bfr[j], acc[i][j]);
            }
          }
        }
        if constexpr (WIDE) {
          if ((kt + 1) % TPB == 0) {
            // end of a 128-wide scale block: acc += part * (row scale) * (column block scale)
#pragma unroll
            for (int j = 0; j < C::NFRAG; ++j) {
              const float sb = sSb[cur][(lane & 16) ? 1 : 0];   // columns 0..15 gate, 16..31 up
#pragma unroll
              for (int i = 0; i < NI; ++i) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  const f32x4 sa =
                      *reinterpret_cast<const f32x4*>(&sSa[cur][wm * WM + i * 32 + 8 * q + 4 * (lane >> 5)]);
#pragma unroll
                  for (int u = 0; u < 4; ++u)
                    acc[i][j][4 * q + u] = fmaf(part[i][j][4 * q + u], sa[u] * sb, acc[i][j][4 * q + u]);
                }
                part[i][j] = AccT{};
              }
            }
          }
        }
      } else {
        // 16x16x128 fp8: lane holds row (lane & 15), K bytes 32 * (lane >> 4) .. +32 of the tile
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int jh = 0; jh < 2; ++jh) {                 // column fragments in two halves
          i32x8 bfr[C::NFRAG / 2];
          float sb[C::NFRAG / 2];
#pragma unroll
          for (int jj = 0; jj < C::NFRAG / 2; ++jj) {
            const int j = jh * (C::NFRAG / 2) + jj;
            const i32x4 lo = *reinterpret_cast<const i32x4*>(Bs + b_lds[0] + b_frag_row(j) * ROWB);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(Bs + b_lds[1] + b_frag_row(j) * ROWB);
            bfr[jj] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            sb[jj] = sSb[cur][b_frag_row(j) >= BN / 2 ? 1 : 0];
          }
#pragma unroll
          for (int i = 0; i < NI; ++i) {
            const i32x4 lo = *reinterpret_cast<const i32x4*>(As + a_lds[0] + i * C::FR * ROWB);
            const i32x4 hi = *reinterpret_cast<const i32x4*>(As + a_lds[1] + i * C::FR * ROWB);
            const i32x8 afr = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const f32x4 sa = *reinterpret_cast<const f32x4*>(&sSa[cur][wm * WM + i * C::FR + 4 * (lane >> 4)]);
#pragma unroll
            for (int jj = 0; jj < C::NFRAG / 2; ++jj) {
              const int j = jh * (C::NFRAG / 2) + jj;
              const f32x4 pr = mfma_16x16x128_e4m3(afr, bfr[jj], zero);
#pragma unroll
              for (int q = 0; q < 4; ++q) acc[i][j][q] = fmaf(pr[q], sa[q] * sb[jj], acc[i][j][q]);
            }
          }
        }
      }
    };

    // the K loop for a wave with NI active row fragments (no per-fragment branches inside)
    auto kloop = [&](auto NI_) __attribute__((always_inline)) {
      load(0);
      store(0);
      __syncthreads();
      for (int kt = 0; kt < KT; ++kt) {
        if (kt + 1 < KT) load(kt + 1);
        // keep the loads in flight across the MFMAs: without these fences the scheduler
        // sinks the waits on the loads above the MFMA block
        __builtin_amdgcn_sched_barrier(0);
        compute(NI_, kt);
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < KT) store((kt + 1) & 1);
        __syncthreads();
      }
    };
    // row fragments of this wave that hold rows of the tile, in groups of 32 rows
    const int groups = min(4, max(0, (rows - wm * WM + 31) / 32));
    switch (groups) {
      case 4: kloop(std::integral_constant<int, 4 * MG>{}); break;
      case 3: kloop(std::integral_constant<int, 3 * MG>{}); break;
      case 2: kloop(std::integral_constant<int, 2 * MG>{}); break;
      case 1: kloop(std::integral_constant<int, 1 * MG>{}); break;
      default: kloop(std::integral_constant<int, 0>{}); break;
    }

    // epilogue
    if constexpr (F8) {
      // 16x16 fragment (i, j): element q at row i*16 + 4*(lane>>4) + q, column j*16 + (lane & 15)
#pragma unroll
      for (int i = 0; i < C::MFRAG; ++i) {
        if (wm * WM + i * 16 >= rows) break;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = wm * WM + i * 16 + 4 * (lane >> 4) + q;
          if (r < rows) {
            const float wt = sWt[r];
            const int64_t tok = sTok[r];
#pragma unroll
            for (int j = 0; j < C::NFRAG; ++j) {
              const int col = nt * BN + b_frag_row(j) + (lane & 15);
              if (col < ncols) {
                if (MODE == kDownAtomic) unsafeAtomicAdd(g.acc_out + tok * g.H + col, wt * acc[i][j][q]);
                else g.slot_out[tok * g.H + col] = wt * acc[i][j][q];
              }
            }
          }
        }
      }
    } else {
      // 32x32 fragment (i, j): element v at row i*32 + 8*(v/4) + 4*(lane>>5) + (v%4), column lane & 31
#pragma unroll
      for (int i = 0; i < C::MFRAG; ++i) {
        if (wm * WM + i * 32 >= rows) break;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int r = wm * WM + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
          float up_w = 0.f;
          if constexpr (WIDE) up_w = __shfl_xor(acc[i][0][v], 16);  // lane n (< 16) pairs with lane n + 16
          if (r >= rows) continue;
          if constexpr (MODE == kGateUp) {
            if constexpr (WIDE) {
              const float gt = acc[i][0][v], up = up_w;
              const int col = nt * (BN / 2) + wn * 16 + (lane & 15);
              if (!(lane & 16) && col < ncols)
                static_cast<float*>(g.act_out)[(int64_t)(row0 + r) * g.I + col] = silu_exact(gt) * up;
            } else {
              const int col = nt * (BN / 2) + wn * (WN / 2) + (lane & 31);
              if (col < ncols) {
                const float a = silu_fast(acc[i][0][v]) * acc[i][1][v];
                static_cast<uint16_t*>(g.act_out)[(int64_t)(row0 + r) * g.I + col] = (uint16_t)f32_to_bf16_bits(a);
              }
            }
          } else {
            const float wt = sWt[r];
            const int64_t tok = sTok[r];
#pragma unroll
            for (int j = 0; j < C::NFRAG; ++j) {
              const int col = nt * BN + b_frag_row(j) + (lane & 31);
              if (col < ncols) {
                if (MODE == kDownAtomic) unsafeAtomicAdd(g.acc_out + tok * g.H + col, wt * acc[i][j][v]);
                else g.slot_out[tok * g.H + col] = wt * acc[i][j][v];
              }
            }
          }
        }
      }
    }
    __syncthreads();  // sTok / sWt / LDS tiles are reused by the next item
  }
}

template <int MODE, int OP>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL((grouped_fp8_kernel<MODE, OP>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int grouped_fp8_bm() { return BM; }
int down_fp8_cols() { return Cfg<kOpFp8>::BN; }

hipError_t launch_down_fp8(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.slot_out) return launch<kDownSlots, kOpFp8>(g, grid, s);
  return launch<kDownAtomic, kOpFp8>(g, grid, s);
}

}  // namespace moe
