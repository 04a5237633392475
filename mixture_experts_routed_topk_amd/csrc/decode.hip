// Decode path: few tokens, so the experts forward is bound by reading the selected
// experts' weights from HBM.  The Experts backends page ("Decode stage switch"
// section, and the "batched_mm" row of the backend table) switches to a batched
// product for the decode stage, which copies the chosen experts' parameters once per
// token; here every selected expert's weights are instead streamed exactly once,
// against all of that expert's tokens at the same time.
//
// Work item = (active expert, block of 64 output columns); 4 waves, each wave owns
// 16 weight rows (for gate/up: 16 gate rows and the 16 matching up rows).  The
// expert's token rows (at most 16 per pass) are staged in LDS; the weight rows go
// straight from HBM into MFMA operand registers (no LDS round trip), 64 contiguous
// bytes per lane per 128-wide K step, so each wave reads whole 256-byte row segments.
// v_mfma_f32_16x16x32_bf16 takes the weights as the 16-row A operand and the tokens as
// the 16-column B operand; any split of K across lanes works as long as both operands
// use the same one, and lane group g here holds K chunks 4g..4g+3 of the step.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int KS = 2048;          // K elements of token rows staged per slice (16 rows: 64 KB)
constexpr int kTok = 16;          // tokens per MFMA pass

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };

__device__ __forceinline__ int xswz(int tok, int chunk) { return tok * KS + ((chunk ^ (tok & 7)) << 3); }

template <int MODE>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(GroupedArgs g) {
  __shared__ __attribute__((aligned(16))) uint16_t sX[kTok * KS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, grp = lane >> 4;
  const int n_items = g.mt[g.E] * g.NT;
  const uint16_t* __restrict__ X = static_cast<const uint16_t*>(g.a);
  const uint16_t* __restrict__ W = static_cast<const uint16_t*>(g.b);

  for (int w = blockIdx.x; w < n_items; w += gridDim.x) {
    const int e = find_group(g.mt, g.E, g.NT, w);
    const int cb = w - g.mt[e] * g.NT;
    const int off = g.offsets[e];
    const int n_e = g.offsets[e + 1] - off;
    const int wrow = cb * 64 + wave * 16 + r;                 // this lane's weight row (gate or down)
    const uint16_t* pg = W + (int64_t)e * g.b_expert_stride + (int64_t)wrow * g.K + grp * 32;
    const uint16_t* pu = pg + (int64_t)g.I * g.K;            // matching up row (gate/up only)

    for (int t0 = 0; t0 < n_e; t0 += kTok) {
      const int nt = min(kTok, n_e - t0);
      f32x4 accg = {0.f, 0.f, 0.f, 0.f}, accu = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < g.K; k0 += KS) {
        const int ks = min(KS, g.K - k0);
        const int cpr = ks / 8;                               // 16-byte chunks per token row
        __syncthreads();                                      // earlier readers of sX are done
        for (int c = tid; c < kTok * cpr; c += kThreads) {
          const int tr = c / cpr, ch = c - tr * cpr;
          i32x4 v = {0, 0, 0, 0};
          if (tr < nt) {
            const int p = off + t0 + tr;
            const int64_t src = g.a_rows ? (int64_t)(g.a_rows[p] / g.a_row_div) : (int64_t)p;
            v = *reinterpret_cast<const i32x4*>(X + src * g.lda + k0 + ch * 8);
          }
          *reinterpret_cast<i32x4*>(&sX[xswz(tr, ch)]) = v;
        }
        __syncthreads();
#pragma unroll 2
        for (int kk = 0; kk < ks; kk += 128) {
          i32x4 wg[4], wu[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            wg[j] = *reinterpret_cast<const i32x4*>(pg + k0 + kk + j * 8);
            if (MODE == kGateUp) wu[j] = *reinterpret_cast<const i32x4*>(pu + k0 + kk + j * 8);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const bf16x8 xb = *reinterpret_cast<const bf16x8*>(&sX[xswz(r, kk / 8 + 4 * grp + j)]);
            accg = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, wg[j]), xb, accg);
            if (MODE == kGateUp) accu = mfma_16x16x32_bf16(__builtin_bit_cast(bf16x8, wu[j]), xb, accu);
          }
        }
      }
      // lane holds token column r, weight rows 4*grp + q of this wave's 16
      if (r < nt) {
        const int p = off + t0 + r;
        const int col0 = cb * 64 + wave * 16 + 4 * grp;
        if (MODE == kGateUp) {
          uint16_t* o = static_cast<uint16_t*>(g.act_out) + (int64_t)p * g.I + col0;
          const uint32_t lo = pack_bf16x2(gate_fn<true>(g.gate, accg[0]) * accu[0], gate_fn<true>(g.gate, accg[1]) * accu[1]);
          const uint32_t hi = pack_bf16x2(gate_fn<true>(g.gate, accg[2]) * accu[2], gate_fn<true>(g.gate, accg[3]) * accu[3]);
          *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
        } else {
          const int slot = g.perm[p];
          const float wt = g.topk_w[slot];
          if (MODE == kDownAtomic) {
            float* o = g.acc_out + (int64_t)(slot / g.k) * g.H + col0;
#pragma unroll
            for (int q = 0; q < 4; ++q) unsafeAtomicAdd(o + q, wt * accg[q]);
          } else {
            float* o = g.slot_out + (int64_t)slot * g.H + col0;
            *reinterpret_cast<f32x4*>(o) = f32x4{wt * accg[0], wt * accg[1], wt * accg[2], wt * accg[3]};
          }
        }
      }
    }
  }
}

}  // namespace

int decode_bm() { return 1 << 30; }  // one row group per active expert

hipError_t launch_decode_gateup(const GroupedArgs& g, int grid, hipStream_t s) {
  hipLaunchKernelGGL(decode_kernel<kGateUp>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

hipError_t launch_decode_down(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.slot_out) hipLaunchKernelGGL(decode_kernel<kDownSlots>, dim3(grid), dim3(kThreads), 0, s, g);
  else hipLaunchKernelGGL(decode_kernel<kDownAtomic>, dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace moe
