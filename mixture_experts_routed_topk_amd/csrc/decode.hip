// Decode path: few tokens, so the experts forward is bound by reading the selected
// experts' weights from HBM.  The Experts backends page ("Decode stage switch"
// section, and the "batched_mm" row of the backend table) switches to a batched
// product for the decode stage, which copies the chosen experts' parameters once per
// token; here every selected expert's weights are instead streamed once, against all
// of that expert's tokens (up to 16 per pass) at the same time.
//
// A work item is (expert, pass of at most 16 of its sorted rows, group of weight rows)
// and belongs to one workgroup of four waves.  Each wave owns one 16-row weight tile:
// gate_up -- 8 gate rows and the 8 matching up rows (the item: 32 SwiGLU columns);
// down -- 16 rows of W_down (the item: 64 hidden columns).  The passes of one expert are
// adjacent items and go to workgroups of one XCD, which then share those weights in L2.
//
// HBM is read best in long runs of each weight row: a DMA instruction of a wave (1 KB)
// covers 2 rows x 512 bytes (or 4 x 256 when K is not a multiple of 256), where the
// MFMA's own register layout would cover 16 rows x 64 bytes.  So K advances in steps of
// KC = 256 (or 128) through a three-slot LDS ring filled by global->LDS DMA: while step s
// is multiplied, steps s + 1 and s + 2 are in flight; one barrier per step publishes a
// slot and frees the one before.  A slot holds the pass's 16 token rows (shared by the
// four waves; rows past the pass's last row repeat it, and their results are dropped)
// and the four weight tiles.  In a slot, the 16-byte chunk c of tile row r sits at chunk
// c ^ (r & 15) of its row, so the 16 lanes of a fragment read hit 16 different banks.
// Every table an item needs (pass starts, offsets, the sorted permutation, routing
// weights) is built in LDS first (route_in_lds, below: the decode path launches no
// separate routing kernel), so finding the next item never waits for the loads in
// flight.
//
// v_mfma_f32_16x16x32_bf16 takes the weights as the 16-row A operand and the tokens as
// the 16-column B operand; MFMA j of a step reads logical chunk 4 j + g (g = lane >> 4) of
// both, eight k each.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kWaves = 4;                            // waves per workgroup, one weight tile each
constexpr int kThreads = kWave * kWaves;
constexpr int kTok = 16;                             // sorted rows per pass (the MFMA's 16 columns)
constexpr int kTileRows = 16;                        // weight rows per wave
constexpr int kSlots = 3;                            // ring slots
constexpr int kMaxKC = 256;                          // K per step (largest)
constexpr int kSlotRows = kTok + kWaves * kTileRows; // token rows, then the four weight tiles
constexpr int kSlotBytes = kSlotRows * kMaxKC * 2;   // 40 KB
constexpr int kMaxE = 1024;

enum { kGateUp = 0, kDownAtomic = 1, kDownSlots = 2 };

// Item: expert e, first sorted row row0, rows in the pass nt (1..16), weight-row group cg.
struct Item {
  int e, row0, nt, cg;
};

// Routing bookkeeping of the decode path, in LDS, by every workgroup of both decode
// kernels (the same deterministic steps on the same ids, so all of them obtain the
// order the routing kernel would): expert counts, exclusive-scan offsets and pass
// starts, and the stable rank of each slot among the slots of its expert.  Wave 0
// ranks 64 slots per round in slot order: lanes holding the same expert are found with
// one ballot per bit of (expert + 1) (out-of-range ids form a group of their own that
// is dropped), a lane's rank is its count of such lanes below it plus the expert's
// running count, and the group's last lane advances that count.
__device__ __forceinline__ void route_in_lds(const int32_t* __restrict__ idx, int A, int E, int* sIdx, int* sRank, int* sCnt,
                             int* sOff, int* sMt, int* sBad) {
  const int tid = threadIdx.x, lane = tid & 63;
  for (int a = tid; a < A; a += kThreads) sIdx[a] = idx[a];
  for (int e = tid; e < E; e += kThreads) sCnt[e] = 0;
  __syncthreads();
  if (tid < kWave) {
    int bad = 0;
    for (int a0 = 0; a0 < A; a0 += kWave) {
      const int a = a0 + lane;
      const int e = a < A ? sIdx[a] : -1;
      const bool valid = a < A && e >= 0 && e < E;
      bad += __popcll(__ballot(a < A && !valid));
      const int key = valid ? e + 1 : 0;   // <= 1024: 11 bits
      uint64_t same = ~0ull;
#pragma unroll
      for (int bit = 0; bit < 11; ++bit) {
        const uint64_t on = __ballot((key >> bit) & 1);
        same &= ((key >> bit) & 1) ? on : ~on;
      }
      const int below = __popcll(same & ((1ull << lane) - 1ull));
      if (valid) {
        const int base = sCnt[e];
        sRank[a] = base + below;
        if ((same >> lane) == 1ull) sCnt[e] = base + below + 1;   // last lane of the group
      }
    }
    // exclusive scans of the counts (offsets) and of the 16-row passes (pass starts)
    const int per = (E + kWave - 1) / kWave;
    int sc = 0, sm = 0;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E) {
        sc += sCnt[e];
        sm += (sCnt[e] + kTok - 1) / kTok;
      }
    }
    int ic = sc, im = sm;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
      const int tc = __shfl_up(ic, d), tm = __shfl_up(im, d);
      if (lane >= d) {
        ic += tc;
        im += tm;
      }
    }
    int oc = ic - sc, om = im - sm;
    for (int i = 0; i < per; ++i) {
      const int e = lane * per + i;
      if (e < E) {
        sOff[e] = oc;
        sMt[e] = om;
        oc += sCnt[e];
        om += (sCnt[e] + kTok - 1) / kTok;
      }
    }
    if (lane == kWave - 1) {
      sOff[E] = ic;
      sMt[E] = im;
      *sBad = bad;
    }
  }
  __syncthreads();
}

template <int MODE, int KC>
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(GroupedArgs g) {
  constexpr int RB = KC * 2;              // bytes of one row in a slot
  constexpr int CPR = KC / 8;             // 16-byte chunks per row
  constexpr int RPI = kWave / CPR;        // rows per DMA instruction (1 KB)
  constexpr int NWI = kTileRows / RPI;    // DMA instructions of a wave's weight tile per step
  constexpr int NXI = kTok / RPI / kWaves;// DMA instructions of token rows per wave per step
  constexpr int NV = NWI + NXI;           // vector-memory instructions per wave per step
  constexpr int NMF = KC / 32;            // MFMAs per step
  constexpr int SLOT = kSlotRows * RB;
  static_assert(RPI * CPR == kWave && NXI * RPI * kWaves == kTok && CPR >= 16, "DMA layout");
  static_assert(SLOT <= kSlotBytes && NV < 64 && NMF % 2 == 0, "ring");

  __shared__ __attribute__((aligned(1024))) char ring[kSlots * kSlotBytes];
  __shared__ int sMt[kMaxE + 1];
  __shared__ int sOff[kMaxE + 1];
  __shared__ int sRow[kDecodeMaxSlots];     // gate_up: source row of sorted row p; down: its slot
  __shared__ float sWt[kDecodeMaxSlots];    // down: routing weight of sorted row p

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int E = g.E;
  {
    // the ring is free until the first DMA: it holds the routing scratch meanwhile
    int* sIdx = reinterpret_cast<int*>(ring);
    int* sRank = sIdx + kDecodeMaxSlots;
    int* sCnt = sRank + kDecodeMaxSlots;
    int* sBad = sCnt + kMaxE;
    const int A = g.A_slots;
    route_in_lds(g.topk_idx, A, E, sIdx, sRank, sCnt, sOff, sMt, sBad);
    const bool publish = MODE == kGateUp && blockIdx.x == 0;   // inv and the bad-id count
    for (int a = tid; a < A; a += kThreads) {
      const int e = sIdx[a];
      const bool valid = e >= 0 && e < E;
      const int p = valid ? sOff[e] + sRank[a] : -1;
      if (valid) {
        if (MODE == kGateUp) {
          sRow[p] = a / g.k;
        } else {
          sRow[p] = a;
          sWt[p] = g.topk_w[a];
        }
      }
      if (publish) g.inv_out[a] = p;
    }
    if (publish && tid == 0 && g.bad_out != nullptr) *g.bad_out = *sBad;
  }
  __syncthreads();

  // items b, b + G, ... with b = this workgroup's place in XCD-major order (G % 8 == 0)
  const int G = gridDim.x;
  const int b = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  const int n_items = sMt[E] * g.NT;
  const int mine = b < n_items ? (n_items - 1 - b) / G + 1 : 0;
  const int KST = g.K / KC;
  const int total = mine * KST;           // steps of this workgroup
  if (total == 0) return;                 // (the whole workgroup)

  auto item_at = [&](int j) __attribute__((always_inline)) -> Item {
    const int w = b + j * G;
    int lo = 0, hi = E - 1;               // expert: largest e with sMt[e] * NT <= w
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (sMt[mid] * g.NT <= w) lo = mid; else hi = mid - 1;
    }
    const int mt_e = sMt[lo + 1] - sMt[lo];
    const int local = w - sMt[lo] * g.NT;
    const int cg = local / mt_e;
    const int pass = local - cg * mt_e;
    Item it;
    it.e = lo;
    it.row0 = sOff[lo] + pass * kTok;
    it.nt = min(kTok, sOff[lo + 1] - it.row0);
    it.cg = cg;
    return it;
  };

  const char* __restrict__ Wb = static_cast<const char*>(g.b);
  const char* __restrict__ Xb = static_cast<const char*>(g.a);
  const uint32_t w_row_bytes = (uint32_t)g.K * 2;
  const uint32_t x_row_bytes = (uint32_t)(g.lda * 2);
  const uint32_t ring0 = lds_addr(ring);
  // DMA lane L fills chunk slot (L % CPR) of row (L / CPR) of its instruction's rows
  const int ld_row = lane / CPR, ld_slot = lane % CPR;

  // ---- load side: the item and step whose DMA is issued next.  32-bit offsets: an
  // expert's weights and the token rows are < 4 GiB (checked on the host).
  int lj = 0, ls = 0;
  const char* lw = nullptr;               // this item's expert weights
  uint32_t woff[NWI], xoff[NXI];
  auto set_load_item = [&](int j) __attribute__((always_inline)) {
    const Item it = item_at(j);
    lw = Wb + (int64_t)it.e * g.b_expert_stride * 2;
#pragma unroll
    for (int i = 0; i < NWI; ++i) {
      const int rho = i * RPI + ld_row;   // tile row
      int row;
      if (MODE == kGateUp) {
        const int c0 = it.cg * 32 + wave * 8;
        row = rho < 8 ? c0 + rho : g.I + c0 + rho - 8;
      } else {
        row = it.cg * 64 + wave * 16 + rho;
      }
      woff[i] = (uint32_t)row * w_row_bytes + (uint32_t)((ld_slot ^ (rho & 15)) << 4);
    }
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int rho = (wave * NXI + i) * RPI + ld_row;   // token row of the slot
      const int p = it.row0 + min(rho, it.nt - 1);
      const uint32_t src = MODE == kGateUp ? (uint32_t)sRow[p] : (uint32_t)p;
      xoff[i] = src * x_row_bytes + (uint32_t)((ld_slot ^ (rho & 15)) << 4);
    }
  };
  // DMA of the current load step into ring slot `slot`, then advance
  auto issue = [&](int slot) __attribute__((always_inline)) {
    const uint32_t st = ring0 + (uint32_t)(slot * SLOT);
    const char* wsrc = lw + ls * RB;
    const char* xsrc = Xb + ls * RB;
#pragma unroll
    for (int i = 0; i < NWI; ++i)
      dma_lds_x4(wsrc, woff[i], st + (uint32_t)((kTok + wave * kTileRows) * RB + i * 1024));
#pragma unroll
    for (int i = 0; i < NXI; ++i) dma_lds_x4(xsrc, xoff[i], st + (uint32_t)((wave * NXI + i) * 1024));
    if (++ls == KST && lj + 1 < mine) {
      ls = 0;
      set_load_item(++lj);
    }
  };

  // ---- compute side
  const int r = lane & 15, grp = lane >> 4;
  uint32_t foff[NMF];   // fragment reads: row r, logical chunk 4 j + grp
#pragma unroll
  for (int j = 0; j < NMF; ++j) foff[j] = (uint32_t)(r * RB + (((4 * j + grp) ^ r) << 4));

  auto epilogue = [&](const Item& it, f32x4 acc) __attribute__((always_inline)) {
    // lane: token column r (sorted row row0 + r), tile rows 4 grp + q
    const int p = it.row0 + r;
    if (MODE == kGateUp) {
      // tile rows 0..7 are gate rows, 8..15 the matching up rows: lane l (grp < 2) takes
      // the up values of lane l + 32
      f32x4 up;
#pragma unroll
      for (int q = 0; q < 4; ++q) up[q] = __shfl_xor(acc[q], 32);
      if (grp < 2 && r < it.nt) {
        const int col = it.cg * 32 + wave * 8 + 4 * grp;
        uint16_t* o = static_cast<uint16_t*>(g.act_out) + (int64_t)p * g.I + col;
        const uint32_t lo = pack_bf16x2(gate_fn<true>(g.gate, acc[0]) * up[0], gate_fn<true>(g.gate, acc[1]) * up[1]);
        const uint32_t hi = pack_bf16x2(gate_fn<true>(g.gate, acc[2]) * up[2], gate_fn<true>(g.gate, acc[3]) * up[3]);
        *reinterpret_cast<uint2*>(o) = make_uint2(lo, hi);
      }
    } else if (r < it.nt) {
      const int slot = sRow[p];
      const float wt = sWt[p];
      const int col = it.cg * 64 + wave * 16 + 4 * grp;
      if (MODE == kDownAtomic) {
        float* o = g.acc_out + (int64_t)(slot / g.k) * g.H + col;
#pragma unroll
        for (int q = 0; q < 4; ++q) unsafeAtomicAdd(o + q, wt * acc[q]);
      } else {
        *reinterpret_cast<f32x4*>(g.slot_out + (int64_t)slot * g.H + col) =
            f32x4{wt * acc[0], wt * acc[1], wt * acc[2], wt * acc[3]};
      }
    }
  };

  set_load_item(0);
  issue(0);
  if (1 < total) issue(1);

  int cj = 0, cs = 0, slot = 0;
  Item cit = item_at(0);
  f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  for (int u = 0; u < total; ++u) {
    if (u + 1 < total) wait_vmcnt<NV>();   // step u has landed (u + 1 may not) ...
    else wait_vmcnt<0>();
    __syncthreads();                       // ... for every wave; slot (u + 2) % 3 is free
    if (u + 2 < total) issue(slot == 0 ? 2 : slot - 1);
    const char* sp = ring + slot * SLOT;
    const char* wt = sp + (kTok + wave * kTileRows) * RB;
#pragma unroll
    for (int j = 0; j < NMF; j += 2) {
      acc0 = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(wt + foff[j]),
                                *reinterpret_cast<const bf16x8*>(sp + foff[j]), acc0);
      acc1 = mfma_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(wt + foff[j + 1]),
                                *reinterpret_cast<const bf16x8*>(sp + foff[j + 1]), acc1);
    }
    if (++cs == KST) {
      epilogue(cit, acc0 + acc1);
      acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
      acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
      cs = 0;
      if (++cj < mine) cit = item_at(cj);
    }
    slot = slot == 2 ? 0 : slot + 1;
  }
}

template <int MODE>
hipError_t launch(const GroupedArgs& g, int grid, hipStream_t s) {
  if (g.K % 256 == 0) hipLaunchKernelGGL((decode_kernel<MODE, 256>), dim3(grid), dim3(kThreads), 0, s, g);
  else hipLaunchKernelGGL((decode_kernel<MODE, 128>), dim3(grid), dim3(kThreads), 0, s, g);
  return hipGetLastError();
}

}  // namespace

int decode_bm() { return kTok; }
int decode_gateup_cols() { return kWaves * kTileRows / 2; }   // 8 gate rows per wave
int decode_down_cols() { return kWaves * kTileRows; }
int decode_groups_per_cu() { return 1; }                      // LDS: one 144 KB workgroup per CU

hipError_t launch_decode_gateup(const GroupedArgs& g, int grid, hipStream_t s) { return launch<kGateUp>(g, grid, s); }

hipError_t launch_decode_down(const GroupedArgs& g, int grid, hipStream_t s) {
  return g.slot_out ? launch<kDownSlots>(g, grid, s) : launch<kDownAtomic>(g, grid, s);
}

}  // namespace moe
