// Routing bookkeeping: histogram of chosen experts, exclusive-scan offsets, stable
// sort-by-expert permutation and its inverse, and the per-expert M-tile starts the
// grouped GEMMs walk.  The Experts backends page (backend table, "grouped_mm" row)
// sorts tokens by their selected expert before one grouped GEMM; this is that sort
// of the T*k (token, slot) pairs, done as a counting sort.
//
// One workgroup of 512 threads (8 waves).  Wave w owns a contiguous range of slots;
// per-wave histograms live in LDS, so the placement of slot a is
//     offsets[e] + (slots of e in earlier waves) + (slots of e earlier in this wave),
// which keeps equal experts in slot order.  Inside a wave, lanes holding the same
// expert are found with one ballot per bit of the expert id (a multi-split), so a
// 64-slot piece is ranked without atomics.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kBatch = 8;             // 64-slot pieces whose ids are loaded together

// Exclusive scan over v[0..n) in LDS (n <= 2 * kRouteThreads); returns the total.
__device__ int block_exclusive_scan(int32_t* v, int n, int32_t* wave_sums) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = 2 * tid;
  const int a = i0 < n ? v[i0] : 0;
  const int b = i0 + 1 < n ? v[i0 + 1] : 0;
  int s = a + b;
  for (int d = 1; d < 64; d <<= 1) {  // inclusive wave scan
    const int t = __shfl_up(s, d, 64);
    if (lane >= d) s += t;
  }
  if (lane == 63) wave_sums[wave] = s;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < kRouteWaves; ++w) {
    const int t = wave_sums[w];
    if (w < wave) before += t;
    total += t;
  }
  const int excl = before + s - (a + b);
  if (i0 < n) v[i0] = excl;
  if (i0 + 1 < n) v[i0 + 1] = excl + a;
  __syncthreads();  // v visible, wave_sums reusable
  return total;
}

__global__ __launch_bounds__(kRouteThreads) void route_kernel(RouteArgs p) {
  extern __shared__ int32_t lds[];
  const int E = p.E;
  const int A = p.A;
  int32_t* hist = lds;                   // [kRouteWaves][E]: per-wave counts, then cursors
  int32_t* offs = hist + kRouteWaves * E;  // [E]
  int32_t* tiles = offs + E;             // [E]
  __shared__ int32_t wave_sums[kRouteWaves];
  __shared__ int32_t bad;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();

  // contiguous slot range of this wave, in whole 64-slot pieces
  const int per = ((A + kRouteWaves - 1) / kRouteWaves + 63) & ~63;
  const int beg = min(A, wave * per);
  const int end = min(A, beg + per);

  // 1. per-wave histograms (ids loaded kBatch pieces at a time to overlap latency)
  int nbad = 0;
  for (int a0 = beg; a0 < end; a0 += 64 * kBatch) {
    int ids[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int a = a0 + 64 * u + lane;
      ids[u] = a < end ? p.idx[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (a0 + 64 * u + lane >= end) continue;
      const int e = ids[u];
      if (e >= 0 && e < E) atomicAdd(&hist[wave * E + e], 1);
      else ++nbad;
    }
  }
  if (nbad) atomicAdd(&bad, nbad);
  __syncthreads();

  // 2. per-expert totals; hist[w][e] becomes the count of e in waves before w
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = 0;
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    offs[e] = run;
    if (p.counts) p.counts[e] = run;
  }
  __syncthreads();
  const int valid = block_exclusive_scan(offs, E, wave_sums);  // offs = exclusive offsets
  for (int e = tid; e < E; e += kRouteThreads) {
    p.offsets[e] = offs[e];
    for (int w = 0; w < kRouteWaves; ++w) hist[w * E + e] += offs[e];
  }
  if (tid == 0) {
    p.offsets[E] = valid;
    if (p.bad) *p.bad = bad;
  }

  // 3. M-tile starts for up to two tile heights: mt[e] = sum_{e' < e} ceil(count / bm)
  for (int t = 0; t < 2; ++t) {
    const int bm = t == 0 ? p.bm0 : p.bm1;
    int32_t* mt = t == 0 ? p.mt0 : p.mt1;
    if (bm <= 0 || mt == nullptr) continue;
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) {
      const int c = (e + 1 < E ? offs[e + 1] : valid) - offs[e];
      tiles[e] = c == 0 ? 0 : (c - 1) / bm + 1;
    }
    __syncthreads();
    const int nt = block_exclusive_scan(tiles, E, wave_sums);
    for (int e = tid; e < E; e += kRouteThreads) mt[e] = tiles[e];
    if (tid == 0) mt[E] = nt;
  }
  __syncthreads();

  // 4. stable placement, one 64-slot piece at a time per wave (ids batched as above)
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int b0 = beg; b0 < end; b0 += 64 * kBatch) {
    int ids[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int a = b0 + 64 * u + lane;
      ids[u] = a < end ? p.idx[a] : -1;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int a = b0 + 64 * u + lane;
      const bool in = a < end;
      const int e = ids[u];
      const bool ok = in && e >= 0 && e < E;
      uint64_t same = __ballot(ok);
      for (int bit = 0; bit < p.id_bits; ++bit) {
        const bool set = ok && ((e >> bit) & 1);
        const uint64_t m = __ballot(set);
        same &= set ? m : ~m;
      }
      if (ok) {
        const int rank = __popcll(same & below);
        const int pos = hist[wave * E + e] + rank;
        p.perm[pos] = a;
        if (p.inv) p.inv[a] = pos;
        // the lowest lane of each group advances that expert's cursor; every lane of
        // the wave has read the cursor above before this store executes
        __builtin_amdgcn_wave_barrier();
        if (rank == 0) hist[wave * E + e] += __popcll(same);
      } else {
        __builtin_amdgcn_wave_barrier();
        if (in && p.inv) p.inv[a] = -1;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

}  // namespace

size_t route_lds_bytes(int E) { return sizeof(int32_t) * (size_t)(kRouteWaves * E + 2 * E); }

hipError_t launch_route(const RouteArgs& args, hipStream_t stream) {
  const size_t lds = route_lds_bytes(args.E);
  hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, args);
  return hipGetLastError();
}

}  // namespace moe
