// Routing bookkeeping: histogram of chosen experts, exclusive-scan offsets, stable
// sort-by-expert permutation and its inverse, and the per-expert M-tile starts the
// grouped GEMMs walk.  The Experts backends page (backend table, "grouped_mm" row)
// sorts tokens by their selected expert before one grouped GEMM; this is that sort
// of the T*k (token, slot) pairs, done as a counting sort.
//
// Small batches run in one workgroup of 512 threads (8 waves).  Wave w owns a
// contiguous range of slots; per-wave histograms live in LDS, so the placement of slot
// a is
//     offsets[e] + (slots of e in earlier waves) + (slots of e earlier in this wave),
// which keeps equal experts in slot order.  Inside a wave, lanes holding the same
// expert are found with one ballot per bit of the expert id (a multi-split), so a
// 64-slot piece is ranked without atomics.
//
// Larger batches are split into G contiguous chunks of slots, one workgroup each, in
// two launches: the first writes every chunk's per-expert counts to a [G][E] table in
// the workspace; the second has every chunk read that table (its experts' totals and
// the counts of earlier chunks), so slot a of chunk g lands at
//     offsets[e] + (slots of e in chunks before g) + (its rank inside chunk g),
// ranked as above.  Chunk 0 also writes the offsets, counts and M-tile tables.
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kBatch = 8;             // 64-slot pieces whose ids are loaded together

// ---------------------------------------------------------------------------- router
// The router of token t, on one wave: softmax over its E logits, the k experts of largest
// probability taken one at a time (softmax is increasing, so by logit; equal logits go
// to the lower id), their probabilities, divided by their sum with renorm.  Lane l holds
// logits l, l + 64, ... (E <= 1024); lane j < k keeps the j-th choice.
__device__ void route_token(const RouteArgs& p, int t) {
  constexpr int J = 16;
  const int lane = threadIdx.x & 63;
  const int E = p.E, k = p.k;
  const float* row = p.logits + (int64_t)t * E;
  float v[J];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    v[j] = e < E ? row[e] : -INFINITY;
    m = fmaxf(m, v[j]);
  }
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j)
    if (lane + 64 * j < E) s += expf(v[j] - m);
  for (int d = 32; d >= 1; d >>= 1) s += __shfl_xor(s, d, 64);
  uint32_t taken = 0;   // bit j: logit j of this lane already chosen
  int my_id = 0;
  float my_w = 0.f, wsum = 0.f;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < J; ++j) {   // this lane's best remaining (ids ascend with j)
      const int e = lane + 64 * j;
      if (e < E && !((taken >> j) & 1u) && (bi == 0x7fffffff || v[j] > bv)) {
        bv = v[j];
        bi = e;
      }
    }
    for (int d = 32; d >= 1; d >>= 1) {   // larger logit, then lower id
      const float ov = __shfl_xor(bv, d, 64);
      const int oi = __shfl_xor(bi, d, 64);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    const float pr = expf(bv - m) / s;
    if (lane == r) {
      my_id = bi;
      my_w = pr;
    }
    wsum += pr;
  }
  if (lane < k) {
    p.idx_out[(int64_t)t * k + lane] = my_id;
    p.w_out[(int64_t)t * k + lane] = p.renorm ? my_w / wsum : my_w;
  }
}

// the router alone, one wave per token (in front of the chunked bookkeeping)
__global__ __launch_bounds__(kRouteThreads) void router_kernel(RouteArgs p) {
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x >> 6);
  if (t < p.A / p.k) route_token(p, t);
}

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
  if (p.logits) {   // the router step first: every token's k choices into idx_out
    for (int t = wave; t < A / p.k; t += kRouteWaves) route_token(p, t);
  }
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

  // 3. M-tile starts of the grouped GEMMs' tile height: mt[e] = sum_{e' < e} ceil(count / bm)
  //    (uniform condition: every thread takes the same branch)
  if (p.bm0 > 0 && p.mt0 != nullptr) {
    const int bm = p.bm0;
    int32_t* mt = p.mt0;
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

// ---------------------------------------------------------------------------- chunked
// Per-wave counts of the ids in [beg, end) (this wave's part of the chunk) into
// hist[wave][*]; returns the number of out-of-range ids this lane saw.
__device__ int wave_histogram(const RouteArgs& p, int beg, int end, int32_t* hist) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
      if (e >= 0 && e < p.E) atomicAdd(&hist[wave * p.E + e], 1);
      else ++nbad;
    }
  }
  return nbad;
}

// the slots of chunk g handled by this wave
__device__ void wave_range(const RouteArgs& p, int g, int* beg, int* end) {
  const int wave = threadIdx.x >> 6;
  const int c0 = g * p.chunk, c1 = min(p.A, c0 + p.chunk);
  const int per = ((c1 - c0 + kRouteWaves - 1) / kRouteWaves + 63) & ~63;
  *beg = min(c1, c0 + wave * per);
  *end = min(c1, *beg + per);
}

// 1. part[g][e] = slots of expert e in chunk g; part[G][g] = out-of-range ids in chunk g
__global__ __launch_bounds__(kRouteThreads) void route_count_kernel(RouteArgs p) {
  extern __shared__ int32_t lds[];
  const int E = p.E, G = gridDim.x, g = blockIdx.x;
  int32_t* hist = lds;   // [kRouteWaves][E]
  __shared__ int32_t bad;
  const int tid = threadIdx.x;
  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist[i] = 0;
  if (tid == 0) bad = 0;
  __syncthreads();
  int beg, end;
  wave_range(p, g, &beg, &end);
  const int nbad = wave_histogram(p, beg, end, hist);
  if (nbad) atomicAdd(&bad, nbad);
  __syncthreads();
  for (int e = tid; e < E; e += kRouteThreads) {
    int c = 0;
    for (int w = 0; w < kRouteWaves; ++w) c += hist[w * E + e];
    p.part[(int64_t)g * E + e] = c;
  }
  if (tid == 0) p.part[(int64_t)G * E + g] = bad;
}

// 2. offsets, tables (chunk 0) and the stable placement of chunk g
__global__ __launch_bounds__(kRouteThreads) void route_place_kernel(RouteArgs p) {
  extern __shared__ int32_t lds[];
  const int E = p.E, G = gridDim.x, g = blockIdx.x;
  int32_t* hist = lds;                     // [kRouteWaves][E]: counts, then cursors
  int32_t* offs = hist + kRouteWaves * E;  // [E]
  int32_t* tiles = offs + E;               // [E]: counts of e in chunks before g, then M tiles
  __shared__ int32_t wave_sums[kRouteWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  for (int i = tid; i < kRouteWaves * E; i += kRouteThreads) hist[i] = 0;
  // expert totals and the counts of earlier chunks, from the count pass (the G loads of
  // an expert are issued eight at a time, not one after the other)
  for (int e = tid; e < E; e += kRouteThreads) {
    int tot = 0, before = 0;
    for (int q0 = 0; q0 < G; q0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = q0 + u < G ? p.part[(int64_t)(q0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        tot += c[u];
        before += q0 + u < g ? c[u] : 0;
      }
    }
    offs[e] = tot;
    tiles[e] = before;
    if (g == 0 && p.counts) p.counts[e] = tot;
  }
  __syncthreads();
  int beg, end;
  wave_range(p, g, &beg, &end);
  (void)wave_histogram(p, beg, end, hist);
  const int valid = block_exclusive_scan(offs, E, wave_sums);   // (contains a barrier)
  for (int e = tid; e < E; e += kRouteThreads) {
    int run = offs[e] + tiles[e];
    for (int w = 0; w < kRouteWaves; ++w) {
      const int c = hist[w * E + e];
      hist[w * E + e] = run;
      run += c;
    }
    if (g == 0) p.offsets[e] = offs[e];
  }
  if (g == 0 && tid == 0) {
    p.offsets[E] = valid;
    if (p.bad) {
      int nb = 0;
      for (int q0 = 0; q0 < G; q0 += 8) {
        int c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) c[u] = q0 + u < G ? p.part[(int64_t)G * E + q0 + u] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) nb += c[u];
      }
      *p.bad = nb;
    }
  }
  __syncthreads();

  if (g == 0 && p.bm0 > 0 && p.mt0 != nullptr) {   // M-tile starts of the grouped GEMMs
    const int bm = p.bm0;
    int32_t* mt = p.mt0;
    __syncthreads();
    for (int e = tid; e < E; e += kRouteThreads) {
      const int c = (e + 1 < E ? offs[e + 1] : valid) - offs[e];
      tiles[e] = c == 0 ? 0 : (c - 1) / bm + 1;
    }
    __syncthreads();
    const int nt = block_exclusive_scan(tiles, E, wave_sums);
    for (int e = tid; e < E; e += kRouteThreads) mt[e] = tiles[e];
    if (tid == 0) mt[E] = nt;
    __syncthreads();
  }

  // stable placement, one 64-slot piece at a time per wave
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

int route_chunks(int A) {
  if (A <= kRouteOneBlockMax) return 1;
  const int chunk = route_chunk(A);
  return (A + chunk - 1) / chunk;
}

int route_chunk(int A) {
  const int want = (A + kRouteMaxChunks - 1) / kRouteMaxChunks;
  const int c = (want + 63) & ~63;
  return c < 1024 ? 1024 : c;
}

hipError_t launch_route(const RouteArgs& args, hipStream_t stream) {
  const size_t lds = route_lds_bytes(args.E);
  const int G = route_chunks(args.A);
  if (G <= 1 || args.part == nullptr) {
    hipLaunchKernelGGL(route_kernel, dim3(1), dim3(kRouteThreads), lds, stream, args);
    return hipGetLastError();
  }
  RouteArgs a = args;
  a.chunk = route_chunk(args.A);
  if (args.logits) {
    const int T = args.A / args.k;
    hipLaunchKernelGGL(router_kernel, dim3((T + kRouteWaves - 1) / kRouteWaves), dim3(kRouteThreads), 0, stream, a);
    const hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess) return e0;
  }
  hipLaunchKernelGGL(route_count_kernel, dim3(G), dim3(kRouteThreads), sizeof(int32_t) * (size_t)kRouteWaves * args.E,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(route_place_kernel, dim3(G), dim3(kRouteThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace moe
