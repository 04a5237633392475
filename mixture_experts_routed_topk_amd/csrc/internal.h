// Internal launch interfaces between the C ABI layer (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------------------- routing
struct RouteArgs {
  const int32_t* idx;  // [A] flattened topk_idx (with logits: the router's output, idx_out)
  int A;
  int E;
  int id_bits;         // bits needed for ids in [0, E)
  int32_t* counts;     // [E] (may be null)
  int32_t* offsets;    // [E+1]
  int32_t* perm;       // [A]
  int32_t* inv;        // [A] (may be null)
  int32_t* bad;        // [1] out-of-range ids (may be null)
  int bm0;             // tile height of the M-tile table mt0 (0 = no table)
  int32_t* mt0;        // [E+1]
  // batches of more than kRouteOneBlockMax slots are routed in route_chunks(A) chunks of
  // route_chunk(A) slots; part holds (E + 1) * route_chunks(A) ints of scratch (when
  // null, one workgroup routes the whole batch)
  int32_t* part;
  int chunk;           // (set by launch_route)
  // optional router step in front: logits [T][E] float32 -> idx_out [T][k], w_out [T][k]
  const float* logits;
  int k;
  int renorm;          // divide the k weights by their sum
  int32_t* idx_out;
  float* w_out;
};
constexpr int kRouteOneBlockMax = 4096;
constexpr int kRouteMaxChunks = 64;
size_t route_lds_bytes(int E);
int route_chunks(int A);
int route_chunk(int A);
hipError_t launch_route(const RouteArgs& args, hipStream_t stream);

// ---------------------------------------------------------------------------- grouped GEMMs
// Common description of one grouped GEMM over expert-sorted rows.
struct GroupedArgs {
  // A operand: row p of the sorted order reads source row src(p) of `a`,
  // src(p) = a_rows ? a_rows[p] / a_row_div : p
  const void* a;
  const int32_t* a_rows;
  int a_row_div;
  int64_t lda;              // elements per source row
  const float* a_scale;     // fp8 only: [rows][K/128] float32 scales of `a`
  // B operand: weights [E][n_total][K]
  const void* b;
  int64_t b_expert_stride;  // elements
  const void* b_scale;      // fp8 only: [E][b_rows/128][K/128] float32 or uint8 (UE8M0)
  int b_scale_ue8m0;
  int b_rows;               // rows of one expert's weight matrix (2I or H)
  int K;
  int E;
  int NT;                   // number of N tiles
  const int32_t* offsets;   // [E+1] sorted-row offsets per expert
  const int32_t* mt;        // [E+1] M-tile starts for this GEMM's tile height
  int item_mb;              // work-item order: blocks of item_mb M tiles (blocked_tile)
  // gate_up epilogue
  int I;                    // intermediate size (up rows start at I)
  void* act_out;            // [A][I] SwiGLU output: bf16 / f32, or e4m3 codes (fp8, fp4)
  float* act_scale_out;     // fp8, fp4: [A][I/128] float32 scales of the e4m3 codes
  // down epilogue
  const int32_t* perm;      // sorted position -> slot
  const float* topk_w;      // [A] routing weights by slot
  int k;
  int H;
  float* acc_out;           // [T][H] float32 accumulator (atomic combine), or
  float* slot_out;          // [A][H] per-slot rows (per-slot combine): float32, or bf16
  int slot_bf16;            //   bits when slot_bf16 (bf16 down kernel only)
  // bf16 gate_up only: clear zero_n4 float4s at zero_out after its last tile (the
  // accumulator the down kernel adds into), or nothing when zero_out is null
  float* zero_out;
  int64_t zero_n4;
  int gate;                 // gate function of the gated activation (kGate*)
  // decode path only: the kernels route in LDS themselves from the [A] expert ids;
  // the gate/up kernel also writes inv [A] (sorted position or -1) and the number of
  // out-of-range ids (bad_out, may be null)
  const int32_t* topk_idx;
  int A_slots;
  int32_t* inv_out;
  int32_t* bad_out;
};

// Upper bound on M tiles for a tile height (host-side grid sizing).
inline int64_t max_mtiles(int64_t A, int E, int bm) { return A / bm + (A < E ? A : E); }

// bf16 MFMA grouped GEMMs (persistent grid, LDS ring filled by DMA)
int grouped_mfma_bm();            // tile height of the bf16 grouped GEMMs
int gateup_bf16_cols();           // SwiGLU columns per N tile of the gate/up kernel
int down_bf16_cols();             // hidden columns per N tile of the down kernel
hipError_t launch_gateup_bf16(const GroupedArgs& g, int grid, hipStream_t s);
hipError_t launch_down_bf16(const GroupedArgs& g, int grid, hipStream_t s);

// e4m3 (128x128 block-scaled) MFMA grouped GEMMs (persistent grid)
int grouped_fp8_bm();             // tile height of both e4m3 GEMMs
int gateup_fp8_cols();
int down_fp8_cols();
hipError_t launch_gateup_fp8(const GroupedArgs& g, int grid, hipStream_t s);
hipError_t launch_down_fp8(const GroupedArgs& g, int grid, hipStream_t s);

// e2m1 (FP4, 1x32 UE8M0 scales) x e4m3-row MFMA grouped GEMMs (persistent grid); B is
// packed [E][b_rows][K/2] bytes (b_expert_stride in bytes), b_scale [E][b_rows][K/32]
int grouped_fp4_bm();             // tile height of both fp4 GEMMs
int gateup_fp4_cols();
int down_fp4_cols();
hipError_t launch_gateup_fp4(const GroupedArgs& g, int grid, hipStream_t s);
hipError_t launch_down_fp4(const GroupedArgs& g, int grid, hipStream_t s);

int gateup_f32_bm();
int down_f32_bm();
hipError_t launch_gateup_f32(const GroupedArgs& g, int64_t max_items, hipStream_t s);
hipError_t launch_down_f32(const GroupedArgs& g, int64_t max_items, hipStream_t s);

// ---------------------------------------------------------------------------- decode path
// Small-T path: each active expert's weights are streamed once from HBM against its
// few rows; one workgroup per work item (expert, pass of decode_bm() sorted rows, group
// of decode_*_cols() output columns), persistent grid of decode_groups_per_cu()
// workgroups per CU.  The routing tables are copied to LDS, so A = T * k <= kDecodeMaxSlots.
constexpr int kDecodeMaxSlots = 2048;
int decode_bm();
int decode_gateup_cols();
int decode_down_cols();
int decode_groups_per_cu();
hipError_t launch_decode_gateup(const GroupedArgs& g, int grid, hipStream_t s);
hipError_t launch_decode_down(const GroupedArgs& g, int grid, hipStream_t s);

// ---------------------------------------------------------------------------- fp8 rows
// Per-row, per-128-column e4m3 quantisation: scale = amax/448 (1 if amax == 0).
hipError_t launch_quant_rows_bf16(const void* x, int64_t rows, int cols, uint8_t* q, float* scales,
                                  hipStream_t s);

// ---------------------------------------------------------------------------- instruction check
// nblocks independent 16x16x128 block products on the block-scaled MFMA (fmt 0: e4m3 x e4m3,
// fmt 1: e4m3 x e2m1 with per-32 UE8M0 exponents), zero accumulator, one wave per block.
hipError_t launch_mfma_block_check(const uint8_t* a, const uint8_t* b, const uint8_t* b_scale, float* d, int nblocks,
                                   int fmt, hipStream_t s);

// ---------------------------------------------------------------------------- elementwise
hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t s);
// out[t][h] = round(acc[t][h]) (out_bf16 != 0: bf16 RNE, else float32 copy)
hipError_t launch_finalize_acc(const float* acc, void* out, int64_t T, int H, int out_bf16,
                               hipStream_t s);
// out[t][h] = round(sum_j slot_rows[t*k + j][h]) over slots with inv != -1, in slot order
hipError_t launch_finalize_slots(const float* slot_rows, const int32_t* inv, void* out, int64_t T,
                                 int k, int H, int out_bf16, hipStream_t s);
hipError_t launch_finalize_slots_bf16(const uint16_t* slot_rows, const int32_t* inv, void* out, int64_t T,
                                      int k, int H, int out_bf16, hipStream_t s);

}  // namespace moe
