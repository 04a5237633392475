// C ABI of the routed top-k experts forward: argument validation (before any HIP
// call, so every error path is testable without a GPU), the workspace carve-up,
// the lazy per-device record, path selection and the kernel launches.
#include <hip/hip_runtime.h>

#include <mutex>
#include <stdio.h>
#include <string.h>

#include "../../include/moe_experts.h"
#include "device_common.h"
#include "internal.h"

namespace moe {
namespace {

constexpr int kMaxDevices = 64;
// The decode path is chosen by default while the experts average at most one 16-row pass
// and the batch has at most 512 slots (T * k <= min(16 E, 512)).  Measured: on the Qwen-shaped
// layer (E = 60, k = 4, uniform routing) the decode path is faster than the grouped path up to
// T = 192 and slower from T = 256; on the DeepSeek-shaped layer (E = 256, k = 8, Zipf-skewed)
// it is faster at T = 16 and 4% slower at T = 64, 17% at T = 128 (hot experts need many 16-row
// passes, each streaming the expert's weights again).
constexpr int64_t kDecodeMaxSlotsPerExpert = 16;
constexpr int64_t kDecodeDefaultMaxSlots = 512;

struct DeviceRecord {
  bool ready = false;
  int cus = 0;
};
DeviceRecord g_devices[kMaxDevices];
std::mutex g_devices_mu;

// ---------------------------------------------------------------------------- validation

bool is_fp8(const moe_problem& p) { return p.weight_dtype == MOE_FP8_E4M3; }
bool is_fp4(const moe_problem& p) { return p.weight_dtype == MOE_FP4_E2M1; }
// fp8 and fp4 experts take e4m3 activation rows with dynamic per-row scales
bool quant_acts(const moe_problem& p) { return is_fp8(p) || is_fp4(p); }

moe_status validate_problem(const moe_problem* p) {
  if (!p) return MOE_ERR_NULL_ARG;
  const bool combo_f32 = p->act_dtype == MOE_F32 && p->weight_dtype == MOE_F32 && p->scale_fmt == MOE_SCALE_NONE;
  const bool combo_bf16 = p->act_dtype == MOE_BF16 && p->weight_dtype == MOE_BF16 && p->scale_fmt == MOE_SCALE_NONE;
  const bool combo_fp8 = p->act_dtype == MOE_BF16 && p->weight_dtype == MOE_FP8_E4M3 &&
                         (p->scale_fmt == MOE_SCALE_F32 || p->scale_fmt == MOE_SCALE_UE8M0);
  const bool combo_fp4 = p->act_dtype == MOE_BF16 && p->weight_dtype == MOE_FP4_E2M1 &&
                         p->scale_fmt == MOE_SCALE_UE8M0;
  if (!(combo_f32 || combo_bf16 || combo_fp8 || combo_fp4)) return MOE_ERR_UNSUPPORTED;
  const uint32_t known = MOE_FLAG_CHECK_INDICES | MOE_FLAG_DETERMINISTIC | MOE_FLAG_FORCE_GROUPED |
                         MOE_FLAG_FORCE_DECODE | MOE_FLAG_ATOMIC_COMBINE | MOE_FLAG_ACT_GELU |
                         MOE_FLAG_ACT_RELU;
  if (p->flags & ~known) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_FORCE_GROUPED) && (p->flags & MOE_FLAG_FORCE_DECODE)) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_DETERMINISTIC) && (p->flags & MOE_FLAG_ATOMIC_COMBINE)) return MOE_ERR_UNSUPPORTED;
  if ((p->flags & MOE_FLAG_ACT_GELU) && (p->flags & MOE_FLAG_ACT_RELU)) return MOE_ERR_UNSUPPORTED;
  if (p->T < 0 || p->E < 1 || p->E > 1024 || p->k < 1 || p->k > p->E) return MOE_ERR_BAD_SHAPE;
  if (p->H <= 0 || p->I <= 0 || p->H > 65536 || p->I > 65536) return MOE_ERR_BAD_SHAPE;
  if (p->H % 128 != 0) return MOE_ERR_BAD_SHAPE;
  if (p->I % (quant_acts(*p) ? 128 : 64) != 0) return MOE_ERR_BAD_SHAPE;
  const int64_t A = p->T * (int64_t)p->k;
  if (A >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  // work-item counts of the grouped kernels must fit in int32
  const int64_t items_gu = max_mtiles(A, p->E, 64) * (2 * (int64_t)p->I / 64);
  const int64_t items_dn = max_mtiles(A, p->E, 64) * ((int64_t)p->H / 64);
  if (items_gu >= (int64_t(1) << 31) || items_dn >= (int64_t(1) << 31)) return MOE_ERR_BAD_SHAPE;
  // the grouped kernels address rows with 32-bit byte offsets: hidden [T,H], the SwiGLU
  // rows [T*k, I] and one expert's weight matrix must each stay below 4 GiB
  const int64_t esz = p->weight_dtype == MOE_F32 ? 4 : 2;
  const int64_t lim = int64_t(1) << 32;
  if (p->T * p->H * esz >= lim || A * p->I * esz >= lim || 2 * (int64_t)p->I * p->H * esz >= lim)
    return MOE_ERR_BAD_SHAPE;
  return MOE_OK;
}

bool aligned16(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; }
bool aligned4(const void* q) { return (reinterpret_cast<uintptr_t>(q) & 3u) == 0; }

// ---------------------------------------------------------------------------- plan

enum Path { kGrouped = 0, kDecode = 1 };

struct Plan {
  Path path;
  int bm;     // row-group height of the M-tile table both GEMMs walk
};

// Combine by per-slot rows (each slot's weighted row stored, the k rows of a token summed
// in slot order) rather than float atomics: always with MOE_FLAG_DETERMINISTIC, and by
// default while the slot rows stay small: float32 rows up to 512 MiB, the bf16 rows of a
// bf16, fp8 or fp4 layer up to 1 GiB (the DeepSeek-shaped fp8 and fp4 layers, 470 MB of
// bf16 rows: 3.2-3.3% faster per step than the float atomics).  Measured on MI355X: with 134 MB of slot rows (Qwen prefill,
// T*k = 16384, H = 2048) the down kernel plus the slot sum take 12% less time than the
// atomic combine; on the DeepSeek prefill layer (T*k = 65536, H = 7168) float32 rows
// (1.9 GB) lose to the atomics by 3%, bf16 rows (0.94 GB) win by 1.4% of the whole step.
constexpr int64_t kSlotCombineMaxBytes = int64_t(512) << 20;
constexpr int64_t kSlotCombineMaxBytesBf16 = int64_t(1) << 30;
bool slot_combine(const moe_problem& p) {
  if (p.flags & MOE_FLAG_DETERMINISTIC) return true;
  if (p.flags & MOE_FLAG_ATOMIC_COMBINE) return false;
  const int64_t rows = (int64_t)p.T * p.k * p.H;
  if (4 * rows <= kSlotCombineMaxBytes) return true;
  // larger bf16 layers take the grouped path (the decode path stops at T * k <= 2048),
  // whose default slot rows are bf16
  return (p.weight_dtype == MOE_BF16 || quant_acts(p)) && p.act_dtype == MOE_BF16 &&
         2 * rows <= kSlotCombineMaxBytesBf16;
}

// The per-slot rows of the grouped path's default combine (bf16, fp8 and fp4 layers) are
// stored as bf16: each
// slot's weighted row is rounded once to bf16 and the k rows of a token are summed in
// float32 (MOE_FLAG_DETERMINISTIC keeps float32 rows).  On the Qwen prefill layer this
// moves half the bytes of float32 rows; the extra rounding stays far inside the bf16
// tolerance (simulated on sampled tokens: worst error 0.12 of the tolerance, against
// 0.065 with float32 rows).
bool slot_rows_bf16(const moe_problem& p, bool decode) {
  return slot_combine(p) && !(p.flags & MOE_FLAG_DETERMINISTIC) && !decode &&
         (p.weight_dtype == MOE_BF16 || quant_acts(p)) && p.act_dtype == MOE_BF16;
}

bool decode_capable(const moe_problem& p) {
  return p.weight_dtype == MOE_BF16 && p.I % 128 == 0 && p.T * p.k <= kDecodeMaxSlots;
}

Plan make_plan(const moe_problem& p) {
  Plan pl;
  bool decode = p.T * p.k <= kDecodeMaxSlotsPerExpert * p.E && p.T * p.k <= kDecodeDefaultMaxSlots;
  if (p.flags & MOE_FLAG_FORCE_GROUPED) decode = false;
  if (p.flags & MOE_FLAG_FORCE_DECODE) decode = true;
  if (!decode_capable(p)) decode = false;
  pl.path = decode ? kDecode : kGrouped;
  if (decode) pl.bm = decode_bm();
  else if (is_fp4(p)) pl.bm = grouped_fp4_bm();
  else pl.bm = p.weight_dtype == MOE_F32 ? gateup_f32_bm() : (is_fp8(p) ? grouped_fp8_bm() : grouped_mfma_bm());
  return pl;
}

// ---------------------------------------------------------------------------- workspace

struct Layout {
  size_t bad, counts, offsets, mt, perm, inv;
  size_t route_part; // chunked routing: per-chunk expert counts [G][E] and bad-id counts [G]
  size_t act;        // SwiGLU rows [A][I]: f32 (f32 weights) or bf16 (bf16 weights); none for fp8 / fp4
  size_t act_q;      // fp8 / fp4: e4m3 SwiGLU rows [A][I]
  size_t act_s;      // fp8 / fp4: their scales [A][I/128]
  size_t x_q, x_s;   // fp8 / fp4: e4m3 hidden rows [T][H] and scales [T][H/128]
  size_t acc, slots, total;
};

size_t up256(size_t v) { return (v + 255) & ~size_t(255); }

Layout make_layout(const moe_problem& p) {
  const size_t A = (size_t)p.T * p.k, E = p.E, T = (size_t)p.T, H = p.H, I = p.I;
  Layout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = up256(o + bytes);
    return at;
  };
  L.bad = take(4);
  L.counts = take(4 * E);
  L.offsets = take(4 * (E + 1));
  L.mt = take(4 * (E + 1));
  L.perm = take(4 * A);
  L.inv = take(4 * A);
  L.route_part = take(4 * (E + 1) * (size_t)kRouteMaxChunks);
  const bool fp8 = quant_acts(p);
  // (fp8 / fp4: the gate_up kernels write e4m3 codes and scales only, no float rows)
  L.act = fp8 ? o : take((p.weight_dtype == MOE_BF16 ? 2 : 4) * A * I);
  L.act_q = fp8 ? take(A * I) : o;
  L.act_s = fp8 ? take(4 * A * (I / 128)) : o;
  L.x_q = fp8 ? take(T * H) : o;
  L.x_s = fp8 ? take(4 * T * (H / 128)) : o;
  const bool det = slot_combine(p);
  L.acc = det ? o : take(4 * T * H);
  const bool rows16 = slot_rows_bf16(p, make_plan(p).path == kDecode);
  L.slots = det ? take((rows16 ? 2 : 4) * A * H) : o;
  L.total = o;
  return L;
}

// ---------------------------------------------------------------------------- device

moe_status device_record(DeviceRecord** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_devices_mu);
  DeviceRecord& r = g_devices[dev];
  if (!r.ready) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return MOE_ERR_HIP;
    r.cus = cus > 0 ? cus : 1;
    r.ready = true;
  }
  *out = &r;
  return MOE_OK;
}

int id_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b;
}

int persistent_grid(int cus, int per_cu, int64_t max_items) {
  int64_t g = (int64_t)cus * per_cu;
  if (max_items < g) g = max_items;
  g = (g + 7) / 8 * 8;
  return (int)(g < 8 ? 8 : g);
}

// per-thread stage-event hook (moe_set_stage_events)
thread_local hipEvent_t t_stage_events[2 * MOE_STAGE_COUNT] = {};
thread_local bool t_stage_hook = false;

hipError_t stage_mark(int stage, int edge, hipStream_t s) {
  if (!t_stage_hook) return hipSuccess;
  hipEvent_t ev = t_stage_events[2 * stage + edge];
  return ev ? hipEventRecord(ev, s) : hipSuccess;
}

#define MOE_HIP_CHECK(expr)                  \
  do {                                       \
    if ((expr) != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL_ARG: return "null argument";
    case MOE_ERR_BAD_SHAPE: return "bad shape, size or alignment";
    case MOE_ERR_UNSUPPORTED: return "unsupported dtype, scale format or flag combination";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case MOE_ERR_BAD_INDEX: return "expert id outside [0, E)";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

moe_status moe_workspace_size(const moe_problem* p, size_t* bytes) {
  const moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (!bytes) return MOE_ERR_NULL_ARG;
  *bytes = make_layout(*p).total;
  return MOE_OK;
}

moe_status moe_plan_describe(const moe_problem* p, char* buf, size_t len) {
  const moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (!buf || len == 0) return MOE_ERR_NULL_ARG;
  const Plan pl = make_plan(*p);
  const Layout L = make_layout(*p);
  const char* wname = p->weight_dtype == MOE_F32    ? "f32"
                      : p->weight_dtype == MOE_BF16 ? "bf16"
                      : is_fp4(*p)                  ? "fp4_e2m1"
                                                    : "fp8_e4m3";
  const char* sname = p->scale_fmt == MOE_SCALE_F32 ? "f32" : (p->scale_fmt == MOE_SCALE_UE8M0 ? "ue8m0" : "none");
  const char* kern = pl.path == kDecode ? "stream_16tok_mfma16x16x32_lds_dma_ring3"
                     : p->weight_dtype == MOE_F32 ? "fma_64x64"
                     : p->weight_dtype == MOE_BF16 ? "mfma32x32x16_bf16_160x256_k64_lds_dma_ring3"
                     : is_fp4(*p) ? "mfma16x16x128_e4m3xe2m1_scaled_128x256_ring3"
                                  : "mfma16x16x128_e4m3_scaled_128x256_ring3";
  const char* gname = (p->flags & MOE_FLAG_ACT_GELU) ? "geglu" : ((p->flags & MOE_FLAG_ACT_RELU) ? "reglu" : "swiglu");
  const int n = snprintf(buf, len, "path=%s weights=%s scales=%s kernels=%s activation=%s combine=%s workspace_bytes=%zu",
                         pl.path == kDecode ? "decode" : "grouped", wname, sname, kern, gname,
                         slot_combine(*p) ? (slot_rows_bf16(*p, pl.path == kDecode) ? "slot_rows_bf16" : "slot_rows_f32")
                                          : "atomic_f32", L.total);
  if (quant_acts(*p) && n > 0 && (size_t)n < len)
    snprintf(buf + n, len - n, " act_codes_offset=%zu act_scales_offset=%zu", L.act_q, L.act_s);
  return MOE_OK;
}

moe_status moe_route(const moe_problem* p, const int32_t* topk_idx, int32_t* counts, int32_t* offsets, int32_t* perm,
                     int32_t* inv, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (!counts || !offsets || !workspace) return MOE_ERR_NULL_ARG;
  if (p->T > 0 && (!topk_idx || !perm || !inv)) return MOE_ERR_NULL_ARG;
  if (!aligned4(topk_idx) || !aligned4(counts) || !aligned4(offsets) || !aligned4(perm) || !aligned4(inv) ||
      !aligned16(workspace))
    return MOE_ERR_BAD_SHAPE;
  const Layout L = make_layout(*p);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  DeviceRecord* dev = nullptr;
  if ((st = device_record(&dev)) != MOE_OK) return st;
  (void)hipGetLastError();  // see moe_experts_forward
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  RouteArgs r{};
  r.idx = topk_idx;
  r.A = (int)(p->T * p->k);
  r.E = p->E;
  r.id_bits = id_bits(p->E);
  r.counts = counts;
  r.offsets = offsets;
  r.perm = perm;
  r.inv = inv;
  r.bad = reinterpret_cast<int32_t*>(ws + L.bad);
  r.part = reinterpret_cast<int32_t*>(ws + L.route_part);
  MOE_HIP_CHECK(launch_route(r, s));
  if (p->flags & MOE_FLAG_CHECK_INDICES) {
    int32_t bad = 0;
    MOE_HIP_CHECK(hipMemcpyAsync(&bad, r.bad, 4, hipMemcpyDeviceToHost, s));
    MOE_HIP_CHECK(hipStreamSynchronize(s));
    if (bad) return MOE_ERR_BAD_INDEX;
  }
  return MOE_OK;
}

moe_status moe_route_logits(const moe_problem* p, const float* logits, int renorm, int32_t* topk_idx,
                            float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* inv, void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (p->k > 64) return MOE_ERR_UNSUPPORTED;
  if (!counts || !offsets || !workspace) return MOE_ERR_NULL_ARG;
  if (p->T > 0 && (!logits || !topk_idx || !topk_w || !perm || !inv)) return MOE_ERR_NULL_ARG;
  if (!aligned4(logits) || !aligned4(topk_idx) || !aligned4(topk_w) || !aligned4(counts) || !aligned4(offsets) ||
      !aligned4(perm) || !aligned4(inv) || !aligned16(workspace))
    return MOE_ERR_BAD_SHAPE;
  const Layout L = make_layout(*p);
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  DeviceRecord* dev = nullptr;
  if ((st = device_record(&dev)) != MOE_OK) return st;
  (void)hipGetLastError();  // see moe_experts_forward
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  RouteArgs r{};
  r.idx = topk_idx;
  r.A = (int)(p->T * p->k);
  r.E = p->E;
  r.id_bits = id_bits(p->E);
  r.counts = counts;
  r.offsets = offsets;
  r.perm = perm;
  r.inv = inv;
  r.bad = reinterpret_cast<int32_t*>(ws + L.bad);
  r.part = reinterpret_cast<int32_t*>(ws + L.route_part);
  r.logits = logits;
  r.k = p->k;
  r.renorm = renorm != 0;
  r.idx_out = topk_idx;
  r.w_out = topk_w;
  MOE_HIP_CHECK(launch_route(r, s));   // (T = 0: zero counts and offsets only)
  return MOE_OK;
}

}  // extern "C"

namespace moe {
namespace {

// Host-side checks of a forward call that need no HIP call (workspace size aside).
moe_status check_forward_args(const moe_problem* p, const void* hidden, const int32_t* topk_idx, const float* topk_w,
                              const void* w_gate_up, const void* w_down, const void* w_gate_up_scale,
                              const void* w_down_scale, const void* out) {
  moe_status st = validate_problem(p);
  if (st != MOE_OK) return st;
  if (p->T == 0) return MOE_OK;
  if (!hidden || !topk_idx || !topk_w || !w_gate_up || !w_down || !out) return MOE_ERR_NULL_ARG;
  if (quant_acts(*p) && (!w_gate_up_scale || !w_down_scale)) return MOE_ERR_NULL_ARG;
  if (!aligned16(hidden) || !aligned16(w_gate_up) || !aligned16(w_down) || !aligned16(out) || !aligned4(topk_idx) ||
      !aligned4(topk_w) || !aligned4(w_gate_up_scale) || !aligned4(w_down_scale))
    return MOE_ERR_BAD_SHAPE;
  if ((p->flags & MOE_FLAG_FORCE_DECODE) && !decode_capable(*p)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// The forward's launches, arguments already checked (check_forward_args, T > 0) and the
// workspace (16-byte aligned) holding at least make_layout(*p).total bytes.  Everything it
// reads from the workspace is written first by its own kernels, so the workspace's
// previous contents do not matter.
moe_status forward_launch(const moe_problem* p, const void* hidden, const int32_t* topk_idx, const float* topk_w,
                          const void* w_gate_up, const void* w_down, const void* w_gate_up_scale,
                          const void* w_down_scale, void* out, void* workspace, DeviceRecord* dev, void* stream) {
  const bool fp8 = quant_acts(*p);     // e4m3 activation rows (fp8 and fp4 weights)
  const bool fp4 = is_fp4(*p);
  const Layout L = make_layout(*p);
  const Plan pl = make_plan(*p);
  // launch errors are read with hipGetLastError(); drop an error left behind by an
  // earlier, unrelated HIP call on this thread so it is not reported as ours
  (void)hipGetLastError();
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const int64_t A = p->T * p->k;
  const bool det = slot_combine(*p);   // per-slot rows + slot-order sum (else float atomics)
  const bool f32 = p->weight_dtype == MOE_F32;

  int32_t* bad = reinterpret_cast<int32_t*>(ws + L.bad);
  int32_t* offsets = reinterpret_cast<int32_t*>(ws + L.offsets);
  int32_t* mt = reinterpret_cast<int32_t*>(ws + L.mt);
  int32_t* perm = reinterpret_cast<int32_t*>(ws + L.perm);
  int32_t* inv = reinterpret_cast<int32_t*>(ws + L.inv);
  float* acc = det ? nullptr : reinterpret_cast<float*>(ws + L.acc);
  float* slots = det ? reinterpret_cast<float*>(ws + L.slots) : nullptr;
  const bool rows16 = slot_rows_bf16(*p, pl.path == kDecode);   // (slots then holds bf16 bits)

  // the atomic combine adds into a cleared float32 accumulator; the bf16 grouped
  // gate_up kernel clears it itself after its tiles, other paths launch a fill
  const bool zero_in_gateup = !det && pl.path != kDecode && p->weight_dtype == MOE_BF16;
  if (!det && !zero_in_gateup) {
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_ZERO, 0, s));
    MOE_HIP_CHECK(launch_zero_f32(acc, p->T * (int64_t)p->H, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_ZERO, 1, s));
  }

  RouteArgs r{};
  r.idx = topk_idx;
  r.A = (int)A;
  r.E = p->E;
  r.id_bits = id_bits(p->E);
  r.counts = reinterpret_cast<int32_t*>(ws + L.counts);
  r.offsets = offsets;
  r.perm = perm;
  r.inv = inv;
  r.bad = bad;
  r.bm0 = pl.bm;
  r.mt0 = mt;
  r.part = reinterpret_cast<int32_t*>(ws + L.route_part);
  if (pl.path != kDecode) {   // (the decode kernels route in LDS themselves)
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_ROUTE, 0, s));
    MOE_HIP_CHECK(launch_route(r, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_ROUTE, 1, s));
  }

  GroupedArgs g{};
  g.E = p->E;
  g.gate = (p->flags & MOE_FLAG_ACT_GELU) ? kGateGelu : ((p->flags & MOE_FLAG_ACT_RELU) ? kGateRelu : kGateSilu);
  g.offsets = offsets;
  g.mt = mt;
  // grouped GEMM items in blocks of 8 M tiles x 4 N tiles (the 32 workgroups of an XCD in
  // one round): measured on the DeepSeek-shaped bf16 layer, the same time as M-fastest order
  // (7.57-7.62 ms per step for blocks of 0, 4, 8 and 16 M tiles) with fewer operand fetches
  // beyond L2
  g.item_mb = 8;
  g.I = p->I;
  g.H = p->H;
  g.k = p->k;
  g.perm = perm;
  g.topk_w = topk_w;
  g.acc_out = acc;
  g.slot_out = slots;
  g.slot_bf16 = rows16;
  g.b_scale_ue8m0 = p->scale_fmt == MOE_SCALE_UE8M0;

  // gate_up + SwiGLU: rows = hidden rows gathered through perm (token = slot / k)
  GroupedArgs gu = g;
  gu.a = fp8 ? (const void*)(ws + L.x_q) : hidden;
  gu.a_scale = fp8 ? reinterpret_cast<const float*>(ws + L.x_s) : nullptr;
  gu.a_rows = perm;
  gu.a_row_div = p->k;
  gu.lda = p->H;
  gu.b = w_gate_up;
  gu.b_scale = w_gate_up_scale;
  gu.b_rows = 2 * p->I;
  gu.b_expert_stride = 2 * (int64_t)p->I * p->H / (fp4 ? 2 : 1);   // (fp4: bytes)
  gu.K = p->H;
  gu.act_out = fp8 ? (void*)(ws + L.act_q) : (void*)(ws + L.act);
  gu.act_scale_out = fp8 ? reinterpret_cast<float*>(ws + L.act_s) : nullptr;
  if (zero_in_gateup) {
    gu.zero_out = acc;
    gu.zero_n4 = p->T * (int64_t)p->H / 4;   // H is a multiple of 128
  }
  // down + routing weight + combine: rows = SwiGLU rows in sorted order
  GroupedArgs dn = g;
  dn.a = fp8 ? (const void*)(ws + L.act_q) : (const void*)(ws + L.act);
  dn.a_scale = fp8 ? reinterpret_cast<const float*>(ws + L.act_s) : nullptr;
  dn.a_rows = nullptr;
  dn.a_row_div = 1;
  dn.lda = p->I;
  dn.b = w_down;
  dn.b_scale = w_down_scale;
  dn.b_rows = p->H;
  dn.b_expert_stride = (int64_t)p->H * p->I / (fp4 ? 2 : 1);
  dn.K = p->I;

  if (fp8) {
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_QUANT_X, 0, s));
    MOE_HIP_CHECK(launch_quant_rows_bf16(hidden, p->T, p->H, reinterpret_cast<uint8_t*>(ws + L.x_q),
                                         reinterpret_cast<float*>(ws + L.x_s), s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_QUANT_X, 1, s));
  }

  if (pl.path == kDecode) {
    gu.NT = p->I / decode_gateup_cols();
    dn.NT = p->H / decode_down_cols();
    gu.topk_idx = dn.topk_idx = topk_idx;
    gu.A_slots = dn.A_slots = (int)A;
    gu.inv_out = inv;   // for the slot-order combine
    gu.bad_out = bad;
    const int64_t passes = max_mtiles(A, p->E, decode_bm());
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 0, s));
    MOE_HIP_CHECK(launch_decode_gateup(gu, persistent_grid(dev->cus, decode_groups_per_cu(), passes * gu.NT), s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 1, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 0, s));
    MOE_HIP_CHECK(launch_decode_down(dn, persistent_grid(dev->cus, decode_groups_per_cu(), passes * dn.NT), s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 1, s));
  } else if (f32) {
    gu.NT = p->I / 32;
    dn.NT = p->H / 64;
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 0, s));
    MOE_HIP_CHECK(launch_gateup_f32(gu, max_mtiles(A, p->E, pl.bm) * gu.NT, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 1, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 0, s));
    MOE_HIP_CHECK(launch_down_f32(dn, max_mtiles(A, p->E, pl.bm) * dn.NT, s));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 1, s));
  } else {
    const int gu_cols = fp4 ? gateup_fp4_cols() : (fp8 ? gateup_fp8_cols() : gateup_bf16_cols());
    const int dn_cols = fp4 ? down_fp4_cols() : (fp8 ? down_fp8_cols() : down_bf16_cols());
    gu.NT = (p->I + gu_cols - 1) / gu_cols;
    dn.NT = (p->H + dn_cols - 1) / dn_cols;
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 0, s));
    const int gu_grid = persistent_grid(dev->cus, 1, max_mtiles(A, p->E, pl.bm) * gu.NT);
    MOE_HIP_CHECK(fp4 ? launch_gateup_fp4(gu, gu_grid, s)
                      : (fp8 ? launch_gateup_fp8(gu, gu_grid, s) : launch_gateup_bf16(gu, gu_grid, s)));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_GATE_UP, 1, s));   // (fp8 / fp4: a quantised in its epilogue)
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 0, s));
    const int dn_grid = persistent_grid(dev->cus, 1, max_mtiles(A, p->E, pl.bm) * dn.NT);
    MOE_HIP_CHECK(fp4 ? launch_down_fp4(dn, dn_grid, s)
                      : (fp8 ? launch_down_fp8(dn, dn_grid, s) : launch_down_bf16(dn, dn_grid, s)));
    MOE_HIP_CHECK(stage_mark(MOE_STAGE_DOWN, 1, s));
  }

  const int out_bf16 = p->act_dtype == MOE_BF16;
  MOE_HIP_CHECK(stage_mark(MOE_STAGE_FINALIZE, 0, s));
  if (det && rows16)
    MOE_HIP_CHECK(launch_finalize_slots_bf16(reinterpret_cast<const uint16_t*>(slots), inv, out, p->T, p->k, p->H,
                                             out_bf16, s));
  else if (det) MOE_HIP_CHECK(launch_finalize_slots(slots, inv, out, p->T, p->k, p->H, out_bf16, s));
  else MOE_HIP_CHECK(launch_finalize_acc(acc, out, p->T, p->H, out_bf16, s));
  MOE_HIP_CHECK(stage_mark(MOE_STAGE_FINALIZE, 1, s));

  if (p->flags & MOE_FLAG_CHECK_INDICES) {
    int32_t nbad = 0;
    MOE_HIP_CHECK(hipMemcpyAsync(&nbad, bad, 4, hipMemcpyDeviceToHost, s));
    MOE_HIP_CHECK(hipStreamSynchronize(s));
    if (nbad) return MOE_ERR_BAD_INDEX;
  }
  return MOE_OK;
}

// ---------------------------------------------------------------------------- allocation-free forward
// The workspace of moe_experts_forward_noalloc: a file-scope device array, one copy per GPU,
// held for the life of the process.  Host code never passes the array's name to a kernel or
// a copy (on the host it names a stand-in, not device memory); it uses the device address
// that hipGetSymbolAddress returns, looked up once per device and kept in g_scratch.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

struct ScratchRecord {
  bool ready = false;
  void* ptr = nullptr;
};
ScratchRecord g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

moe_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  ScratchRecord& r = g_scratch[dev];
  if (!r.ready) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return MOE_ERR_HIP;
    r.ptr = ptr;
    r.ready = true;
  }
  *out = r.ptr;
  return MOE_OK;
}

}  // namespace
}  // namespace moe

extern "C" {

moe_status moe_experts_forward(const moe_problem* p, const void* hidden, const int32_t* topk_idx, const float* topk_w,
                               const void* w_gate_up, const void* w_down, const void* w_gate_up_scale,
                               const void* w_down_scale, void* out, void* workspace, size_t workspace_bytes,
                               void* stream) {
  moe_status st = check_forward_args(p, hidden, topk_idx, topk_w, w_gate_up, w_down, w_gate_up_scale, w_down_scale,
                                     out);
  if (st != MOE_OK || p->T == 0) return st;
  if (!workspace) return MOE_ERR_NULL_ARG;
  if (!aligned16(workspace)) return MOE_ERR_BAD_SHAPE;
  if (workspace_bytes < make_layout(*p).total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  DeviceRecord* dev = nullptr;
  if ((st = device_record(&dev)) != MOE_OK) return st;
  return forward_launch(p, hidden, topk_idx, topk_w, w_gate_up, w_down, w_gate_up_scale, w_down_scale, out, workspace,
                        dev, stream);
}

size_t moe_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

moe_status moe_experts_forward_noalloc(const moe_problem* p, const void* hidden, const int32_t* topk_idx,
                                       const float* topk_w, const void* w_gate_up, const void* w_down,
                                       const void* w_gate_up_scale, const void* w_down_scale, void* out,
                                       void* stream) {
  moe_status st = check_forward_args(p, hidden, topk_idx, topk_w, w_gate_up, w_down, w_gate_up_scale, w_down_scale,
                                     out);
  if (st != MOE_OK || p->T == 0) return st;
  if (make_layout(*p).total > kNoAllocScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  DeviceRecord* dev = nullptr;
  if ((st = device_record(&dev)) != MOE_OK) return st;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != MOE_OK) return st;
  return forward_launch(p, hidden, topk_idx, topk_w, w_gate_up, w_down, w_gate_up_scale, w_down_scale, out, ws, dev,
                        stream);
}

moe_status moe_set_stage_events(void* const* events, int n) {
  if (events == nullptr || n == 0) {
    t_stage_hook = false;
    for (auto& e : t_stage_events) e = nullptr;
    return MOE_OK;
  }
  if (n != 2 * MOE_STAGE_COUNT) return MOE_ERR_BAD_SHAPE;
  for (int i = 0; i < n; ++i) t_stage_events[i] = static_cast<hipEvent_t>(events[i]);
  t_stage_hook = true;
  return MOE_OK;
}

moe_status moe_quantize_rows_fp8(const void* x_bf16, int64_t rows, int32_t cols, uint8_t* q, float* scales,
                                 void* stream) {
  if (rows < 0 || cols <= 0 || cols % 128 != 0) return MOE_ERR_BAD_SHAPE;
  if (rows == 0) return MOE_OK;
  if (!x_bf16 || !q || !scales) return MOE_ERR_NULL_ARG;
  if (!aligned16(x_bf16) || (reinterpret_cast<uintptr_t>(q) & 7u) || !aligned4(scales)) return MOE_ERR_BAD_SHAPE;
  (void)hipGetLastError();  // see moe_experts_forward
  MOE_HIP_CHECK(launch_quant_rows_bf16(x_bf16, rows, cols, q, scales, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

moe_status moe_check_mfma_blocks(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* b_scale, float* d,
                                 int nblocks, void* stream) {
  if (fmt < 0 || fmt > 2) return MOE_ERR_UNSUPPORTED;
  if (nblocks < 0) return MOE_ERR_BAD_SHAPE;
  if (nblocks == 0) return MOE_OK;
  if (!a || !b || !d || (fmt != 0 && !b_scale)) return MOE_ERR_NULL_ARG;
  if (!aligned16(a) || !aligned16(b) || !aligned4(d)) return MOE_ERR_BAD_SHAPE;
  (void)hipGetLastError();  // see moe_experts_forward
  MOE_HIP_CHECK(launch_mfma_block_check(a, b, b_scale, d, nblocks, fmt, static_cast<hipStream_t>(stream)));
  return MOE_OK;
}

}  // extern "C"
