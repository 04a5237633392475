/*
 * moe_experts.h -- C ABI of the MI355X (gfx950) routed top-k experts forward.
 *
 * What is computed (Hugging Face Transformers docs, "Experts backends" page,
 * introduction): for each token a router has chosen k experts; the token's hidden
 * state is projected through each chosen expert and the k results are summed with
 * the routing weights.  The expert is a gated MLP -- gate/up projection, SwiGLU,
 * down projection (same page, backend table "deepgemm_megamoe" row and the
 * "SonicMoE" section, where silu maps to SwiGLU):
 *
 *     out[t,:] = sum_{j<k} w[t,j] * W_down[e] ( silu(W_gate[e] x_t) * (W_up[e] x_t) ),
 *     e = idx[t,j],  silu(z) = z / (1 + exp(-z)).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers, row-major, contiguous, 16-byte
 *     aligned, owned by the caller.  The library never frees or retains them.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns without waiting, except where stated.
 *   - Every argument is validated on the host before the first HIP call; on a
 *     validation error nothing is enqueued and no output is written.
 *   - The library allocates no device memory per call: scratch comes from the
 *     caller's workspace (size from moe_workspace_size).  Its only state is a
 *     lazily built per-device record (CU count), made on the first call on a
 *     device (the page's "DeepGEMM" section loads its kernel lazily as well).
 *   - Calls on one stream are ordered; two calls that share a workspace must not
 *     overlap in time.
 */
#ifndef MOE_EXPERTS_H
#define MOE_EXPERTS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 1

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL_ARG = 1,            /* a required pointer is NULL                     */
  MOE_ERR_BAD_SHAPE = 2,           /* sizes out of range / not multiples / misaligned */
  MOE_ERR_UNSUPPORTED = 3,         /* dtype / scale-format combination not provided  */
  MOE_ERR_WORKSPACE_TOO_SMALL = 4, /* workspace_bytes < moe_workspace_size()         */
  MOE_ERR_BAD_INDEX = 5,           /* an expert id outside [0, E) (CHECK_INDICES)    */
  MOE_ERR_HIP = 6                  /* a HIP runtime call failed                      */
} moe_status;

typedef enum {
  MOE_F32 = 0,      /* IEEE binary32                                   */
  MOE_BF16 = 1,     /* bfloat16                                        */
  MOE_FP8_E4M3 = 2, /* OCP 8-bit E4M3 ("e4m3fn": max 448, no infinity) */
  MOE_FP4_E2M1 = 3  /* OCP 4-bit E2M1 (MX FP4: max 6), two codes per byte     */
} moe_dtype;

typedef enum {
  MOE_SCALE_NONE = 0,
  MOE_SCALE_F32 = 1,   /* fp8: one float32 scale per 128x128 weight block          */
  MOE_SCALE_UE8M0 = 2  /* one uint8 exponent b per block, scale = 2^(b-127); the
                          block is 128x128 for fp8 weights and 1x32 (one weight
                          row, 32 consecutive input channels) for fp4 weights      */
} moe_scale_fmt;

enum {
  /* Synchronise `stream` after the forward and return MOE_ERR_BAD_INDEX if any
   * topk_idx entry was outside [0, E).  Without it such a slot contributes
   * nothing and the call still returns MOE_OK. */
  MOE_FLAG_CHECK_INDICES = 1u,
  /* Bit-reproducible combine at every size: each slot's weighted expert output is
   * written to its own row and the k rows of a token are summed in slot order.
   * Without the flag this combine is used while the slot rows are small (float32
   * rows, 4*T*k*H bytes, at most 512 MiB; the bf16 rows of a bf16, fp8 or fp4 layer
   * on the grouped path, 2*T*k*H bytes, at most 1 GiB), and floating-point atomic adds
   * into a [T, H] accumulator above (or always with MOE_FLAG_ATOMIC_COMBINE). */
  MOE_FLAG_DETERMINISTIC = 2u,
  /* Path selection (both give the same result within tolerance): the grouped
   * path sorts slots by expert and runs grouped GEMMs; the decode path streams
   * each selected expert's weights once against its few tokens.  Default: decode
   * when T * k <= min(16 * E, 512) (at most one 16-row pass per expert on average)
   * and the decode path takes the problem, grouped otherwise.  The decode path takes bf16 weights with
   * I % 128 == 0 and T * k <= 2048 (its routing tables live in LDS); forcing it
   * on any other problem returns MOE_ERR_UNSUPPORTED. */
  MOE_FLAG_FORCE_GROUPED = 4u,
  MOE_FLAG_FORCE_DECODE = 8u,
  /* Combine with floating-point atomic adds into a float32 [T, H] accumulator at
   * every size (the smaller workspace); not with MOE_FLAG_DETERMINISTIC. */
  MOE_FLAG_ATOMIC_COMBINE = 16u,
  /* The gated activation a = gate(g) * u of the expert MLP (SonicMoE section: gated
   * activations silu, gelu or relu map to SwiGLU, GeGLU or ReGLU).  Default: SwiGLU,
   * gate = silu.  GELU: gate = GELU in its exact form z * Phi(z).  RELU: gate =
   * max(z, 0).  At most one of the two. */
  MOE_FLAG_ACT_GELU = 32u,
  MOE_FLAG_ACT_RELU = 64u
};

/* Problem description (plain values; no pointers). */
typedef struct {
  int64_t T;            /* tokens, >= 0                                              */
  int32_t H;            /* hidden size                                               */
  int32_t I;            /* expert intermediate size                                  */
  int32_t E;            /* number of experts, 1..1024                                */
  int32_t k;            /* experts per token, 1..E                                   */
  int32_t act_dtype;    /* moe_dtype of hidden and out: MOE_F32 or MOE_BF16          */
  int32_t weight_dtype; /* moe_dtype of the weights: MOE_F32 (with act MOE_F32),
                           MOE_BF16 (with act MOE_BF16), MOE_FP8_E4M3 or
                           MOE_FP4_E2M1 (act MOE_BF16)                               */
  int32_t scale_fmt;    /* moe_scale_fmt: != NONE exactly when weights are fp8 or
                           fp4; fp4 takes MOE_SCALE_UE8M0 only                       */
  uint32_t flags;       /* MOE_FLAG_*                                                */
} moe_problem;

/* Shape rules checked by every call taking a moe_problem:
 *   H % 128 == 0, I % 64 == 0 (f32, bf16 weights); H % 128 == 0, I % 128 == 0 (fp8, fp4);
 *   1 <= E <= 1024, 1 <= k <= E, T * k < 2^31, H, I <= 65536, and each of hidden,
 *   the intermediate [T*k, I] rows and one expert's W_gate_up below 4 GiB.            */

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status s);

/* Bytes of device workspace moe_experts_forward needs for problem *p (host only,
 * closed form, no HIP call).  The page's backend table sets the memory of the
 * "grouped_mm" row (tokens sorted by expert, activations of the selected experts
 * only) against the "batched_mm" row (the selected experts' parameters duplicated
 * per token); this sizes the grouped form's buffers, which hold the sorted slots
 * and their activations, never a copy of a weight.  Grows with T*k*(I + H) and T*H.
 * Errors: NULL_ARG (p or bytes NULL), BAD_SHAPE / UNSUPPORTED as for the forward.  When the k rows of a
 * token are combined as per-slot rows (always with MOE_FLAG_DETERMINISTIC; by default
 * while 4*T*k*H <= 512 MiB, or 2*T*k*H <= 1 GiB for a bf16, fp8 or fp4 layer, where that combine is
 * the faster one; never with MOE_FLAG_ATOMIC_COMBINE) it holds a [T*k, H] buffer instead
 * of the float32 [T, H]
 * accumulator: float32 rows with MOE_FLAG_DETERMINISTIC, and bf16 rows (each slot's
 * weighted row rounded once, the k rows summed in float32) on the default grouped path
 * of bf16, fp8 and fp4 layers. */
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/*
 * The routed top-k experts forward.
 *
 *   hidden          [T, H]        act_dtype
 *   topk_idx        [T, k] int32  chosen expert ids, 0 <= id < E (a repeated id in
 *                                 one row counts once per slot)
 *   topk_w          [T, k] float32 routing weights (used as given; no renormalising)
 *   w_gate_up       [E, 2I, H]    weight_dtype; rows [0, I) of expert e are the gate
 *                                 projection, rows [I, 2I) the up projection
 *   w_down          [E, H, I]     weight_dtype
 *   w_gate_up_scale [E, 2I/128, H/128]  fp8 only: float32, or uint8 for UE8M0; NULL otherwise
 *   w_down_scale    [E, H/128, I/128]   fp8 only; NULL otherwise
 *                   fp4 weights instead: w_gate_up [E, 2I, H/2] and w_down [E, H, I/2]
 *                   uint8, byte j of a row holding element 2j in its low nibble and
 *                   2j + 1 in its high nibble; UE8M0 scales w_gate_up_scale [E, 2I, H/32],
 *                   w_down_scale [E, H, I/32] (uint8, 4-byte aligned)
 *   out             [T, H]        act_dtype; overwritten (never accumulated into)
 *   workspace       device scratch of workspace_bytes >= moe_workspace_size(p)
 *
 * fp8 weights (page section "FP8 and FP4 quantized experts" and its note: float32
 * or UE8M0 block scales consumed directly; dynamic per-row activation scales):
 * the bf16 hidden states are quantised per token and per 128 channels to e4m3
 * with a float32 scale amax/448, and so is the SwiGLU output before the down
 * projection; weight block (r, c) dequantises to code * scale[r/128][c/128].
 * fp4 weights (same section: packed two per int8 with UE8M0 scales, DeepSeek-V4
 * style): the activations are quantised exactly as for fp8, and weight (r, c)
 * dequantises to e2m1(code) * 2^(scale[r][c/32] - 127).
 *
 * Returns MOE_OK once the work is enqueued (T == 0: nothing is enqueued).
 * Errors: NULL_ARG, BAD_SHAPE, UNSUPPORTED, WORKSPACE_TOO_SMALL before any HIP
 * call; BAD_INDEX only with MOE_FLAG_CHECK_INDICES (after a stream sync); HIP.
 *
 * Stream capture: without MOE_FLAG_CHECK_INDICES the call only launches kernels on
 * `stream` (no host wait, no memset, no allocation), with grids fixed by T, k, E, H
 * and I, so it can be captured into a HIP graph once (after one call outside the
 * capture on the device) and replayed for any ids and weights written into the same
 * buffers.
 */
moe_status moe_experts_forward(const moe_problem* p, const void* hidden, const int32_t* topk_idx,
                               const float* topk_w, const void* w_gate_up, const void* w_down,
                               const void* w_gate_up_scale, const void* w_down_scale, void* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * The forward without a workspace argument and without any allocation, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * moe_experts_forward, minus workspace and workspace_bytes: the workspace is a device
 * array inside the library of moe_noalloc_scratch_bytes() bytes (128 MiB), one copy per
 * GPU, held until the process ends (looked up once per device on its first call).
 * Problems whose moe_workspace_size exceeds it return MOE_ERR_WORKSPACE_TOO_SMALL before
 * any HIP call (the Qwen1.5-MoE-A2.7B-shaped prefill layer, T = 4096, needs 108 MiB; the
 * DeepSeek-V3-shaped layers need more: use moe_experts_forward for them).  The call makes
 * no hipMalloc, hipFree or other allocation.  Every call on one GPU uses that GPU's one
 * array: calls that overlap on one GPU (on different streams, or from different host
 * threads without ordering) race and may produce wrong results; calls ordered on one
 * stream are safe.  The array keeps the last call's contents; nothing the forward reads
 * from it needs to start at zero.
 */
moe_status moe_experts_forward_noalloc(const moe_problem* p, const void* hidden, const int32_t* topk_idx,
                                       const float* topk_w, const void* w_gate_up, const void* w_down,
                                       const void* w_gate_up_scale, const void* w_down_scale, void* out,
                                       void* stream);

/* Bytes of the allocation-free forward's device array (its largest workspace). */
size_t moe_noalloc_scratch_bytes(void);

/*
 * Routing bookkeeping alone: the stable sort of the T*k slots a = t*k + j by
 * chosen expert (page backend table, "grouped_mm" row: tokens are sorted by
 * their selected expert before one grouped GEMM).
 *
 *   counts  [E]   int32  slots choosing expert e
 *   offsets [E+1] int32  exclusive prefix sum of counts (offsets[E] = valid slots)
 *   perm    [T*k] int32  perm[p] = the slot at sorted position p; slots of one
 *                        expert stay in increasing slot order
 *   inv     [T*k] int32  inv[perm[p]] = p; -1 for a slot whose id is out of range
 *
 * Same workspace rules as moe_experts_forward (size from moe_workspace_size).
 * Out-of-range ids are left out of every output; with MOE_FLAG_CHECK_INDICES
 * the call synchronises and returns MOE_ERR_BAD_INDEX if there were any.
 */
moe_status moe_route(const moe_problem* p, const int32_t* topk_idx, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* inv, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * The router step in front of the routing bookkeeping (Experts backends page,
 * introduction: tokens go to the top-k experts the router scores, and their
 * outputs are combined with the routing weights).  For each token t:
 *   p[e]        = softmax over the E logits of row t (float32: max-shifted expf,
 *                 divided by the sum);
 *   topk_idx[t] = the k experts of largest p in decreasing order, equal logits
 *                 going to the lower expert id (softmax is increasing, so the
 *                 choice is made on the logits themselves, exactly);
 *   topk_w[t]   = their p, divided by the sum of the k when renorm != 0;
 * then the bookkeeping of moe_route on the chosen ids, in the same pass.
 *
 *   logits   [T, E] float32, device; every row needs a finite entry and no NaN
 *   topk_idx [T, k] int32 out;  topk_w [T, k] float32 out
 *   counts, offsets, perm, inv: as moe_route
 *
 * k <= 64 (MOE_ERR_UNSUPPORTED above).  Same workspace rules as moe_route;
 * ids are always in range, so no index check is needed.
 */
moe_status moe_route_logits(const moe_problem* p, const float* logits, int renorm, int32_t* topk_idx,
                            float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* inv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Dynamic per-row e4m3 quantisation (page section "FP8 and FP4 quantized
 * experts": per-row activation scales, static per-tensor scales rejected).
 * For each row and each group of 128 consecutive columns:
 *   amax = max |x| (float32), s = amax / 448 (float32, correctly rounded; 1 if
 *   amax == 0), q = e4m3(x / s) (float32 division, round to nearest even,
 *   saturating at +-448).
 *
 *   x_bf16 [rows, cols] bf16;  q [rows, cols] uint8 e4m3 codes;
 *   scales [rows, cols/128] float32.   cols % 128 == 0, rows >= 0.
 */
moe_status moe_quantize_rows_fp8(const void* x_bf16, int64_t rows, int32_t cols, uint8_t* q,
                                 float* scales, void* stream);

/* Describe the plan chosen for *p into buf (NUL terminated, truncated to len):
 * the path ("grouped" or "decode"), weight and scale formats, activation, combine,
 * tile shapes and workspace bytes.  Host only, no HIP call.  This is the library's
 * counterpart of the page's get_experts_implementation() ("Set an experts backend"
 * section), which reports the experts backend a model will run with; here the
 * choice between the sort-then-group path and the few-token decode path ("Decode
 * stage switch" section) is made per call from T, k, E and the flags, and this
 * reports it.  For fp8 and fp4 weights it also gives act_codes_offset and
 * act_scales_offset: byte offsets into the forward's workspace of the e4m3 SwiGLU
 * rows [T*k][I] (uint8) and their scales [T*k][I/128] (float32), in expert-sorted
 * slot order (the order of moe_route's perm); they hold the last forward's values
 * until the workspace is reused.  Errors: NULL_ARG (p or buf NULL, or len == 0),
 * BAD_SHAPE / UNSUPPORTED as for the forward. */
moe_status moe_plan_describe(const moe_problem* p, char* buf, size_t len);

/*
 * Instruction check (test export): nblocks independent block products on the block-scaled
 * 16x16x128 MFMA that the e4m3 and FP4 grouped kernels use for each 128-long block of
 * their dot products ("FP8 and FP4 quantized experts" section: the fp8 and fp4 expert
 * GEMMs), with the same operand layout and a zero accumulator.  It exists so that the
 * instruction's accumulation can be compared with exact sums; the parity window of the
 * requantised SwiGLU rows rests on that comparison.
 *
 *   fmt 0: a [nblocks][16][128] e4m3 codes, b [nblocks][16][128] e4m3 codes;
 *   fmt 1: a as above, b [nblocks][16][64] bytes of e2m1 codes (element k in the low
 *          nibble of byte k/2 for even k), b_scale [nblocks][16][4] UE8M0 exponents (one
 *          per column and 32-long k block);
 *   fmt 2: a and b as for fmt 0, b_scale [nblocks][16][4] UE8M0 bytes passed as the
 *          instruction's B scales by lane (column, k block) as for fmt 1; only one
 *          exponent per block (all 64 equal, as the e4m3 kernels pass UE8M0 weight
 *          scales) has a defined result;
 *   d [nblocks][16][16] float32 out: d[i][r][n] = sum_k a[i][r][k] * b[i][n][k] (fmt 1:
 *          times 2^(b_scale[i][n][k/32] - 127); fmt 2: times 2^(s - 127), s the block's
 *          exponent).
 * Device pointers; a and b 16-byte aligned.  Errors: UNSUPPORTED (fmt), BAD_SHAPE,
 * NULL_ARG, HIP.  Asynchronous on `stream`.
 */
moe_status moe_check_mfma_blocks(int fmt, const uint8_t* a, const uint8_t* b, const uint8_t* b_scale, float* d,
                                 int nblocks, void* stream);

/* Stages of one forward, in launch order (a stage a path does not use is skipped). */
enum {
  MOE_STAGE_ZERO = 0,      /* clear the float32 accumulator                      */
  MOE_STAGE_ROUTE = 1,     /* routing bookkeeping                                */
  MOE_STAGE_QUANT_X = 2,   /* fp8 only: quantise the hidden states               */
  MOE_STAGE_GATE_UP = 3,   /* gate/up projection + SwiGLU                        */
  MOE_STAGE_QUANT_ACT = 4, /* not launched: fp8 / fp4 gate_up kernels quantise the
                              SwiGLU output in their epilogue                    */
  MOE_STAGE_DOWN = 5,      /* down projection + routing weight + combine         */
  MOE_STAGE_FINALIZE = 6,  /* round the accumulator to the output type           */
  MOE_STAGE_COUNT = 7
};

/*
 * Per-stage timing hook for profilers and benchmarks.  `events` points to
 * 2 * MOE_STAGE_COUNT hipEvent_t handles (entries may be NULL); while set, each
 * later moe_experts_forward on the calling host thread records events[2*s] on its
 * stream just before stage s and events[2*s+1] just after it.  The handles are
 * copied; the caller keeps ownership of the events.  events == NULL (or n == 0)
 * clears the hook.  n must be 0 or 2 * MOE_STAGE_COUNT (else MOE_ERR_BAD_SHAPE).
 */
moe_status moe_set_stage_events(void* const* events, int n);

#ifdef __cplusplus
}
#endif

#endif /* MOE_EXPERTS_H */
