/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts expert layer.
 *
 * The operations follow these documentation pages (cited by title and section):
 *   [StepFun]  "flashinfer.experimental.cake_stepfun_moe": intro (stage list:
 *              routing with Renormalize top-k, FC1 with the StepFun epilogue, FC2,
 *              finalize), "Unified MoE API opt-in" (SwiGLUStep(limit) with a
 *              per-expert clamp limit, default 7.0), "Prepared launches"
 *              (no allocation, no host synchronisation; expanded_idx_to_permuted_idx).
 *   [W4A8]     "flashinfer.fused_moe.cake / cake_cute (MXFP4 SiTU routed MoE)":
 *              "Host plan" (workspace sized from the token count; canonical
 *              [up | gate] w1 bank; tensor layouts; expert parallel arguments).
 *   [GGEMM]    "Cake ragged BF16 grouped GEMM (experimental)": intro and operation
 *              table (fwd / dgrad / wgrad; offs or m_indptr read on the device; no
 *              padding; empty groups give zero weight gradients), "Prepared
 *              launches" (new offsets may be written between launches).
 *   [BGMV]     "flashinfer.fused_moe.prepare_bgmv_moe": signature, Parameters and
 *              description (MoE-LoRA shrink + expand, fixed-order accumulation,
 *              hidden split with a last-workgroup reduction).
 *   [SM90]     "flashinfer.fused_moe.cute_dsl_fused_moe_bf16": formula
 *              out[t] = sum_k scale[t,k] * ffn(x[t]; e[t,k]), "Supported
 *              configuration" (shape rules, num_tokens == 0, EP shard),
 *              Parameters (use_fused_finalize, moe_output).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor argument is a DEVICE pointer to dense row-major memory owned by
 *   the caller; bf16 tensors are passed as `const void*` (IEEE bfloat16 bits).
 *   Tensor pointers are 16-byte aligned (MOE_ERR_ALIGN otherwise): the kernels move
 *   whole 16-byte chunks of rows.
 * - `stream` is a hipStream_t (NULL = the null stream). Work is only enqueued:
 *   no call allocates device or host memory, synchronises the host, or reads
 *   device memory from the host. Outputs are valid once the stream reaches them.
 * - Device data is never validated (that would need a host synchronisation).
 *   Routing ids outside [0, num_experts) are treated as routes to a foreign
 *   expert; non-monotone group offsets are undefined behaviour.
 * - Every call returns moe_status: MOE_OK (0) or an error; on error nothing has
 *   been enqueued, except MOE_ERR_HIP (a launch failed after earlier launches of
 *   the same call were enqueued). Nothing throws, aborts or prints.
 * - Calls keep no state between invocations; concurrent calls on different
 *   streams are safe when their outputs and workspaces are distinct. Exceptions:
 *   moe_tune (which also synchronises its stream) records tile choices in a
 *   per-process table that moe_tune_clear empties and the GEMM stages read, and
 *   moe_ffn_forward_noalloc uses one fixed scratch array per device.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;

#define MOE_OK               0
#define MOE_ERR_NULL         1  /* a required pointer is NULL */
#define MOE_ERR_SHAPE        2  /* a size is negative, zero where it must not be, or breaks a divisibility rule */
#define MOE_ERR_DTYPE        3  /* unknown or unsupported dtype / mode enum */
#define MOE_ERR_ALIGN        4  /* a tensor pointer is not 16-byte aligned */
#define MOE_ERR_UNSUPPORTED  5  /* valid request this library does not serve */
#define MOE_ERR_WORKSPACE    6  /* workspace NULL or smaller than the *_workspace_size query */
#define MOE_ERR_HIP          7  /* a kernel launch failed */
#define MOE_ERR_TOO_LARGE    8  /* moe_ffn_forward_noalloc: the request needs more than its fixed scratch */

/* Element types. */
#define MOE_DTYPE_BF16 0
#define MOE_DTYPE_F32  1

/* Activation applied to the FC1 output h = [up | gate] ([W4A8] Host plan: up rows then gate rows). */
#define MOE_ACT_SWIGLU      0  /* silu(gate) * up  ([SM90] formula) */
#define MOE_ACT_SWIGLU_STEP 1  /* silu(clamp(gate,-L,L)) * clamp(up,-L,L), L per expert ([StepFun]) */

/* How moe_ffn_forward combines the top-k route outputs ([SM90] use_fused_finalize). */
#define MOE_FINALIZE_DETERMINISTIC 0  /* FC2 rows, then the fixed-order fp32 combine (moe_finalize) */
#define MOE_FINALIZE_FUSED         1  /* FC2 epilogue adds w*y into a zeroed output with bf16 atomics */
#define MOE_FINALIZE_NONE          2  /* stop after FC2: return y rows and e2p ([StepFun] do_finalize=False) */

/* Number formats of moe_ffn_forward's operands ([W4A8] Host plan, Inputs). */
#define MOE_WFMT_BF16  0  /* x, w1, w2 in bf16 */
#define MOE_WFMT_MXFP4 1  /* w1, w2 MXFP4 (e2m1 pairs + UE8M0 per 32), x MXFP8 (e4m3 + UE8M0 per 32);
                             the FC1 output is requantized to MXFP8 with the round-up rule */
#define MOE_WFMT_MXFP8 2  /* as MXFP4 but w1, w2 MXFP8: one e4m3fn code byte per element, UE8M0
                             per 32 ([StepFun] intro lists mxfp8 among the weight families) */
#define MOE_WFMT_FP8   3  /* fp8 with per-tensor scales ([StepFun] intro: its list of weight families):
                             x, w1, w2 e4m3fn code bytes; x_sf -> float x_scale [1], w1_sf ->
                             float w1_scale [L], w2_sf -> float w2_scale [L] (value = code value *
                             scale); the FC1 output is requantized with the caller's static
                             act_scale: code = e4m3_rne(clamp(a * (1/act_scale), -448, 448)) */

/* Meaning of a grouped-GEMM offsets array ([GGEMM] intro). */
#define MOE_OFFS_ENDS   0  /* offs[E]: cumulative end row of each group */
#define MOE_OFFS_INDPTR 1  /* m_indptr[E+1]: leading zero, then cumulative ends */

/* Human-readable name of a status code (static string, never NULL). */
const char* moe_status_string(moe_status status);

/* Library version string (static). */
const char* moe_version(void);

/*
 * moe_route -- renormalized top-k routing from logits ([StepFun] intro: routing,
 * Renormalize top-k).
 *   logits        [T, num_experts] float32
 *   topk_ids      [T, top_k] int32 out: slot s holds the expert with the (s+1)-th
 *                 largest logit; equal logits go to the lower expert id
 *   topk_weights  [T, top_k] float32 out: softmax of the selected logits (equal to
 *                 softmax over all experts renormalized over the k selected)
 * Rules: 1 <= num_experts <= 1024, 1 <= top_k <= min(num_experts, 16). T == 0 is a no-op.
 * NaN logits are not supported.
 */
moe_status moe_route(const float* logits, int64_t T, int32_t num_experts, int32_t top_k,
                     int32_t* topk_ids, float* topk_weights, void* stream);

/*
 * moe_sort -- stable, unpadded counting sort of the T*top_k routes by local expert
 * ([GGEMM] intro: consecutive row groups, offs / m_indptr, no padding; [StepFun]
 * Prepared launches: expanded_idx_to_permuted_idx; [SM90] Parameters: EP shard of
 * num_local_experts experts starting at global id local_expert_offset).
 * Expanded index i = t*top_k + s. Route i is local when
 * 0 <= topk_ids[i] < num_experts and 0 <= topk_ids[i]-local_expert_offset < num_local_experts.
 *   offs      [L] int32 out: cumulative end row of each local expert
 *   m_indptr  [L+1] int32 out, may be NULL: [0, offs...]
 *   e2p       [T*top_k] int32 out: permuted row of route i, -1 if foreign
 *   p2e       [T*top_k] int32 out (capacity): p2e[p] = route i of permuted row p,
 *             for p < n_local; entries past n_local are not written
 *   n_local   [1] int32 out: number of local routes
 *   ws        workspace of moe_sort_workspace_size(T, top_k, L) bytes (device)
 * Within an expert, rows keep ascending expanded-index order. T == 0 still writes
 * zero offsets and n_local = 0.
 */
size_t moe_sort_workspace_size(int64_t T, int32_t top_k, int32_t num_local_experts);
moe_status moe_sort(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t num_experts,
                    int32_t num_local_experts, int32_t local_expert_offset,
                    int32_t* offs, int32_t* m_indptr, int32_t* e2p, int32_t* p2e,
                    int32_t* n_local, void* ws, size_t ws_bytes, void* stream);

/*
 * Ragged bf16 grouped GEMMs ([GGEMM] operation table). Group e owns rows
 * [offs[e-1], offs[e]) of the packed row operands (offs[-1] = 0); `offs` is
 * read on the device at every launch. fp32 accumulation in a fixed order (no
 * atomics): results are bitwise reproducible. Rows past the last offset are
 * neither read nor written (wgrad ignores them).
 *   offs_kind  MOE_OFFS_ENDS (offs has E entries) or MOE_OFFS_INDPTR (E+1 entries)
 * Shape rules: E >= 1, N % 32 == 0, K % 32 == 0, sum_m >= 0.
 *
 * grouped_gemm_fwd:   y[r] = x[r] @ w[e].T      x [sum_m,K], w [E,N,K] -> y [sum_m,N] bf16
 * grouped_gemm_dgrad: dx[r] = g[r] @ w[e]       g [sum_m,N], w [E,N,K] -> dx [sum_m,K] bf16
 *                     (w is read in place, not transposed or copied)
 * grouped_gemm_wgrad: dw[e] = g[rows e].T @ x[rows e]  -> dw [E,N,K], out_dtype bf16 or f32;
 *                     an empty group's dw[e] is written as exact zeros.
 * fwd / dgrad ws, ws_bytes (optional, NULL / 0 allowed): the split workspace of moe_fc1 /
 * moe_fc2 (at least moe_gemm_split_workspace_size() bytes, 16-byte aligned, not shared
 * by calls that may overlap). With it, the tiles of a last, mostly idle round of
 * workgroups are cut along the contraction and their fp32 partials summed in a fixed
 * order: the same result on every run, whose rounding differs from the uncut order
 * within fp32 and depends on the tile count. Without it every tile is whole, and each
 * output element's summation order depends only on K (the same bits for a group
 * computed alone or among others). With it and at least 16 groups of at most 384 rows
 * on average, fwd instead runs one workgroup per CU taking whole tiles from a queue
 * (counters in the same workspace): the bits of the call without a workspace.
 */
moe_status grouped_gemm_fwd(const void* x, const void* w, const int32_t* offs, int32_t offs_kind,
                            int32_t E, int64_t sum_m, int32_t N, int32_t K, void* y, void* ws,
                            size_t ws_bytes, void* stream);
moe_status grouped_gemm_dgrad(const void* g, const void* w, const int32_t* offs, int32_t offs_kind,
                              int32_t E, int64_t sum_m, int32_t N, int32_t K, void* dx, void* ws,
                              size_t ws_bytes, void* stream);
size_t grouped_gemm_wgrad_workspace_size(int32_t E, int64_t sum_m, int32_t N, int32_t K,
                                         int32_t out_dtype);
moe_status grouped_gemm_wgrad(const void* g, const void* x, const int32_t* offs, int32_t offs_kind,
                              int32_t E, int64_t sum_m, int32_t N, int32_t K, void* dw,
                              int32_t out_dtype, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_ffn_forward -- the expert layer after routing ([SM90] formula):
 *   out[t] = sum over slots s of topk_weights[t,s] * ffn(x[t]; topk_ids[t,s]),
 *   ffn(x; e) = act(x @ w1[e].T) @ w2[e].T, routes to foreign experts contribute 0.
 * Steps: moe_sort -> FC1 grouped GEMM over gathered x rows with the activation in
 * its epilogue (act rows in bf16) -> FC2 grouped GEMM -> combine per finalize_mode.
 */
typedef struct moe_ffn_desc {
  int64_t T;                  /* tokens (>= 0) */
  int32_t H;                  /* hidden size, H % 64 == 0 */
  int32_t I;                  /* intermediate size, I % 32 == 0 */
  int32_t num_experts;        /* global experts E_g */
  int32_t num_local_experts;  /* L; 0 means num_experts */
  int32_t local_expert_offset;/* global id of local expert 0 */
  int32_t top_k;              /* 1..16 */
  int32_t activation;         /* MOE_ACT_* */
  int32_t finalize_mode;      /* MOE_FINALIZE_* (MXFP4 / MXFP8 / FP8: DETERMINISTIC or NONE) */
  int32_t weight_format;      /* MOE_WFMT_*; MXFP4 / MXFP8 / FP8 need H % 128 == 0, I % 128 == 0 */
} moe_ffn_desc;

typedef struct moe_ffn_tensors {
  const void* x;              /* [T, H] bf16, or e4m3fn codes (MXFP4 / MXFP8 / FP8 formats) */
  const int32_t* topk_ids;    /* [T, top_k] int32 global expert ids */
  const float* topk_weights;  /* [T, top_k] float32, normalized by the caller */
  const void* w1;             /* [L, 2I, H] bf16: rows 0..I-1 up, I..2I-1 gate
                                 (MXFP4: [L, 2I, H/2] bytes, element 2j in the low nibble;
                                 MXFP8, FP8: [L, 2I, H] e4m3fn codes) */
  const void* w2;             /* [L, H, I] bf16 (MXFP4: [L, H, I/2] bytes; MXFP8, FP8: [L, H, I] codes) */
  const float* clamp_limit;   /* [L] float32 SwiGLUStep limits, or NULL for 7.0 */
  void* out;                  /* [T, H] bf16 (DETERMINISTIC / FUSED), fully overwritten */
  void* y;                    /* NONE only: [T*top_k, H] bf16 capacity, FC2 rows in permuted order */
  int32_t* e2p;               /* NONE only (optional otherwise): [T*top_k] int32 */
  const void* x_sf;           /* MXFP4 / MXFP8 formats: [T, H/32] UE8M0 codes (uint8); FP8: float [1] */
  const void* w1_sf;          /* MXFP4 / MXFP8 formats: [L, 2I, H/32] UE8M0; FP8: float [L] */
  const void* w2_sf;          /* MXFP4 / MXFP8 formats: [L, H, I/32] UE8M0; FP8: float [L] */
  const float* act_scale;     /* FP8 only: [1] float32 scale of the requantized FC1 output */
} moe_ffn_tensors;

size_t moe_ffn_workspace_size(const moe_ffn_desc* desc);
moe_status moe_ffn_forward(const moe_ffn_desc* desc, const moe_ffn_tensors* tensors,
                           void* ws, size_t ws_bytes, void* stream);

/*
 * moe_ffn_forward_noalloc -- moe_ffn_forward without a caller workspace, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. Same desc, tensors, kernels and results as
 * moe_ffn_forward (the outputs are bitwise equal); the workspace is instead a fixed
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until
 * the process ends. The call itself allocates nothing. A request whose
 * moe_ffn_workspace_size(desc) exceeds MOE_NOALLOC_SCRATCH_BYTES returns
 * MOE_ERR_TOO_LARGE with nothing enqueued (for bf16 weights the workspace is 64 MiB
 * of split-tile partials plus about (I + H) * 2 bytes per route: e.g. T * top_k up to
 * ~3600 routes at H = 7168, I = 2048). The first call on a device looks up the array's
 * device address (a host-side query, no allocation); a caller that captures graphs
 * makes one call before capturing. Every call on a GPU shares that GPU's array, and
 * nothing needs it cleared between calls (the sort clears the split-tile counters on
 * every call), but calls that overlap in time on one GPU (other streams or threads)
 * race on it: serialise them.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
moe_status moe_ffn_forward_noalloc(const moe_ffn_desc* desc, const moe_ffn_tensors* tensors,
                                   void* stream);

/*
 * The two GEMM stages of moe_ffn_forward as separate calls ([StepFun] One-shot
 * functions: fc1, fc2), for callers that run routing, sort and finalize
 * themselves. `offs` [L] and `p2e` come from moe_sort over the same topk_ids;
 * rows are in permuted (expert-sorted) order and only the first offs[L-1] rows
 * are touched; row capacity is T*top_k.
 *
 * moe_fc1: act[p, :] = activation(x[p2e[p] / top_k] @ w1[e].T) for the rows p of
 *          local expert e. x [T,H] bf16, w1 [L,2I,H] bf16 ([up | gate] rows),
 *          clamp_limit [L] float32 or NULL (7.0) for MOE_ACT_SWIGLU_STEP,
 *          act [T*top_k, I] bf16 out.
 * moe_fc2: y[p, :] = act[p] @ w2[e].T. finalize_mode DETERMINISTIC or NONE writes
 *          the unscaled rows to `dst` = y [T*top_k, H] bf16. FUSED zero-fills
 *          `dst` = out [T, H] bf16 and adds topk_weights[p2e[p]] * y[p] into row
 *          p2e[p] / top_k with bf16 atomics (not bitwise reproducible for top_k > 2).
 *
 * ws / ws_bytes (optional, NULL / 0 allowed): at least
 * moe_gemm_split_workspace_size() bytes, 16-byte aligned, owned by the caller and
 * not shared by calls that may overlap. With it, the tiles of a last, mostly idle
 * round of workgroups are cut along the contraction and their fp32 partials summed
 * in a fixed order (same result on every run; rounding differs from the unsplit
 * order within fp32). Without it no tile is cut. Where the local experts are at least
 * 16 and expect at most 384 rows each (T*top_k / num_experts), the workspace instead
 * serves a work queue: one workgroup per CU takes whole tiles (the bits of the call
 * without a workspace). moe_ffn_forward does this with its own workspace.
 * MOE_ERR_WORKSPACE if ws is given but too small or unaligned.
 */
size_t moe_gemm_split_workspace_size(void);
moe_status moe_fc1(const moe_ffn_desc* desc, const void* x, const void* w1,
                   const float* clamp_limit, const int32_t* offs, const int32_t* p2e, void* act,
                   void* ws, size_t ws_bytes, void* stream);
moe_status moe_fc2(const moe_ffn_desc* desc, const void* act, const void* w2,
                   const int32_t* offs, const int32_t* p2e, const float* topk_weights, void* dst,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * The block-scaled stages ([W4A8] Host plan, Inputs; intro: fp32 accumulation, UE8M0
 * round-up requantization). desc->weight_format must be MOE_WFMT_MXFP4 (W4A8) or
 * MOE_WFMT_MXFP8 (w1 / w2 as e4m3fn code bytes, same scale layout); otherwise
 * MOE_ERR_DTYPE.
 * moe_fc1_mx: act = MXFP8(activation(x[p2e[p]/top_k] @ w1[e].T)) with, per row and
 *             block of 32 columns, the smallest power-of-two scale 2^s such that the
 *             block maximum is <= 448 * 2^s (code s+127) and elements rounded to
 *             nearest even e4m3fn. act [T*top_k, I] e4m3 codes, act_sf [T*top_k, I/32].
 * moe_fc2_mx: y[p, :] = act[p] @ w2[e].T, bf16 rows [T*top_k, H] in permuted order.
 */
moe_status moe_fc1_mx(const moe_ffn_desc* desc, const void* x, const void* x_sf, const void* w1,
                      const void* w1_sf, const float* clamp_limit, const int32_t* offs,
                      const int32_t* p2e, void* act, void* act_sf, void* stream);
moe_status moe_fc2_mx(const moe_ffn_desc* desc, const void* act, const void* act_sf,
                      const void* w2, const void* w2_sf, const int32_t* offs, void* y,
                      void* stream);

/*
 * moe_tune -- per-bucket tile choice for the layer's two GEMM stages ([SM90]
 * Parameters: the autotuner profiles the legal tiles per token bucket and caches the
 * winner; tile_size follows the rows per expert). For the layer described by desc /
 * tensors (any weight_format; x, topk_ids, w1, w2, clamp_limit and, for the
 * fp8-activation formats, x_sf, w1_sf, w2_sf, act_scale are read), it sorts the
 * routes, then times FC1 and FC2 with each tile family -- bf16: the 256-row tile and
 * the 128-row tile (when the stage's contraction is a multiple of 64); MXFP4 / MXFP8 /
 * FP8: the 256-row tile and, where the shape allows it, the 32-row streaming tile --
 * one warm-up and 3 timed launches each, and records the faster family under (stage,
 * weight format, H, I, L, rows per local expert rounded up to a power of two). Later
 * launches of that stage, shape and bucket, by any entry point of this process
 * (moe_ffn_forward and its variants, moe_fc1 / moe_fc2 and the fp8-activation stages),
 * use the recorded family; everything else keeps the built-in rule (bf16: the 128-row
 * tile when T * top_k <= 64 * num_experts, else the 256-row tile; fp8 activations: the
 * streaming tile up to 3 / 12 / 24 rows per local expert for FC1 (MXFP4 / MXFP8 /
 * FP8) and up to 2 for FC2 with 8-bit weights, never for the MXFP4 FC2). choice (optional, [2]) receives the FC1 / FC2 picks: 1 the smaller family
 * (128-row or streaming), 0 the 256-row tile.
 * This call and moe_tune_clear are the exceptions to the conventions above: moe_tune
 * synchronises the stream (it is a tuning step, not a prepared launch) and both act on a
 * per-process table, which the other entry points only read. ws as
 * moe_ffn_workspace_size for the same desc with MOE_FINALIZE_DETERMINISTIC.
 * Thread-safe. moe_tune_clear forgets every recorded choice.
 */
moe_status moe_tune(const moe_ffn_desc* desc, const moe_ffn_tensors* tensors, void* ws,
                    size_t ws_bytes, void* stream, int32_t* choice);
/* moe_tune_set records a choice (0 / 1 as above) for stage 1 (FC1) or 2 (FC2) of the
 * shape and bucket that desc describes, as moe_tune would after timing it: for callers
 * that keep tuned choices across processes, and for tests of each family. */
moe_status moe_tune_set(const moe_ffn_desc* desc, int32_t stage, int32_t choice);
void moe_tune_clear(void);

/*
 * The fp8 per-tensor stages ([StepFun] intro: the per-tensor fp8 weight family);
 * desc->weight_format must be MOE_WFMT_FP8, otherwise MOE_ERR_DTYPE. x, w1, w2, act
 * are e4m3fn code bytes; x_scale [1], w1_scale / w2_scale [L] and act_scale [1] are
 * float32 device values (value = code value * scale). fp32 accumulation.
 * moe_fc1_fp8: act[p, :] = e4m3_rne(clamp(activation(x_scale * w1_scale[e] *
 *              (x[p2e[p]/top_k] @ w1[e].T)) * (1/act_scale), -448, 448)), the
 *              reciprocal taken in float32. act [T*top_k, I] e4m3 codes.
 * moe_fc2_fp8: y[p, :] = bf16(act_scale * w2_scale[e] * (act[p] @ w2[e].T)), rows in
 *              permuted order [T*top_k, H].
 */
moe_status moe_fc1_fp8(const moe_ffn_desc* desc, const void* x, const float* x_scale,
                       const void* w1, const float* w1_scale, const float* act_scale,
                       const float* clamp_limit, const int32_t* offs, const int32_t* p2e,
                       void* act, void* stream);
moe_status moe_fc2_fp8(const moe_ffn_desc* desc, const void* act, const float* act_scale,
                       const void* w2, const float* w2_scale, const int32_t* offs, void* y,
                       void* stream);

/*
 * Training: forward with saved tensors, then the backward ([GGEMM] Autograd
 * section: the backward of a grouped product is its dgrad and wgrad; the rest is
 * the chain rule through the [SM90] formula). bf16 weights and
 * MOE_FINALIZE_DETERMINISTIC only, otherwise MOE_ERR_UNSUPPORTED (size functions
 * return 0).
 *
 * moe_ffn_forward_train: moe_ffn_forward (same tensors; tensors->e2p is ignored)
 *   whose workspace is the caller's `saved` buffer of moe_ffn_saved_size(desc)
 *   bytes, which afterwards holds what the backward reads: the routing metadata,
 *   the FC1 pre-activations h [T*k, 2I] ([up | gate], float32: the values the
 *   forward's activation and clamp saw), act and the unscaled FC2 rows y (bf16),
 *   all in permuted order. Keep it unchanged until the backward.
 * moe_ffn_backward: for the upstream gradient dout = d loss / d out [T, H] bf16,
 *   with the same desc and tensors (x, topk_weights, w1, w2, clamp_limit):
 *     dtopk_weights[t,s] = <dout[t], y[t,s]> (0 for foreign routes; float32),
 *     dy = w[t,s] dout[t];  dw2[e] = sum over e's routes of dy^T act;
 *     dh = act'(h) (dy @ w2[e]) -- SwiGLU: du = da silu(g), dg = da u silu'(g);
 *       SwiGLUStep: the same at the clamped values, zero where |v| > L;
 *     dw1[e] = sum of dh^T x[t];  dx[t] = sum over the token's local routes of
 *     dh @ w1[e] (float32, slots ascending, one rounding; 0 for no local route).
 *   dw1 [L, 2I, H], dw2 [L, H, I] in grad_dtype (fully overwritten; exactly zero
 *   for an expert without routes), dx [T, H] bf16. Intermediates dy, dh are bf16;
 *   every sum runs in a fixed order (bitwise reproducible). ws: at least
 *   moe_ffn_backward_workspace_size(desc) bytes, 16-byte aligned; it holds dy, dh,
 *   the dx rows and 64 MiB of fp32 partial tiles with their arrival counters (the
 *   dgrad's last round of tiles is cut along the contraction), so calls sharing
 *   one ws must not overlap.
 */
typedef struct moe_ffn_grads {
  const void* dout;           /* [T, H] bf16 */
  void* dx;                   /* [T, H] bf16 out */
  void* dw1;                  /* [L, 2I, H] out, grad_dtype */
  void* dw2;                  /* [L, H, I] out, grad_dtype */
  float* dtopk_weights;       /* [T, top_k] float32 out, or NULL */
  int32_t grad_dtype;         /* MOE_DTYPE_BF16 or MOE_DTYPE_F32 */
} moe_ffn_grads;

size_t moe_ffn_saved_size(const moe_ffn_desc* desc);
moe_status moe_ffn_forward_train(const moe_ffn_desc* desc, const moe_ffn_tensors* tensors,
                                 void* saved, size_t saved_bytes, void* stream);
size_t moe_ffn_backward_workspace_size(const moe_ffn_desc* desc);
moe_status moe_ffn_backward(const moe_ffn_desc* desc, const moe_ffn_tensors* tensors,
                            const moe_ffn_grads* grads, const void* saved, size_t saved_bytes,
                            void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_backward -- gradient of the routing logits through the Renormalize
 * weights ([StepFun] intro): w[t,:] = softmax of the k selected logits, so for the
 * expert j selected at slot s, dlogits[t, j] = w[t,s] (dw[t,s] - sum_r w[t,r] dw[t,r])
 * (float32, r ascending); every other logit gets 0 (the selection is piecewise
 * constant). topk_ids / topk_weights as returned by moe_route, dtopk_weights
 * [T, top_k] float32, dlogits [T, num_experts] float32 fully overwritten.
 * Rules as moe_route.
 */
moe_status moe_route_backward(const int32_t* topk_ids, const float* topk_weights,
                              const float* dtopk_weights, int64_t T, int32_t num_experts,
                              int32_t top_k, float* dlogits, void* stream);

/*
 * moe_bgmv -- BGMV MoE-LoRA shrink + expand over routed pairs ([BGMV] signature,
 * Parameters, description). For pair p with token t = sorted_token_ids[p], expert
 * e = expert_ids[p] and LoRA l = lora_indices[t]:
 *   shrink_out[p, :] = bf16_rne(x[t] @ lora_a[l, e].T)                    (rank values)
 *   y_accum[t, :]    = sum over t's pairs in ascending p of
 *                      topk_weights[p] * (shrink_out[p] @ lora_b[l, e].T)   (float32)
 * y_accum rows are fully overwritten (row stride ldy >= feat_out elements; it may be
 * a column slice of a wider buffer); a token without a valid pair gets a zero row.
 * A pair whose token, expert or LoRA index is out of range contributes nothing
 * (its shrink row is zero); indices are not validated otherwise (device data).
 * Shapes: x [T, H] bf16; lora_a [num_loras, E, rank, H] bf16; lora_b
 * [num_loras, E, feat_out, rank] bf16 (one LoRA slice); sorted_token_ids,
 * expert_ids [num_pairs] int32 in any order; lora_indices [T] int32; topk_weights
 * [num_pairs] float32; shrink_out [num_pairs, rank] bf16 or NULL (kept in ws).
 * Rules: rank in {8, 16, 32, 64}; H and feat_out multiples of 8; x, lora_a,
 * lora_b, shrink_out 16-byte aligned. Bitwise reproducible: every output has one
 * owner that sums in a fixed order. ws: moe_bgmv_workspace_size(desc) bytes.
 */
typedef struct moe_bgmv_desc {
  int64_t num_tokens;         /* T */
  int64_t num_pairs;          /* routed (token, expert) pairs */
  int32_t hidden;             /* H */
  int32_t feat_out;           /* LoRA-B output width */
  int32_t rank;
  int32_t num_loras;
  int32_t num_experts;
  int32_t mode;               /* MOE_BGMV_* */
} moe_bgmv_desc;

/* Pipelines of moe_bgmv ([BGMV] Parameters: grouped). The per-pair pipeline reads
 * every pair's LoRA slices; the grouped one groups the pairs by (LoRA, expert) bin
 * (order within a bin does not affect the results), runs the shrink and the expand on
 * MFMA tiles of 32 pairs of one bin
 * (each bin's weights streamed once per tile of pairs), stores w[p] times each pair's
 * fp32 expand row and sums a token's rows in ascending pair order. Both are
 * deterministic; they round differently within float32 (the shrink's and the expand's
 * sums run in other orders). AUTO takes the grouped pipeline when num_pairs >= 48 *
 * num_loras * num_experts; GROUPED needs num_loras * num_experts <= 1024. */
#define MOE_BGMV_AUTO     0
#define MOE_BGMV_PER_PAIR 1
#define MOE_BGMV_GROUPED  2

size_t moe_bgmv_workspace_size(const moe_bgmv_desc* desc);
moe_status moe_bgmv(const moe_bgmv_desc* desc, const void* x, const void* lora_a,
                    const void* lora_b, const int32_t* sorted_token_ids,
                    const int32_t* expert_ids, const int32_t* lora_indices,
                    const float* topk_weights, void* shrink_out, float* y_accum, int64_t ldy,
                    void* ws, size_t ws_bytes, void* stream);

/*
 * moe_finalize -- deterministic top-k combine ([SM90] use_fused_finalize=False):
 *   out[t,:] = bf16_rne( sum over s = 0..top_k-1 with e2p[t*top_k+s] >= 0 of
 *                        topk_weights[t,s] * y[e2p[t*top_k+s], :] )
 * summed in float32 in ascending s, one rounding at the end; tokens with no local
 * route get a zero row. y [*, H] bf16 rows in permuted order; out [T, H] bf16.
 * Rules: H % 8 == 0, 1 <= top_k <= 16.
 */
moe_status moe_finalize(const void* y, const int32_t* e2p, const float* topk_weights, int64_t T,
                        int32_t top_k, int32_t H, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
