// C-ABI entry points that chain the kernels: the grouped GEMMs and the MoE
// expert-layer forward. Argument rules and layouts are documented in moe.h.
#include <algorithm>
#include <mutex>

#include "common.h"

namespace moe {
// defined in sort.hip / finalize.hip / gemm_bf16.hip
size_t sort_workspace_bytes(int64_t T, int32_t k, int32_t L);
moe_status sort_enqueue(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t L,
                        int32_t off, int32_t* offs, int32_t* m_indptr, int32_t* e2p,
                        int32_t* p2e, int32_t* n_local, void* ws, hipStream_t st,
                        int32_t* zero = nullptr, int n_zero = 0);
moe_status finalize_enqueue(const void* y, const int32_t* e2p, const float* w, int64_t T, int k,
                            int H, void* out, hipStream_t st);
moe_status gemm_nt_enqueue(int epi, const void* A, const int32_t* a_gather, int a_div,
                           const void* B, int NB, int E, const int32_t* ends, int64_t M, int N,
                           int K, void* C, int64_t ldc, int I, const float* limits,
                           float def_limit, const float* route_w, const int32_t* p2e, int top_k,
                           hipStream_t st, void* split_ws = nullptr,
                           int32_t* split_cnt = nullptr, void* h_out = nullptr, int tm = 256,
                           int rows_hint = 0);
moe_status gemm_dgrad_enqueue(const void* G, const void* W, const int32_t* ends, int E, int64_t M,
                              int N, int K, void* DX, hipStream_t st, int act = 0,
                              const void* h = nullptr, const float* limits = nullptr,
                              float def_limit = 7.0f, void* split_ws = nullptr,
                              int32_t* split_cnt = nullptr);
moe_status gemm_wgrad_enqueue(const void* G, const void* X, const int32_t* ends, int E, int64_t M,
                              int N, int K, void* DW, bool out_f32, hipStream_t st);
// defined in backward.hip
moe_status gather_rows_enqueue(const void* src, const int32_t* p2e, const int32_t* ends, int L,
                               int k, int H, int64_t R, void* dst, hipStream_t st);
moe_status permute_bwd_enqueue(const void* dout, const int32_t* e2p, const float* w, const void* y,
                               int64_t T, int k, int H, void* dy, float* dw, hipStream_t st);
moe_status zero_fill(void* p, size_t bytes, hipStream_t st);
// defined in gemm_mx.hip
moe_status mx_fc1_enqueue(int activation, int wf, const void* x, const void* x_sf,
                          const int32_t* p2e, int top_k, const void* w1, const void* w1_sf, int L,
                          const int32_t* offs, int64_t R, int H, int I, const float* limits,
                          void* act, void* act_sf, const float* act_scale, hipStream_t st,
                          int force = -1, int32_t* qcnt = nullptr, int rows_hint = 0);
moe_status mx_fc2_enqueue(int wf, const void* act, const void* act_sf, const void* w2,
                          const void* w2_sf, int L, const int32_t* offs, int64_t R, int H, int I,
                          void* y, hipStream_t st, int force = -1, int32_t* qcnt = nullptr,
                          int rows_hint = 0);
bool mx_small_possible(int stage, int wf, int H, int I, int64_t R);
// defined in tune.hip
void tune_store(int stage, int wf, int K, int NB, int L, int64_t R, int choice);
int tune_lookup(int stage, int wf, int K, int NB, int L, int64_t R);

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

namespace {
// the fp8-activation weight formats (MXFP4, MXFP8: block scales; FP8: per-tensor
// scales), all served by the scaled-MFMA kernels, and their index there
inline bool is_mx(int32_t wfmt) {
  return wfmt == MOE_WFMT_MXFP4 || wfmt == MOE_WFMT_MXFP8 || wfmt == MOE_WFMT_FP8;
}
inline bool block_scaled(int32_t wfmt) { return wfmt == MOE_WFMT_MXFP4 || wfmt == MOE_WFMT_MXFP8; }
inline int mx_wf(int32_t wfmt) { return wfmt - MOE_WFMT_MXFP4; }

constexpr int EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_STEP = 2, EPI_FUSED = 3;
constexpr int64_t U32_ELEMS = (int64_t)1 << 32;

// Resolve an offsets argument to a pointer at E cumulative ends.
inline const int32_t* ends_of(const int32_t* offs, int32_t kind) {
  return kind == MOE_OFFS_INDPTR ? offs + 1 : offs;
}

moe_status check_gemm(const void* p0, const void* p1, const int32_t* offs, int32_t kind, int32_t E,
                      int64_t M, int32_t N, int32_t K, const void* out) {
  if (kind != MOE_OFFS_ENDS && kind != MOE_OFFS_INDPTR) return MOE_ERR_DTYPE;
  if (E < 1 || M < 0 || N < 32 || K < 32 || N % 32 || K % 32) return MOE_ERR_SHAPE;
  if (M > INT32_MAX || M * (int64_t)std::max(N, K) >= U32_ELEMS) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)N * K >= U32_ELEMS) return MOE_ERR_UNSUPPORTED;
  if (!offs || !p1) return MOE_ERR_NULL;
  if (M > 0 && (!p0 || !out)) return MOE_ERR_NULL;  // row operands may be empty
  if (!aligned16(p0) || !aligned16(p1) || !aligned16(out)) return MOE_ERR_ALIGN;
  return MOE_OK;
}

struct FfnLayout {
  size_t sort_ws, offs, e2p, p2e, n_local, act, act_sf, y, split, split_cnt, h, total;
};

// The forward's workspace; with `train`, followed by the FC1 pre-activations h
// [T*k, 2I] float32 that the backward needs (the training forward's saved buffer):
// fp32, the values the forward's activation saw, so that the backward's SwiGLUStep
// clamp masks agree with the forward's clamp.
FfnLayout ffn_layout(const moe_ffn_desc* d, bool train = false) {
  FfnLayout l{};
  const int64_t T = d->T;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int64_t R = T * d->top_k;
  size_t o = 0;
  l.sort_ws = o; o += align_up(sort_workspace_bytes(T, d->top_k, L), 256);
  l.offs = o;    o += align_up((size_t)L * 4, 256);
  l.e2p = o;     o += align_up((size_t)R * 4, 256);
  l.p2e = o;     o += align_up((size_t)R * 4, 256);
  l.n_local = o; o += 256;
  const bool mx = is_mx(d->weight_format);
  l.act = o;     o += align_up((size_t)R * d->I * (mx ? 1 : 2), 256);
  l.act_sf = o;  o += block_scaled(d->weight_format) ? align_up((size_t)R * (d->I / 32), 256) : 0;
  l.y = o;
  if (d->finalize_mode == MOE_FINALIZE_DETERMINISTIC) o += align_up((size_t)R * d->H * 2, 256);
  // bf16 FC1 / FC2 may cut their last round's tiles along K (fp32 partial tiles)
  l.split = o;
  if (!mx) o += (size_t)SPLIT_SLOTS * SPLIT_TILE_BYTES;
  // bf16: the split tiles' arrival counters; every format: the work-queue counters
  l.split_cnt = o;
  o += align_up((size_t)SPLIT_SLOTS * 4, 256);
  l.h = o;
  if (train) o += align_up((size_t)R * 2 * d->I * 4, 256);
  l.total = o;
  return l;
}

// Backward workspace: dy [T*k, H] (later the gathered x rows), dh [T*k, 2I], dx rows
// [T*k, H] (bf16, permuted order).
struct BwdLayout {
  size_t dy, dh, dxp, split, split_cnt, total;
};

BwdLayout bwd_layout(const moe_ffn_desc* d) {
  BwdLayout l{};
  const int64_t R = d->T * d->top_k;
  size_t o = 0;
  l.dy = o;  o += align_up((size_t)R * d->H * 2, 256);
  l.dh = o;  o += align_up((size_t)R * 2 * d->I * 2, 256);
  l.dxp = o; o += align_up((size_t)R * d->H * 2, 256);
  // fp32 partial tiles and arrival counters of the dgrad tiles cut along N
  l.split = o; o += (size_t)SPLIT_SLOTS * SPLIT_TILE_BYTES;
  l.split_cnt = o; o += align_up((size_t)SPLIT_SLOTS * 4, 256);
  l.total = o;
  return l;
}
}  // namespace
}  // namespace moe

using namespace moe;

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_NULL: return "MOE_ERR_NULL: a required pointer is NULL";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: a size is out of range or breaks a divisibility rule";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: unknown or unsupported dtype / mode";
    case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: request outside the served configurations";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
    case MOE_ERR_TOO_LARGE:
      return "MOE_ERR_TOO_LARGE: the request needs more than the no-allocation scratch memory";
    default: return "unknown moe_status";
  }
}

extern "C" const char* moe_version(void) { return "moe-mi355x 0.1 (gfx950)"; }

constexpr size_t SPLIT_CNT_OFF = (size_t)SPLIT_SLOTS * SPLIT_TILE_BYTES;
constexpr size_t SPLIT_WS_BYTES = SPLIT_CNT_OFF + (size_t)SPLIT_SLOTS * 4;

extern "C" size_t moe_gemm_split_workspace_size(void) { return SPLIT_WS_BYTES; }

static moe_status split_args(void* ws, size_t ws_bytes, hipStream_t st, void*& split_ws,
                             int32_t*& split_cnt) {
  split_ws = nullptr;
  split_cnt = nullptr;
  if (!ws) return MOE_OK;
  if (ws_bytes < SPLIT_WS_BYTES || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  split_ws = ws;
  split_cnt = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + SPLIT_CNT_OFF);
  return zero_fill(split_cnt, (size_t)SPLIT_SLOTS * 4, st);
}

extern "C" moe_status grouped_gemm_fwd(const void* x, const void* w, const int32_t* offs,
                                       int32_t kind, int32_t E, int64_t M, int32_t N, int32_t K,
                                       void* y, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_gemm(x, w, offs, kind, E, M, N, K, y);
  if (s != MOE_OK) return s;
  if (M == 0) return MOE_OK;
  void* split_ws;
  int32_t* split_cnt;
  s = split_args(ws, ws_bytes, as_stream(stream), split_ws, split_cnt);
  if (s != MOE_OK) return s;
  return gemm_nt_enqueue(EPI_STORE, x, nullptr, 1, w, N, E, ends_of(offs, kind), M, N, K, y, N, 0,
                         nullptr, 0.f, nullptr, nullptr, 1, as_stream(stream), split_ws,
                         split_cnt, nullptr, 256, (int)(M / E));
}

extern "C" moe_status grouped_gemm_dgrad(const void* g, const void* w, const int32_t* offs,
                                         int32_t kind, int32_t E, int64_t M, int32_t N, int32_t K,
                                         void* dx, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_gemm(g, w, offs, kind, E, M, N, K, dx);
  if (s != MOE_OK) return s;
  if (M == 0) return MOE_OK;
  void* split_ws;
  int32_t* split_cnt;
  s = split_args(ws, ws_bytes, as_stream(stream), split_ws, split_cnt);
  if (s != MOE_OK) return s;
  return gemm_dgrad_enqueue(g, w, ends_of(offs, kind), E, M, N, K, dx, as_stream(stream), 0,
                            nullptr, nullptr, 7.0f, split_ws, split_cnt);
}

extern "C" size_t grouped_gemm_wgrad_workspace_size(int32_t, int64_t, int32_t, int32_t, int32_t) {
  return 0;  // the fixed-order wgrad needs no scratch memory
}

extern "C" moe_status grouped_gemm_wgrad(const void* g, const void* x, const int32_t* offs,
                                         int32_t kind, int32_t E, int64_t M, int32_t N, int32_t K,
                                         void* dw, int32_t out_dtype, void*, size_t, void* stream) {
  if (out_dtype != MOE_DTYPE_BF16 && out_dtype != MOE_DTYPE_F32) return MOE_ERR_DTYPE;
  if (M == 0) {  // only dW has to be written: zeros ([GGEMM] empty groups give zero gradients)
    if (kind != MOE_OFFS_ENDS && kind != MOE_OFFS_INDPTR) return MOE_ERR_DTYPE;
    if (E < 1 || N < 32 || K < 32 || N % 32 || K % 32) return MOE_ERR_SHAPE;
    if (!dw) return MOE_ERR_NULL;
    if (!aligned16(dw)) return MOE_ERR_ALIGN;
    const size_t bytes = (size_t)E * N * K * (out_dtype == MOE_DTYPE_F32 ? 4 : 2);
    return zero_fill(dw, bytes, as_stream(stream));
  }
  moe_status s = check_gemm(g, x, offs, kind, E, M, N, K, dw);
  if (s != MOE_OK) return s;
  return gemm_wgrad_enqueue(g, x, ends_of(offs, kind), E, M, N, K, dw,
                            out_dtype == MOE_DTYPE_F32, as_stream(stream));
}

static moe_status check_ffn(const moe_ffn_desc* d) {
  if (!d) return MOE_ERR_NULL;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  if (d->T < 0 || d->H < 64 || d->H % 64 || d->I < 32 || d->I % 32) return MOE_ERR_SHAPE;
  if (d->num_experts < 1 || d->num_experts > 1024 || d->num_local_experts < 0) return MOE_ERR_SHAPE;
  if (d->local_expert_offset < 0 || d->local_expert_offset + L > d->num_experts) return MOE_ERR_SHAPE;
  if (d->top_k < 1 || d->top_k > 16 || d->top_k > d->num_experts) return MOE_ERR_SHAPE;
  if (d->activation != MOE_ACT_SWIGLU && d->activation != MOE_ACT_SWIGLU_STEP) return MOE_ERR_DTYPE;
  if (d->finalize_mode < MOE_FINALIZE_DETERMINISTIC || d->finalize_mode > MOE_FINALIZE_NONE)
    return MOE_ERR_DTYPE;
  if (d->weight_format != MOE_WFMT_BF16 && !is_mx(d->weight_format)) return MOE_ERR_DTYPE;
  if (is_mx(d->weight_format)) {
    if (d->H % 128 || d->I % 128) return MOE_ERR_SHAPE;
    if (d->finalize_mode == MOE_FINALIZE_FUSED) return MOE_ERR_UNSUPPORTED;
  }
  const int64_t R = d->T * d->top_k;
  if (R > INT32_MAX || R * std::max(d->H, 2 * d->I) >= U32_ELEMS || d->T * d->H >= U32_ELEMS)
    return MOE_ERR_UNSUPPORTED;
  if ((int64_t)2 * d->I * d->H >= U32_ELEMS) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Tile family of the bf16 FC1 (stage 1) and FC2 (stage 2): activation rows per tile,
// 256 or 128. force 0 / 1 picks 256 / 128; otherwise a choice recorded by moe_tune for
// this stage, shape and bucket, else the built-in rule: 128-row tiles when the routes
// spread evenly would give each expert at most 64 rows (measured at H = 4096 / 7168:
// 2-4% faster there, 6-13% slower at 256 and 1024 rows per expert).
constexpr int TUNE_BF16 = -1;   // weight-format key of the bf16 stages in the tune table
static int bf16_tile_rows(const moe_ffn_desc* d, int stage, int K, int NB, int L, int64_t R,
                          int force) {
  if (force < 0) force = tune_lookup(stage, TUNE_BF16, K, NB, L, R);
  if (force < 0) force = R <= (int64_t)64 * d->num_experts ? 1 : 0;
  return force == 1 ? 128 : 256;
}

// Rows a local expert holds on average, as far as the host can tell without reading
// the routing: the routes spread over all experts (a shard's share is its experts').
static int expected_rows(const moe_ffn_desc* d) {
  return (int)(d->T * d->top_k / (d->num_experts > 0 ? d->num_experts : 1));
}

// FC1 over gathered token rows; the activation runs in the GEMM epilogue.
static moe_status fc1_enqueue(const moe_ffn_desc* d, const void* x, const void* w1,
                              const float* limits, const int32_t* offs, const int32_t* p2e,
                              void* act, hipStream_t st, void* split_ws = nullptr,
                              int32_t* split_cnt = nullptr, void* h_out = nullptr,
                              int force = -1) {
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int64_t R = d->T * d->top_k;
  const int epi = d->activation == MOE_ACT_SWIGLU_STEP ? EPI_SWIGLU_STEP : EPI_SWIGLU;
  return gemm_nt_enqueue(epi, x, p2e, d->top_k, w1, 2 * d->I, L, offs, R, d->I, d->H, act, d->I,
                         d->I, limits, 7.0f, nullptr, nullptr, d->top_k, st, split_ws, split_cnt,
                         h_out, bf16_tile_rows(d, 1, d->H, 2 * d->I, L, R, force),
                         expected_rows(d));
}

// FC2: unscaled rows in permuted order, or the fused scaled scatter-add into out.
static moe_status fc2_enqueue(const moe_ffn_desc* d, const void* act, const void* w2,
                              const int32_t* offs, const int32_t* p2e, const float* topk_weights,
                              void* dst, hipStream_t st, void* split_ws = nullptr,
                              int32_t* split_cnt = nullptr, int force = -1) {
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int64_t R = d->T * d->top_k;
  const int tm = bf16_tile_rows(d, 2, d->I, d->H, L, R, force);
  if (d->finalize_mode == MOE_FINALIZE_FUSED) {
    moe_status s = zero_fill(dst, (size_t)d->T * d->H * 2, st);
    if (s != MOE_OK) return s;
    return gemm_nt_enqueue(EPI_FUSED, act, nullptr, 1, w2, d->H, L, offs, R, d->H, d->I, dst, d->H,
                           0, nullptr, 0.f, topk_weights, p2e, d->top_k, st, split_ws, split_cnt,
                           nullptr, tm, expected_rows(d));
  }
  return gemm_nt_enqueue(EPI_STORE, act, nullptr, 1, w2, d->H, L, offs, R, d->H, d->I, dst, d->H, 0,
                         nullptr, 0.f, nullptr, nullptr, d->top_k, st, split_ws, split_cnt, nullptr,
                         tm, expected_rows(d));
}

extern "C" size_t moe_ffn_workspace_size(const moe_ffn_desc* d) {
  if (check_ffn(d) != MOE_OK) return 0;
  return ffn_layout(d).total;
}

static moe_status ffn_forward(const moe_ffn_desc* d, const moe_ffn_tensors* t, void* ws,
                              size_t ws_bytes, void* stream, bool train) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (!t) return MOE_ERR_NULL;
  if (train && (d->weight_format != MOE_WFMT_BF16 || d->finalize_mode != MOE_FINALIZE_DETERMINISTIC))
    return MOE_ERR_UNSUPPORTED;
  if (d->T == 0) return MOE_OK;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int fm = d->finalize_mode;
  const bool mx = is_mx(d->weight_format);
  if (!t->x || !t->topk_ids || !t->topk_weights || !t->w1 || !t->w2) return MOE_ERR_NULL;
  if (mx && (!t->x_sf || !t->w1_sf || !t->w2_sf)) return MOE_ERR_NULL;
  if (d->weight_format == MOE_WFMT_FP8 && !t->act_scale) return MOE_ERR_NULL;
  if (fm != MOE_FINALIZE_NONE && !t->out) return MOE_ERR_NULL;
  if (fm == MOE_FINALIZE_NONE && (!t->y || !t->e2p)) return MOE_ERR_NULL;
  if (!aligned16(t->x) || !aligned16(t->w1) || !aligned16(t->w2) ||
      (t->out && !aligned16(t->out)) || (t->y && !aligned16(t->y)))
    return MOE_ERR_ALIGN;
  if (mx && block_scaled(d->weight_format) &&
      (!aligned16(t->x_sf) || !aligned16(t->w1_sf) || !aligned16(t->w2_sf)))
    return MOE_ERR_ALIGN;
  const FfnLayout l = ffn_layout(d, train);
  if (!ws || ws_bytes < l.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  char* w = reinterpret_cast<char*>(ws);
  int32_t* offs = reinterpret_cast<int32_t*>(w + l.offs);
  // training keeps e2p in the saved buffer for the backward
  int32_t* e2p = t->e2p && !train ? t->e2p : reinterpret_cast<int32_t*>(w + l.e2p);
  int32_t* p2e = reinterpret_cast<int32_t*>(w + l.p2e);
  int32_t* nloc = reinterpret_cast<int32_t*>(w + l.n_local);
  void* act = w + l.act;
  void* y = fm == MOE_FINALIZE_NONE ? t->y : w + l.y;
  const int H = d->H;

  int32_t* split_cnt = reinterpret_cast<int32_t*>(w + l.split_cnt);
  void* split_ws = mx ? nullptr : w + l.split;
  // the sort also clears the split-tile arrival / work-queue counters
  s = sort_enqueue(t->topk_ids, d->T, d->top_k, d->num_experts, L, d->local_expert_offset, offs,
                   nullptr, e2p, p2e, nloc, w + l.sort_ws, st, split_cnt, SPLIT_SLOTS);
  if (s != MOE_OK) return s;
  if (mx) {
    const int64_t R = d->T * d->top_k;
    const int wf = mx_wf(d->weight_format);
    // FP8: act carries the caller's per-tensor scale instead of block scales
    const void* act_sf = block_scaled(d->weight_format) ? (const void*)(w + l.act_sf)
                                                        : (const void*)t->act_scale;
    s = mx_fc1_enqueue(d->activation, wf, t->x, t->x_sf, p2e, d->top_k, t->w1, t->w1_sf, L, offs,
                       R, H, d->I, t->clamp_limit, act, w + l.act_sf, t->act_scale, st, -1,
                       split_cnt, expected_rows(d));
    if (s != MOE_OK) return s;
    s = mx_fc2_enqueue(wf, act, act_sf, t->w2, t->w2_sf, L, offs, R, H, d->I, y, st, -1,
                       split_cnt, expected_rows(d));
  } else {
    s = fc1_enqueue(d, t->x, t->w1, t->clamp_limit, offs, p2e, act, st, split_ws, split_cnt,
                    train ? w + l.h : nullptr);
    if (s != MOE_OK) return s;
    s = fc2_enqueue(d, act, t->w2, offs, p2e, t->topk_weights, fm == MOE_FINALIZE_FUSED ? t->out : y,
                    st, split_ws, split_cnt);
  }
  if (s != MOE_OK || fm != MOE_FINALIZE_DETERMINISTIC) return s;
  return finalize_enqueue(y, e2p, t->topk_weights, d->T, d->top_k, H, t->out, st);
}

extern "C" moe_status moe_ffn_forward(const moe_ffn_desc* d, const moe_ffn_tensors* t, void* ws,
                                      size_t ws_bytes, void* stream) {
  return ffn_forward(d, t, ws, ws_bytes, stream, false);
}

static bool trainable(const moe_ffn_desc* d) {
  return d->weight_format == MOE_WFMT_BF16 && d->finalize_mode == MOE_FINALIZE_DETERMINISTIC;
}

extern "C" size_t moe_ffn_saved_size(const moe_ffn_desc* d) {
  if (check_ffn(d) != MOE_OK || !trainable(d)) return 0;
  return ffn_layout(d, true).total;
}

extern "C" moe_status moe_ffn_forward_train(const moe_ffn_desc* d, const moe_ffn_tensors* t,
                                            void* saved, size_t saved_bytes, void* stream) {
  return ffn_forward(d, t, saved, saved_bytes, stream, true);
}

extern "C" size_t moe_ffn_backward_workspace_size(const moe_ffn_desc* d) {
  if (check_ffn(d) != MOE_OK || !trainable(d)) return 0;
  return bwd_layout(d).total;
}

extern "C" moe_status moe_ffn_backward(const moe_ffn_desc* d, const moe_ffn_tensors* t,
                                       const moe_ffn_grads* g, const void* saved,
                                       size_t saved_bytes, void* ws, size_t ws_bytes,
                                       void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (!trainable(d)) return MOE_ERR_UNSUPPORTED;
  if (!t || !g) return MOE_ERR_NULL;
  if (g->grad_dtype != MOE_DTYPE_BF16 && g->grad_dtype != MOE_DTYPE_F32) return MOE_ERR_DTYPE;
  if (!g->dw1 || !g->dw2 || !t->w1 || !t->w2) return MOE_ERR_NULL;
  if (!aligned16(g->dw1) || !aligned16(g->dw2) || !aligned16(t->w1) || !aligned16(t->w2))
    return MOE_ERR_ALIGN;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const bool f32 = g->grad_dtype == MOE_DTYPE_F32;
  hipStream_t st = as_stream(stream);
  const int H = d->H, I = d->I, k = d->top_k;
  if (d->T == 0) {  // no rows: the weight gradients are exactly zero
    const size_t es = f32 ? 4 : 2;
    s = zero_fill(g->dw1, (size_t)L * 2 * I * H * es, st);
    if (s != MOE_OK) return s;
    return zero_fill(g->dw2, (size_t)L * H * I * es, st);
  }
  if (!g->dout || !g->dx || !t->x || !t->topk_weights) return MOE_ERR_NULL;
  if (!aligned16(g->dout) || !aligned16(g->dx) || !aligned16(t->x)) return MOE_ERR_ALIGN;
  const FfnLayout l = ffn_layout(d, true);
  if (!saved || saved_bytes < l.total || !aligned16(saved)) return MOE_ERR_WORKSPACE;
  const BwdLayout b = bwd_layout(d);
  if (!ws || ws_bytes < b.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  const char* sv = reinterpret_cast<const char*>(saved);
  const int32_t* offs = reinterpret_cast<const int32_t*>(sv + l.offs);
  const int32_t* e2p = reinterpret_cast<const int32_t*>(sv + l.e2p);
  const int32_t* p2e = reinterpret_cast<const int32_t*>(sv + l.p2e);
  const void* h = sv + l.h;
  const void* act = sv + l.act;
  const void* y = sv + l.y;
  char* w = reinterpret_cast<char*>(ws);
  void* dy = w + b.dy;
  void* dh = w + b.dh;
  void* dxp = w + b.dxp;
  void* split_ws = w + b.split;
  int32_t* split_cnt = reinterpret_cast<int32_t*>(w + b.split_cnt);
  const int64_t R = d->T * k;
  // the counters start at zero; the last part of each split tile resets its own
  s = zero_fill(split_cnt, (size_t)SPLIT_SLOTS * 4, st);
  if (s != MOE_OK) return s;
  // out[t] = sum_s w y  ->  dy rows and the routing-weight gradients
  s = permute_bwd_enqueue(g->dout, e2p, t->topk_weights, y, d->T, k, H, dy, g->dtopk_weights, st);
  if (s != MOE_OK) return s;
  // y = act @ w2^T  ->  da = dy @ w2 (with dh = act'(h) da in the epilogue), dw2 = dy^T act
  const int actk = d->activation == MOE_ACT_SWIGLU_STEP ? 2 : 1;
  s = gemm_dgrad_enqueue(dy, t->w2, offs, L, R, H, I, dh, st, actk, h, t->clamp_limit, 7.0f,
                         split_ws, split_cnt);
  if (s != MOE_OK) return s;
  s = gemm_wgrad_enqueue(dy, act, offs, L, R, H, I, g->dw2, f32, st);
  if (s != MOE_OK) return s;
  // h = x[p2e / k] @ w1^T  ->  dx rows = dh @ w1, dw1 = dh^T x[p2e / k]; the x rows are
  // gathered once into permuted order (into dy's buffer, free after dw2)
  s = gemm_dgrad_enqueue(dh, t->w1, offs, L, R, 2 * I, H, dxp, st, 0, nullptr, nullptr, 7.0f,
                         split_ws, split_cnt);
  if (s != MOE_OK) return s;
  s = gather_rows_enqueue(t->x, p2e, offs, L, k, H, R, dy, st);
  if (s != MOE_OK) return s;
  s = gemm_wgrad_enqueue(dh, dy, offs, L, R, 2 * I, H, g->dw1, f32, st);
  if (s != MOE_OK) return s;
  // the un-permute: dx[t] = sum over the token's local routes of its dx rows
  return finalize_enqueue(dxp, e2p, nullptr, d->T, k, H, g->dx, st);
}

extern "C" moe_status moe_fc1_mx(const moe_ffn_desc* d, const void* x, const void* x_sf,
                                 const void* w1, const void* w1_sf, const float* clamp_limit,
                                 const int32_t* offs, const int32_t* p2e, void* act, void* act_sf,
                                 void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (!block_scaled(d->weight_format)) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!x || !x_sf || !w1 || !w1_sf || !offs || !p2e || !act || !act_sf) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(act) || !aligned16(x_sf) || !aligned16(w1_sf) ||
      !aligned16(act_sf))
    return MOE_ERR_ALIGN;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  return mx_fc1_enqueue(d->activation, mx_wf(d->weight_format), x, x_sf, p2e, d->top_k, w1, w1_sf,
                        L, offs, d->T * d->top_k, d->H, d->I, clamp_limit, act, act_sf, nullptr,
                        as_stream(stream));
}

extern "C" moe_status moe_fc2_mx(const moe_ffn_desc* d, const void* act, const void* act_sf,
                                 const void* w2, const void* w2_sf, const int32_t* offs, void* y,
                                 void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (!block_scaled(d->weight_format)) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!act || !act_sf || !w2 || !w2_sf || !offs || !y) return MOE_ERR_NULL;
  if (!aligned16(act) || !aligned16(w2) || !aligned16(y) || !aligned16(w2_sf)) return MOE_ERR_ALIGN;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  return mx_fc2_enqueue(mx_wf(d->weight_format), act, act_sf, w2, w2_sf, L, offs, d->T * d->top_k, d->H, d->I, y,
                        as_stream(stream));
}

// Times a stage launch: one warm-up, then the mean of `reps` event-timed launches.
static moe_status time_launches(hipStream_t st, int reps, float* ms,
                                moe_status (*launch)(void*), void* ctx) {
  hipEvent_t a, b;
  if (hipEventCreate(&a) != hipSuccess) return MOE_ERR_HIP;
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return MOE_ERR_HIP;
  }
  moe_status s = launch(ctx);
  if (s == MOE_OK && hipEventRecord(a, st) != hipSuccess) s = MOE_ERR_HIP;
  for (int r = 0; s == MOE_OK && r < reps; ++r) s = launch(ctx);
  if (s == MOE_OK && hipEventRecord(b, st) != hipSuccess) s = MOE_ERR_HIP;
  if (s == MOE_OK && hipEventSynchronize(b) != hipSuccess) s = MOE_ERR_HIP;
  if (s == MOE_OK && hipEventElapsedTime(ms, a, b) != hipSuccess) s = MOE_ERR_HIP;
  if (s == MOE_OK) *ms /= reps;
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  return s;
}

struct TuneCtx {
  const moe_ffn_desc* d;
  const moe_ffn_tensors* t;
  const int32_t* offs;
  const int32_t* p2e;
  void* act;
  void* act_sf;
  const void* act_sf_in;
  void* y;
  hipStream_t st;
  int force;
  void* split_ws;        // bf16 stages: the layer's split-tile workspace
  int32_t* split_cnt;
};

static moe_status tune_fc1(void* p) {
  const TuneCtx& c = *reinterpret_cast<TuneCtx*>(p);
  const int32_t L = c.d->num_local_experts > 0 ? c.d->num_local_experts : c.d->num_experts;
  if (c.d->weight_format == MOE_WFMT_BF16)
    return fc1_enqueue(c.d, c.t->x, c.t->w1, c.t->clamp_limit, c.offs, c.p2e, c.act, c.st,
                       c.split_ws, c.split_cnt, nullptr, c.force);
  return mx_fc1_enqueue(c.d->activation, mx_wf(c.d->weight_format), c.t->x, c.t->x_sf, c.p2e,
                        c.d->top_k, c.t->w1, c.t->w1_sf, L, c.offs, c.d->T * c.d->top_k, c.d->H,
                        c.d->I, c.t->clamp_limit, c.act, c.act_sf, c.t->act_scale, c.st, c.force,
                        c.split_cnt, expected_rows(c.d));
}

static moe_status tune_fc2(void* p) {
  const TuneCtx& c = *reinterpret_cast<TuneCtx*>(p);
  const int32_t L = c.d->num_local_experts > 0 ? c.d->num_local_experts : c.d->num_experts;
  if (c.d->weight_format == MOE_WFMT_BF16)
    return fc2_enqueue(c.d, c.act, c.t->w2, c.offs, nullptr, nullptr, c.y, c.st, c.split_ws,
                       c.split_cnt, c.force);
  return mx_fc2_enqueue(mx_wf(c.d->weight_format), c.act, c.act_sf_in, c.t->w2, c.t->w2_sf, L,
                        c.offs, c.d->T * c.d->top_k, c.d->H, c.d->I, c.y, c.st, c.force,
                        c.split_cnt, expected_rows(c.d));
}

extern "C" moe_status moe_tune_set(const moe_ffn_desc* d, int32_t stage, int32_t choice) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if ((stage != 1 && stage != 2) || (choice != 0 && choice != 1)) return MOE_ERR_SHAPE;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int64_t R = d->T * d->top_k;
  const int wf = is_mx(d->weight_format) ? mx_wf(d->weight_format) : TUNE_BF16;
  if (stage == 1)
    tune_store(1, wf, d->H, 2 * d->I, L, R, choice);
  else
    tune_store(2, wf, d->I, d->H, L, R, choice);
  return MOE_OK;
}

extern "C" moe_status moe_tune(const moe_ffn_desc* d, const moe_ffn_tensors* t, void* ws,
                               size_t ws_bytes, void* stream, int32_t* choice) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  const bool mx = is_mx(d->weight_format);
  if (!t) return MOE_ERR_NULL;
  if (d->T == 0) return MOE_OK;
  if (!t->x || !t->topk_ids || !t->w1 || !t->w2) return MOE_ERR_NULL;
  if (mx && (!t->x_sf || !t->w1_sf || !t->w2_sf)) return MOE_ERR_NULL;
  if (d->weight_format == MOE_WFMT_FP8 && !t->act_scale) return MOE_ERR_NULL;
  if (!aligned16(t->x) || !aligned16(t->w1) || !aligned16(t->w2)) return MOE_ERR_ALIGN;
  // the layer's workspace, with room for the FC2 rows (DETERMINISTIC layout)
  moe_ffn_desc dd = *d;
  dd.finalize_mode = MOE_FINALIZE_DETERMINISTIC;
  const FfnLayout l = ffn_layout(&dd);
  if (!ws || ws_bytes < l.total || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  hipStream_t st = as_stream(stream);
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  const int64_t R = d->T * d->top_k;
  const int wf = mx ? mx_wf(d->weight_format) : TUNE_BF16;
  char* w = reinterpret_cast<char*>(ws);
  int32_t* offs = reinterpret_cast<int32_t*>(w + l.offs);
  int32_t* p2e = reinterpret_cast<int32_t*>(w + l.p2e);
  int32_t* split_cnt = reinterpret_cast<int32_t*>(w + l.split_cnt);
  s = sort_enqueue(t->topk_ids, d->T, d->top_k, d->num_experts, L, d->local_expert_offset, offs,
                   nullptr, reinterpret_cast<int32_t*>(w + l.e2p), p2e,
                   reinterpret_cast<int32_t*>(w + l.n_local), w + l.sort_ws, st, split_cnt,
                   SPLIT_SLOTS);
  if (s != MOE_OK) return s;
  TuneCtx c{&dd, t, offs, p2e, w + l.act, w + l.act_sf,
            block_scaled(d->weight_format) ? (const void*)(w + l.act_sf) : (const void*)t->act_scale,
            w + l.y, st, 0, mx ? nullptr : w + l.split, split_cnt};
  for (int stage = 1; stage <= 2; ++stage) {
    int best = 0;
    // the candidates: the 256-row tile and the streaming tile (fp8 activations) or the
    // 128-row tile (bf16), where the shape allows it
    if (mx ? mx_small_possible(stage, wf, d->H, d->I, R)
           : (stage == 1 ? d->H : d->I) % 64 == 0) {
      float ms[2];
      for (int f = 0; f < 2; ++f) {
        c.force = f;
        s = time_launches(st, 3, &ms[f], stage == 1 ? tune_fc1 : tune_fc2, &c);
        if (s != MOE_OK) return s;
      }
      best = ms[1] < ms[0] ? 1 : 0;
    }
    if (stage == 1)
      tune_store(1, wf, d->H, 2 * d->I, L, R, best);
    else
      tune_store(2, wf, d->I, d->H, L, R, best);
    if (choice) choice[stage - 1] = best;
    // FC2's inputs: act from FC1 with the recorded choice
    if (stage == 1) {
      c.force = best;
      s = tune_fc1(&c);
      if (s != MOE_OK) return s;
    }
  }
  return hipStreamSynchronize(st) == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

extern "C" moe_status moe_fc1_fp8(const moe_ffn_desc* d, const void* x, const float* x_scale,
                                  const void* w1, const float* w1_scale, const float* act_scale,
                                  const float* clamp_limit, const int32_t* offs, const int32_t* p2e,
                                  void* act, void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (d->weight_format != MOE_WFMT_FP8) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!x || !x_scale || !w1 || !w1_scale || !act_scale || !offs || !p2e || !act) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(act)) return MOE_ERR_ALIGN;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  return mx_fc1_enqueue(d->activation, mx_wf(MOE_WFMT_FP8), x, x_scale, p2e, d->top_k, w1, w1_scale,
                        L, offs, d->T * d->top_k, d->H, d->I, clamp_limit, act, nullptr, act_scale,
                        as_stream(stream));
}

extern "C" moe_status moe_fc2_fp8(const moe_ffn_desc* d, const void* act, const float* act_scale,
                                  const void* w2, const float* w2_scale, const int32_t* offs,
                                  void* y, void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (d->weight_format != MOE_WFMT_FP8) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!act || !act_scale || !w2 || !w2_scale || !offs || !y) return MOE_ERR_NULL;
  if (!aligned16(act) || !aligned16(w2) || !aligned16(y)) return MOE_ERR_ALIGN;
  const int32_t L = d->num_local_experts > 0 ? d->num_local_experts : d->num_experts;
  return mx_fc2_enqueue(mx_wf(MOE_WFMT_FP8), act, act_scale, w2, w2_scale, L, offs, d->T * d->top_k,
                        d->H, d->I, y, as_stream(stream));
}

// Split-tile workspace of the standalone GEMM stages: partial tiles, then the
// arrival counters, which each call clears first.
extern "C" moe_status moe_fc1(const moe_ffn_desc* d, const void* x, const void* w1,
                              const float* clamp_limit, const int32_t* offs, const int32_t* p2e,
                              void* act, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (d->weight_format != MOE_WFMT_BF16) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!x || !w1 || !offs || !p2e || !act) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(w1) || !aligned16(act)) return MOE_ERR_ALIGN;
  void* split_ws;
  int32_t* split_cnt;
  s = split_args(ws, ws_bytes, as_stream(stream), split_ws, split_cnt);
  if (s != MOE_OK) return s;
  return fc1_enqueue(d, x, w1, clamp_limit, offs, p2e, act, as_stream(stream), split_ws, split_cnt);
}

extern "C" moe_status moe_fc2(const moe_ffn_desc* d, const void* act, const void* w2,
                              const int32_t* offs, const int32_t* p2e, const float* topk_weights,
                              void* dst, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  if (d->weight_format != MOE_WFMT_BF16) return MOE_ERR_DTYPE;
  if (d->T == 0) return MOE_OK;
  if (!act || !w2 || !offs || !dst) return MOE_ERR_NULL;
  if (d->finalize_mode == MOE_FINALIZE_FUSED && (!p2e || !topk_weights)) return MOE_ERR_NULL;
  if (!aligned16(act) || !aligned16(w2) || !aligned16(dst)) return MOE_ERR_ALIGN;
  void* split_ws;
  int32_t* split_cnt;
  s = split_args(ws, ws_bytes, as_stream(stream), split_ws, split_cnt);
  if (s != MOE_OK) return s;
  return fc2_enqueue(d, act, w2, offs, p2e, topk_weights, dst, as_stream(stream), split_ws,
                     split_cnt);
}

// ---------------------------------------------------------------------------
// moe_ffn_forward_noalloc: moe_ffn_forward with its workspace in a file-scope device
// array (one copy per device, held until the process ends) instead of a caller buffer.
// Host code never passes the array's name to a kernel: its address on the current
// device is looked up once per device and kept below, and only that address is used.
// ---------------------------------------------------------------------------
__device__ __align__(256) char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES] = {};

// Address of this device's copy of `scratch`, resolved on the first call per device.
moe_status scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= MAX_DEVICES) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_ffn_forward_noalloc(const moe_ffn_desc* d, const moe_ffn_tensors* t,
                                              void* stream) {
  moe_status s = check_ffn(d);
  if (s != MOE_OK) return s;
  // the same workspace layout as moe_ffn_forward, so both run identical launches
  if (ffn_layout(d).total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  void* ws = nullptr;
  s = scratch_of_current_device(&ws);
  if (s != MOE_OK) return s;
  return ffn_forward(d, t, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream, false);
}
