// Backward of the layer's non-GEMM steps.
//
// Grouped-GEMM page ("Cake ragged BF16 grouped GEMM (experimental)"), Autograd
// section: the products' backward is their dgrad and wgrad (gemm_bf16.hip). What
// remains is the chain rule through the forward formula of the SM90 fused-MoE page,
// out[t] = sum_s w[t,s] y[e2p[t,s]]:
//   permute backward  dy[p] = w[t,s] dout[t] for the permuted row p = e2p[t*k+s],
//                     and the routing-weight gradient dw[t,s] = <dout[t], y[p]>;
//   routing backward  through the Renormalize weights (StepFun page, intro: a
//                     softmax over the k selected logits).
// Both are HBM- or latency-bound elementwise work; sums run in a fixed order.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// One workgroup per token, slots in order. Each thread takes 8-column chunks
// c = tid, tid + 256, ...; the dot product is summed per thread in that order, then
// across the wave by a butterfly and across the 4 waves in wave order.
__global__ __launch_bounds__(256) void k_permute_bwd(const uint4* __restrict__ dout,
                                                     const int32_t* __restrict__ e2p,
                                                     const float* __restrict__ w,
                                                     const uint4* __restrict__ y, int k, int H8,
                                                     uint4* __restrict__ dy, float* __restrict__ dw) {
  __shared__ float part[4];
  const int64_t t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int s = 0; s < k; ++s) {
    const int64_t r = t * k + s;
    const int p = e2p[r];   // the same for the whole workgroup
    if (p < 0) {            // a foreign route: no row, no gradient
      if (dw && tid == 0) dw[r] = 0.f;
      continue;
    }
    const float wt = w[r];
    float dot = 0.f;
    for (int c = tid; c < H8; c += 256) {
      const uint4 d = dout[t * H8 + c];
      const uint4 yv = y[(int64_t)p * H8 + c];
      const uint32_t dv[4] = {d.x, d.y, d.z, d.w};
      const uint32_t vv[4] = {yv.x, yv.y, yv.z, yv.w};
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float d0 = bf16_lo(dv[q]), d1 = bf16_hi(dv[q]);
        o[q] = pack_bf16x2(wt * d0, wt * d1);
        dot = fmaf(d0, bf16_lo(vv[q]), dot);
        dot = fmaf(d1, bf16_hi(vv[q]), dot);
      }
      dy[(int64_t)p * H8 + c] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    if (dw) {
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m);
      if (lane == 0) part[wid] = dot;
      __syncthreads();
      if (tid == 0) dw[r] = ((part[0] + part[1]) + part[2]) + part[3];
      __syncthreads();
    }
  }
}

// Gather of token rows into permuted order for the FC1 weight gradient: dst[p] =
// src[p2e[p] / k] for p below the local route count ends[L - 1] (one 16-byte chunk
// per thread, consecutive threads on consecutive chunks).
__global__ __launch_bounds__(256) void k_gather_rows(const uint4* __restrict__ src,
                                                     const int32_t* __restrict__ p2e,
                                                     const int32_t* __restrict__ ends, int L, int k,
                                                     int H8, int64_t cap, uint4* __restrict__ dst) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = ends[L - 1];
  const int64_t rows = n < cap ? n : cap;
  if (idx >= rows * H8) return;
  const int64_t p = idx / H8;
  const int c = (int)(idx - p * H8);
  dst[idx] = src[(int64_t)(p2e[p] / k) * H8 + c];
}

// dlogits[t, j] = sum over slots s with ids[t,s] == j of w[t,s] (dw[t,s] - sum_r w[t,r] dw[t,r]);
// every element of [T, E] is written (0 for unselected experts).
__global__ __launch_bounds__(256) void k_route_bwd(const int32_t* __restrict__ ids,
                                                   const float* __restrict__ w,
                                                   const float* __restrict__ dw, int64_t T, int E,
                                                   int k, float* __restrict__ dl) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= T * E) return;
  const int64_t t = idx / E;
  const int j = (int)(idx - t * E);
  float inner = 0.f;
  for (int r = 0; r < k; ++r) inner = fmaf(w[t * k + r], dw[t * k + r], inner);
  float g = 0.f;
  for (int s = 0; s < k; ++s)
    if (ids[t * k + s] == j) g += w[t * k + s] * (dw[t * k + s] - inner);
  dl[idx] = g;
}

}  // namespace

moe_status gather_rows_enqueue(const void* src, const int32_t* p2e, const int32_t* ends, int L,
                               int k, int H, int64_t R, void* dst, hipStream_t st) {
  if (R == 0) return MOE_OK;
  const int64_t blocks = (R * (H / 8) + 255) / 256;   // bound: all R rows local
  if (blocks > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  k_gather_rows<<<(unsigned)blocks, 256, 0, st>>>(reinterpret_cast<const uint4*>(src), p2e, ends, L,
                                                  k, H / 8, R, reinterpret_cast<uint4*>(dst));
  return launch_status();
}

moe_status permute_bwd_enqueue(const void* dout, const int32_t* e2p, const float* w, const void* y,
                               int64_t T, int k, int H, void* dy, float* dw, hipStream_t st) {
  if (T == 0) return MOE_OK;
  if (T > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  k_permute_bwd<<<(unsigned)T, 256, 0, st>>>(reinterpret_cast<const uint4*>(dout), e2p, w,
                                             reinterpret_cast<const uint4*>(y), k, H / 8,
                                             reinterpret_cast<uint4*>(dy), dw);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route_backward(const int32_t* topk_ids, const float* topk_weights,
                                         const float* dtopk_weights, int64_t T, int32_t num_experts,
                                         int32_t top_k, float* dlogits, void* stream) {
  if (T < 0 || num_experts < 1 || num_experts > 1024 || top_k < 1 || top_k > 16 ||
      top_k > num_experts)
    return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!topk_ids || !topk_weights || !dtopk_weights || !dlogits) return MOE_ERR_NULL;
  const int64_t n = T * num_experts;
  const int64_t blocks = (n + 255) / 256;
  if (blocks > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  k_route_bwd<<<(unsigned)blocks, 256, 0, as_stream(stream)>>>(topk_ids, topk_weights, dtopk_weights,
                                                                T, num_experts, top_k, dlogits);
  return launch_status();
}
