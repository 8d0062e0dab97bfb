// Renormalized top-k routing from fp32 logits.
//
// StepFun MoE page, intro: the routing stage is "Renormalize top-k": the k
// largest experts are kept and their softmax weights renormalized to sum to 1.
// Selecting on the raw logits is equivalent (softmax is increasing) and makes the
// chosen ids independent of the exponential's rounding. Ties go to the lower id.
//
// Two kernels:
//  * k_route_thread<EMAX>: one thread per token, the token's logits in registers
//    (num_experts <= EMAX <= 32). Each thread reads one contiguous row.
//  * k_route_wave<Q>: one wave64 per token, lane j holds experts j, j+64, ...
//    (num_experts <= 64*Q); each of the k rounds is a wave arg-max by DPP/shuffle.
#include "common.h"

namespace moe {
namespace {

__device__ __forceinline__ bool better(float v, int id, float bv, int bid) {
  return v > bv || (v == bv && id < bid);
}

__device__ __forceinline__ void write_weights(const float* sel, const int* ids, int k,
                                              int32_t* out_ids, float* out_w) {
  float z[16];
  float sum = 0.f;
  for (int s = 0; s < k; ++s) {
    z[s] = __expf(sel[s] - sel[0]);
    sum += z[s];
  }
  float inv = 1.0f / sum;
  for (int s = 0; s < k; ++s) {
    out_ids[s] = ids[s];
    out_w[s] = z[s] * inv;
  }
}

template <int EMAX>
__global__ __launch_bounds__(256) void k_route_thread(const float* __restrict__ logits, int64_t T,
                                                      int E, int k, int32_t* __restrict__ ids_out,
                                                      float* __restrict__ w_out) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  const float* row = logits + t * E;
  float v[EMAX];
#pragma unroll
  for (int j = 0; j < EMAX; ++j) v[j] = (j < E) ? row[j] : -INFINITY;
  uint32_t taken = 0;
  float sel[16];
  int ids[16];
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < EMAX; ++j) {
      bool ok = (j < E) && !((taken >> j) & 1u);
      if (ok && better(v[j], j, bv, bid)) {
        bv = v[j];
        bid = j;
      }
    }
    taken |= 1u << bid;
    sel[s] = bv;
    ids[s] = bid;
  }
  write_weights(sel, ids, k, ids_out + t * k, w_out + t * k);
}

template <int Q>
__global__ __launch_bounds__(256) void k_route_wave(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids_out,
                                                    float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + t * E;
  float v[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    int j = lane + 64 * q;
    v[q] = (j < E) ? row[j] : -INFINITY;
  }
  uint32_t taken = 0;  // bit q: expert lane+64q already chosen
  float sel[16];
  int ids[16];
  for (int s = 0; s < k; ++s) {
    float bv = -INFINITY;
    int bid = 0x7fffffff;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      int j = lane + 64 * q;
      if (j < E && !((taken >> q) & 1u) && better(v[q], j, bv, bid)) {
        bv = v[q];
        bid = j;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float ov = __shfl_xor(bv, off);
      int oid = __shfl_xor(bid, off);
      if (better(ov, oid, bv, bid)) {
        bv = ov;
        bid = oid;
      }
    }
    // every lane now holds the winner; its owner marks it taken
    if ((bid & 63) == lane) taken |= 1u << (bid >> 6);
    sel[s] = bv;
    ids[s] = bid;
  }
  if (lane == 0) write_weights(sel, ids, k, ids_out + t * k, w_out + t * k);
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" moe_status moe_route(const float* logits, int64_t T, int32_t E, int32_t k,
                                int32_t* topk_ids, float* topk_weights, void* stream) {
  if (T < 0 || E < 1 || E > 1024 || k < 1 || k > 16 || k > E) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!logits || !topk_ids || !topk_weights) return MOE_ERR_NULL;
  hipStream_t st = as_stream(stream);
  if (E <= 32) {
    dim3 grid((unsigned)((T + 255) / 256));
    if (E <= 8)
      k_route_thread<8><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 16)
      k_route_thread<16><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
    else
      k_route_thread<32><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
  } else {
    dim3 grid((unsigned)((T + 3) / 4));  // 4 waves (tokens) per block
    if (E <= 64)
      k_route_wave<1><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 128)
      k_route_wave<2><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
    else if (E <= 256)
      k_route_wave<4><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
    else
      k_route_wave<16><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights);
  }
  return launch_status();
}
