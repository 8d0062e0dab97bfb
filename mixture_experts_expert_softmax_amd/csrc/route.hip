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
//  * k_route_wave<Q>: one wave64 per token, lane l holds experts Q*l .. Q*l+Q-1
//    (num_experts <= 64*Q) as keys sorted in the lane; each of the k rounds is a
//    DPP wave maximum over the lanes' head values.
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

// Selection key of (logit v, expert id): the float's bits made order-preserving as
// an unsigned integer (with -0 folded onto +0), then the inverted id, so that the
// larger key is the larger logit and, on a tie, the lower id. Key 0 is below every
// real key and stands for "no expert".
__device__ __forceinline__ uint64_t route_key(float v, int id) {
  const uint32_t b = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
  const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)o << 32) | (uint32_t)~id;
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

// Wave maximum of a 32-bit unsigned value, returned to every lane (uniform):
// rotations by 1, 2, 4, 8 inside each row of 16 lanes, then the GFX9 row
// broadcasts 15 and 31 carry the row maxima up to lane 63, which is read back.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = ROW_MASK == 0xF
                         ? (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true)
                         : (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = dpp_umax<0x121, 0xF>(v);  // row_ror:1
  v = dpp_umax<0x122, 0xF>(v);  // row_ror:2
  v = dpp_umax<0x124, 0xF>(v);  // row_ror:4
  v = dpp_umax<0x128, 0xF>(v);  // row_ror:8
  v = dpp_umax<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_umax<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wave64 per token; lane l holds experts Q*l .. Q*l + Q - 1 (one vector load
// when the row is whole) as selection keys, sorted in the lane once. Each of the
// k rounds takes the wave maximum of the lanes' head keys by their high (value)
// word; among the lanes whose head has that value the lowest one holds the lowest
// id, its head is the winner, and that lane alone advances to its next key.
template <int Q>
__global__ __launch_bounds__(256) void k_route_wave(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids_out,
                                                    float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;  // uniform per wave
  const float* row = logits + t * E;
  float v[Q];
  const int j0 = Q * lane;
  if (E == 64 * Q && (Q == 1 || Q == 2 || Q % 4 == 0)) {
    if (Q == 1) {
      v[0] = row[j0];
    } else if (Q == 2) {
      const float2 p = *reinterpret_cast<const float2*>(row + j0);
      v[0] = p.x;
      v[1] = p.y;
    } else {
#pragma unroll
      for (int q = 0; q < Q; q += 4) {
        const float4 p = *reinterpret_cast<const float4*>(row + j0 + q);
        v[q] = p.x;
        v[q + 1] = p.y;
        v[q + 2] = p.z;
        v[q + 3] = p.w;
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) v[q] = j0 + q < E ? row[j0 + q] : 0.f;
  }
  uint64_t key[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) key[q] = j0 + q < E ? route_key(v[q], j0 + q) : 0ull;
  // descending in-lane sort (odd-even transposition; Q is small)
#pragma unroll
  for (int r = 0; r < Q; ++r)
#pragma unroll
    for (int q = r & 1; q + 1 < Q; q += 2) {
      const uint64_t a = key[q], b = key[q + 1];
      key[q] = a > b ? a : b;
      key[q + 1] = a > b ? b : a;
    }
  float sel[16];
  int ids[16];
  for (int s = 0; s < k; ++s) {
    const uint32_t head = (uint32_t)(key[0] >> 32);
    const uint32_t m = wave_umax(head);
    const unsigned long long hit = __ballot(head == m);
    const int L = __ffsll(hit) - 1;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)key[0], L);
    const uint64_t win = ((uint64_t)m << 32) | lo;
    if (lane == L) {
#pragma unroll
      for (int q = 0; q + 1 < Q; ++q) key[q] = key[q + 1];
      key[Q - 1] = 0ull;
    }
    sel[s] = key_value(win);
    ids[s] = key_id(win);
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
