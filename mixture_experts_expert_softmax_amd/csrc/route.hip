// Renormalized top-k routing from fp32 logits.
//
// StepFun MoE page, intro: the routing stage is the Renormalize top-k mode: the k
// largest experts are kept and their softmax weights renormalized to sum to 1.
// Selecting on the raw logits is equivalent (softmax is increasing) and makes the
// chosen ids independent of the exponential's rounding. Ties go to the lower id.
//
// Three kernels:
//  * k_route_thread<EMAX>: one thread per token, the token's logits in registers
//    (num_experts <= EMAX <= 32). Each thread reads one contiguous row.
//  * k_route_rank4<QL, K2, FULL>: four tokens per wave, one per row of 16 lanes
//    (32 < num_experts <= 256); a threshold from disjoint group maxima leaves a
//    short list of candidates, whose ranks give the k slots.
//  * k_route_rank<Q, K2>: the same selection with one wave64 per token, lane l
//    holding experts Q*l .. Q*l+Q-1 (256 < num_experts <= 1024).
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

// Selection key of (logit v, expert id): ord_key(v) (below) in the high word and the
// inverted id in the low word, so that the larger key is the larger logit and, on a
// tie, the lower id. key_value / key_id decode it.
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t o = (uint32_t)(key >> 32);
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int key_id(uint64_t key) { return (int)~(uint32_t)key; }

// Order-preserving unsigned form of a logit: the float's bits with -0 folded onto +0,
// so that a larger logit gives a larger integer (0 is below every logit and stands
// for "no expert").
__device__ __forceinline__ uint32_t ord_key(float v) {
  const uint32_t b = __float_as_uint(v + 0.0f);  // -0 + 0 = +0
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);   // negative: ~b; else b | sign
}

// DPP helpers: the value of another lane of the same row (quad_perm and mirror
// patterns), or the row broadcasts of GFX9 that carry lane 15 / 31 to the next rows
// (rows outside ROW_MASK keep their own value).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_bcast_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, ROW_MASK, 0xF, false);
}
__device__ __forceinline__ uint32_t umax(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin(uint32_t a, uint32_t b) { return a < b ? a : b; }
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_HALF_MIRROR = 0x141, DPP_MIRROR = 0x140,
              DPP_BCAST15 = 0x142, DPP_BCAST31 = 0x143;

// Threshold for a top-k over one wave's keys: the lanes form K2 >= k disjoint groups
// of 64 / K2 lanes; every group's maximum is a distinct key, so at least K2 keys are
// >= the smallest of the group maxima. Returned uniform.
template <int K2>
__device__ __forceinline__ uint32_t topk_threshold(uint32_t m) {
  constexpr int G = 64 / K2;
  if (G >= 2) m = umax(m, dpp_u<DPP_XOR1>(m));
  if (G >= 4) m = umax(m, dpp_u<DPP_XOR2>(m));
  if (G >= 8) m = umax(m, dpp_u<DPP_HALF_MIRROR>(m));
  if (G >= 16) m = umax(m, dpp_u<DPP_MIRROR>(m));
  if (G == 64) {   // one group: the wave maximum, gathered at lane 63
    m = umax(m, dpp_bcast_u<DPP_BCAST15, 0xA>(m));
    m = umax(m, dpp_bcast_u<DPP_BCAST31, 0xC>(m));
    return (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
  }
  if (G == 32) {   // lanes 31 and 63 hold the two half-wave maxima
    m = umax(m, dpp_bcast_u<DPP_BCAST15, 0xA>(m));
    return umin((uint32_t)__builtin_amdgcn_readlane((int)m, 31),
                (uint32_t)__builtin_amdgcn_readlane((int)m, 63));
  }
  // G <= 16: the minimum over the groups of each row, then over the four rows
  if (G <= 4) m = umin(m, dpp_u<DPP_HALF_MIRROR>(m));
  if (G <= 8) m = umin(m, dpp_u<DPP_MIRROR>(m));
  m = umin(m, dpp_bcast_u<DPP_BCAST15, 0xA>(m));
  m = umin(m, dpp_bcast_u<DPP_BCAST31, 0xC>(m));
  return (uint32_t)__builtin_amdgcn_readlane((int)m, 63);
}

// One wave64 per token; lane l holds experts Q*l .. Q*l + Q - 1 (one vector load per
// 4 values when the row is whole). The k winners are found in three steps:
//  1. a threshold t with at least k keys >= t (topk_threshold: the smallest of K2
//     disjoint group maxima, K2 the power of two >= k);
//  2. every key >= t is a candidate; candidates go to this wave's LDS list as 64-bit
//     selection keys (about 2.5 k of them for normally distributed logits);
//  3. each candidate's rank is the number of candidates with a larger selection key,
//     counted by one lane per candidate over the list; rank s < k is slot s.
// The same k winners in the same slots as a sequence of k maxima, for any data
// (ties included: selection keys are unique), with far fewer wave instructions per
// token.
template <int Q>
__device__ __forceinline__ void load_keys(const float* __restrict__ row, int E, int j0,
                                          uint32_t (&key)[Q]) {
  if (E == 64 * Q && (Q == 1 || Q == 2 || Q % 4 == 0)) {
    if (Q == 1) {
      key[0] = ord_key(row[j0]);
    } else if (Q == 2) {
      const float2 p = *reinterpret_cast<const float2*>(row + j0);
      key[0] = ord_key(p.x);
      key[1] = ord_key(p.y);
    } else {
#pragma unroll
      for (int q = 0; q < Q; q += 4) {
        const float4 p = *reinterpret_cast<const float4*>(row + j0 + q);
        key[q] = ord_key(p.x);
        key[q + 1] = ord_key(p.y);
        key[q + 2] = ord_key(p.z);
        key[q + 3] = ord_key(p.w);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) key[q] = j0 + q < E ? ord_key(row[j0 + q]) : 0u;
  }
}

// Each wave takes tokens t = wave, wave + waves, ... (grid-stride), loading the next
// token's logits before it works on the current one. Per token, the k winners are
// found in three steps:
//  1. a threshold t with at least k keys >= t (topk_threshold: the smallest of K2
//     disjoint group maxima, K2 the power of two >= k);
//  2. every key >= t is a candidate; candidates go to this wave's LDS list as 64-bit
//     selection keys (about 2.5 k of them for normally distributed logits);
//  3. each candidate's rank is the number of candidates with a larger selection key,
//     counted by one lane per candidate over the list; rank s < k is slot s.
// The same k winners in the same slots as a sequence of k maxima, for any data
// (ties included: selection keys are unique), with far fewer wave instructions per
// token.
template <int Q, int K2>
__global__ __launch_bounds__(256) void k_route_rank(const float* __restrict__ logits, int64_t T,
                                                    int E, int k, int32_t* __restrict__ ids_out,
                                                    float* __restrict__ w_out) {
  __shared__ uint64_t cand[4][64 * Q];
  __shared__ float sel_v[4][16];
  __shared__ int sel_id[4][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t stride = (int64_t)gridDim.x * 4;
  int64_t t = (int64_t)blockIdx.x * 4 + w;
  if (t >= T) return;  // uniform per wave
  const int j0 = Q * lane;
  uint32_t nxt[Q];
  load_keys<Q>(logits + t * E, E, j0, nxt);
  uint64_t* list = cand[w];
  for (; t < T; t += stride) {
    uint32_t key[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) key[q] = nxt[q];
    if (t + stride < T) load_keys<Q>(logits + (t + stride) * E, E, j0, nxt);
    uint32_t m = key[0];
#pragma unroll
    for (int q = 1; q < Q; ++q) m = umax(m, key[q]);
    const uint32_t thr = topk_threshold<K2>(m);

    int n = 0;   // candidates so far (uniform)
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const bool c = key[q] >= thr && j0 + q < E;
      const unsigned long long mask = __ballot(c);
      if (c) {
        const int pos = n + __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
        list[pos] = ((uint64_t)key[q] << 32) | (uint32_t)~(j0 + q);
      }
      n += __popcll(mask);
    }
    __builtin_amdgcn_wave_barrier();
    for (int b = 0; b < n; b += 64) {   // uniform; one pass unless ties flood the list
      const int i = b + lane;
      const uint64_t mine = i < n ? list[i] : ~0ull;
      int rank = 0;
      int j = 0;
      for (; j + 4 <= n; j += 4) {
        const uint64_t a0 = list[j], a1 = list[j + 1], a2 = list[j + 2], a3 = list[j + 3];
        rank += (a0 > mine) + (a1 > mine) + (a2 > mine) + (a3 > mine);
      }
      for (; j < n; ++j) rank += list[j] > mine;
      if (i < n && rank < k) {
        sel_v[w][rank] = key_value(mine);
        sel_id[w][rank] = key_id(mine);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // weights: softmax of the k selected logits (lanes s < k), summed over row 0
    const float top = sel_v[w][0];
    float z = 0.f;
    int id = 0;
    if (lane < k) {
      id = sel_id[w][lane];
      z = __expf(sel_v[w][lane] - top);
    }
    float sum = z + __int_as_float(dpp_u<DPP_XOR1>(__float_as_uint(z)));
    sum += __int_as_float(dpp_u<DPP_XOR2>(__float_as_uint(sum)));
    sum += __int_as_float(dpp_u<DPP_HALF_MIRROR>(__float_as_uint(sum)));
    sum += __int_as_float(dpp_u<DPP_MIRROR>(__float_as_uint(sum)));
    if (lane < k) {
      ids_out[t * k + lane] = id;
      w_out[t * k + lane] = z * __builtin_amdgcn_rcpf(sum);
    }
    // the next token rewrites this wave's list and slots
    __builtin_amdgcn_wave_barrier();
  }
}

// DPP row shift right by N within each row of 16 lanes; lanes shifted in from outside
// the row read 0 (bound_ctrl), which makes a 4-step inclusive row scan.
template <int N>
__device__ __forceinline__ int dpp_shr(int v) {
  return __builtin_amdgcn_mov_dpp(v, 0x110 + N, 0xF, 0xF, true);
}

// Four tokens per wave, one per row of 16 lanes: lane i of row r holds experts
// QL*i .. QL*i + QL - 1 of token 4 * wave + r (num_experts <= 16 * QL). Same three
// steps as k_route_rank, each row on its own token:
//  1. threshold: the smallest of K2 >= k disjoint group maxima of the row;
//  2. each lane counts its candidates, a row scan gives its first list slot, and the
//     lane writes its candidates' 64-bit selection keys to the row's LDS list (the
//     list is then padded with zero keys up to the longest list of the wave);
//  3. ranks: lane i counts, over the row's list, the keys above candidates i and
//     i + 16 (and further pairs while the list is longer); rank s < k is slot s.
// Per token this issues about half the wave instructions of one token per wave,
// whose fixed costs (threshold, output, loop control) it shares four ways.
template <int QL, int K2, bool FULL>
__global__ __launch_bounds__(256) void k_route_rank4(const float* __restrict__ logits, int64_t T,
                                                     int E, int k, int32_t* __restrict__ ids_out,
                                                     float* __restrict__ w_out) {
  constexpr int CAP = 16 * QL;   // candidates a row can hold (all of its experts)
  // each row's list, then 16 slots where lanes put the keys that are not candidates
  __shared__ uint64_t cand[4][4][CAP + 16];
  __shared__ float sel_v[4][4][16];
  __shared__ int sel_id[4][4][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int r = lane >> 4, li = lane & 15;
  const int64_t stride = (int64_t)gridDim.x * 16;
  int64_t tb = ((int64_t)blockIdx.x * 4 + w) * 4;   // first token of this wave
  if (tb >= T) return;  // uniform per wave
  const int j0 = QL * li;
  uint32_t nxt[QL];
  auto load = [&](int64_t t, uint32_t (&key)[QL]) {
    if (t < T) {
      const float* row = logits + t * E + j0;
      if (FULL) {
#pragma unroll
        for (int q = 0; q < QL; q += 4) {
          const float4 p = *reinterpret_cast<const float4*>(row + q);
          key[q] = ord_key(p.x);
          key[q + 1] = ord_key(p.y);
          key[q + 2] = ord_key(p.z);
          key[q + 3] = ord_key(p.w);
        }
      } else {
#pragma unroll
        for (int q = 0; q < QL; ++q) key[q] = j0 + q < E ? ord_key(row[q]) : 0u;
      }
    } else {
#pragma unroll
      for (int q = 0; q < QL; ++q) key[q] = 0u;
    }
  };
  load(tb + r, nxt);
  uint64_t* list = cand[w][r];
  for (; tb < T; tb += stride) {
    const int64_t t = tb + r;
    const bool active = t < T;
    uint32_t key[QL];
#pragma unroll
    for (int q = 0; q < QL; ++q) key[q] = nxt[q];
    if (tb + stride < T) load(tb + stride + r, nxt);
    // 1. threshold of the row: group maxima over G lanes, then their minimum
    constexpr int G = 16 / K2;
    uint32_t m = key[0];
#pragma unroll
    for (int q = 1; q < QL; ++q) m = umax(m, key[q]);
    if (G >= 2) m = umax(m, dpp_u<DPP_XOR1>(m));
    if (G >= 4) m = umax(m, dpp_u<DPP_XOR2>(m));
    if (G >= 8) m = umax(m, dpp_u<DPP_HALF_MIRROR>(m));
    if (G >= 16) m = umax(m, dpp_u<DPP_MIRROR>(m));
    if (G <= 1) m = umin(m, dpp_u<DPP_XOR1>(m));
    if (G <= 2) m = umin(m, dpp_u<DPP_XOR2>(m));
    if (G <= 4) m = umin(m, dpp_u<DPP_HALF_MIRROR>(m));
    if (G <= 8) m = umin(m, dpp_u<DPP_MIRROR>(m));
    const uint32_t thr = m;
    // 2. candidates: count, row scan, compacted writes
    bool c[QL];
    int cnt = 0;
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      c[q] = active && key[q] >= thr && (FULL || j0 + q < E);
      cnt += c[q];
    }
    int incl = cnt;
    incl += dpp_shr<1>(incl);
    incl += dpp_shr<2>(incl);
    incl += dpp_shr<4>(incl);
    incl += dpp_shr<8>(incl);
    int pos = incl - cnt;
    const int n0 = __builtin_amdgcn_readlane(incl, 15), n1 = __builtin_amdgcn_readlane(incl, 31),
              n2 = __builtin_amdgcn_readlane(incl, 47), n3 = __builtin_amdgcn_readlane(incl, 63);
    const int n = r == 0 ? n0 : r == 1 ? n1 : r == 2 ? n2 : n3;   // this row's list length
    const int nmax = max(max(n0, n1), max(n2, n3));                 // uniform
    // every key is written (no branches): a candidate to the next list slot, any other
    // key to the lane's own slot past the list, which nothing reads
#pragma unroll
    for (int q = 0; q < QL; ++q) {
      list[c[q] ? pos : CAP + li] = ((uint64_t)key[q] << 32) | (uint32_t)~(j0 + q);
      pos += c[q];
    }
    for (int z = n + li; z < nmax; z += 16) list[z] = 0ull;   // below every real key
    __builtin_amdgcn_wave_barrier();
    // 3. ranks, two candidates per lane and pass
    for (int b = 0; b < nmax; b += 32) {   // uniform
      const int ia = b + li, ib = ia + 16;
      const uint64_t ma = ia < n ? list[ia] : ~0ull;
      const uint64_t mb = ib < n ? list[ib] : ~0ull;
      int ra = 0, rb = 0;
      int j = 0;
      for (; j + 8 <= nmax; j += 8) {   // four 16-byte reads in flight per wait
        uint64_t a[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] = list[j + u];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          ra += a[u] > ma;
          rb += a[u] > mb;
        }
      }
      for (; j < nmax; ++j) {
        const uint64_t a0 = list[j];
        ra += a0 > ma;
        rb += a0 > mb;
      }
      if (ia < n && ra < k) {
        sel_v[w][r][ra] = key_value(ma);
        sel_id[w][r][ra] = key_id(ma);
      }
      if (ib < n && rb < k) {
        sel_v[w][r][rb] = key_value(mb);
        sel_id[w][r][rb] = key_id(mb);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // weights: softmax of the row's k selected logits (lanes li < k), summed over the row
    float z = 0.f;
    int id = 0;
    if (active && li < k) {
      id = sel_id[w][r][li];
      z = __expf(sel_v[w][r][li] - sel_v[w][r][0]);
    }
    float sum = z + __int_as_float(dpp_u<DPP_XOR1>(__float_as_uint(z)));
    sum += __int_as_float(dpp_u<DPP_XOR2>(__float_as_uint(sum)));
    sum += __int_as_float(dpp_u<DPP_HALF_MIRROR>(__float_as_uint(sum)));
    sum += __int_as_float(dpp_u<DPP_MIRROR>(__float_as_uint(sum)));
    if (active && li < k) {
      ids_out[t * k + li] = id;
      w_out[t * k + li] = z * __builtin_amdgcn_rcpf(sum);
    }
    // the next tokens rewrite this wave's lists and slots
    __builtin_amdgcn_wave_barrier();
  }
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
    // 4 waves (tokens) per block; waves loop over tokens beyond 8 blocks per CU
    const int64_t blocks = (T + 3) / 4, cap = (int64_t)device_cu_count() * 8;
    dim3 grid((unsigned)(blocks < cap ? blocks : cap));
    const int K2 = k <= 1 ? 1 : k <= 2 ? 2 : k <= 4 ? 4 : k <= 8 ? 8 : 16;
#define MOE_ROUTE_Q(Q_)                                                                       \
  switch (K2) {                                                                               \
    case 1: k_route_rank<Q_, 1><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights); break; \
    case 2: k_route_rank<Q_, 2><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights); break; \
    case 4: k_route_rank<Q_, 4><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights); break; \
    case 8: k_route_rank<Q_, 8><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights); break; \
    default: k_route_rank<Q_, 16><<<grid, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights); break; \
  }
    if (E <= 256) {
      // four tokens per wave: 16 tokens per block
      const int64_t b4 = (T + 15) / 16;
      dim3 grid4((unsigned)(b4 < cap ? b4 : cap));
      const int QL = E <= 64 ? 4 : E <= 128 ? 8 : 16;
      const bool full = E == 16 * QL;
#define MOE_ROUTE4(QL_, K2_)                                                                   \
  (full ? k_route_rank4<QL_, K2_, true><<<grid4, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights) \
        : k_route_rank4<QL_, K2_, false><<<grid4, 256, 0, st>>>(logits, T, E, k, topk_ids, topk_weights))
#define MOE_ROUTE4_K(QL_)                      \
  switch (K2) {                                \
    case 1: MOE_ROUTE4(QL_, 1); break;         \
    case 2: MOE_ROUTE4(QL_, 2); break;         \
    case 4: MOE_ROUTE4(QL_, 4); break;         \
    case 8: MOE_ROUTE4(QL_, 8); break;         \
    default: MOE_ROUTE4(QL_, 16); break;       \
  }
      if (QL == 4) {
        MOE_ROUTE4_K(4)
      } else if (QL == 8) {
        MOE_ROUTE4_K(8)
      } else {
        MOE_ROUTE4_K(16)
      }
#undef MOE_ROUTE4_K
#undef MOE_ROUTE4
    } else if (E <= 512) {
      MOE_ROUTE_Q(8)
    } else {
      MOE_ROUTE_Q(16)
    }
#undef MOE_ROUTE_Q
  }
  return launch_status();
}
