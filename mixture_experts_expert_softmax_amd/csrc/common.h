// Shared device and host helpers of the gfx950 MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

// ------------------------------------------------------------------ host side
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline moe_status launch_status() {
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Number of compute units of the current device (cached per device id).
int device_cu_count();

// Split-K tiles of the bf16 grouped kernels: at most SPLIT_SLOTS fp32 partial
// 256 x 256 tiles in flight, plus one arrival counter per remainder tile.
constexpr int SPLIT_SLOTS = 256;
constexpr size_t SPLIT_TILE_BYTES = 256 * 256 * 4;

// ------------------------------------------------------------------ device side
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// register staging type for 16-byte copies: a vector, not an aggregate, so that a
// load kept in registers and stored later is not merged into one memory-to-memory copy
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// float -> bf16 bits, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// silu(z) = z / (1 + e^-z), with the hardware base-2 exponential and reciprocal.
__device__ __forceinline__ float silu_f32(float z) {
  float e = __builtin_amdgcn_exp2f(-z * 1.4426950408889634f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// Tile dealing shared by the grouped kernels. Group g < E owns rows
// [end(g - 1), end(g)) of a row-sorted operand, the ends made non-decreasing and
// capped at m_cap (a running maximum, starting from 0). A group's rows split into
// ceil(rows / TM) row blocks times n_tiles column tiles; tiles are numbered
// group-major, then column tile, row block fastest, and block b takes tile
// (b % 8) * per + b / 8 with per = ceil(total / 8), so each of the 8 XCDs works
// through one contiguous share (and its L2 sees few experts). Each wave does the
// bookkeeping with lane-parallel scans over 64 groups at a time: a handful of
// vector loads instead of a chain of dependent scalar loads.
__device__ __forceinline__ int wave_scan_max(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v = v > u ? v : u;
  }
  return v;
}
__device__ __forceinline__ int wave_scan_add(int v, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  return v;
}

// One pass of the scan over 64 groups from c0: this lane's group's clamped end,
// previous end and inclusive tile count; carries the last end (ce) and count (tc).
template <int TM>
__device__ __forceinline__ void tile_scan_pass(const int32_t* __restrict__ ends, int E, int m_cap,
                                               int n_tiles, int c0, int lane, int& ce, int& tc,
                                               int& cend, int& pend, int& incl) {
  const int g = c0 + lane;
  const int v = wave_scan_max(g < E ? ends[g] : 0, lane);
  cend = v > ce ? v : ce;
  cend = cend < m_cap ? cend : m_cap;
  pend = __shfl_up(cend, 1, 64);
  if (lane == 0) pend = ce;
  const int tl = g < E ? (cend - pend + TM - 1) / TM * n_tiles : 0;
  incl = wave_scan_add(tl, lane) + tc;
  ce = __builtin_amdgcn_readlane(cend, 63);
  tc = __builtin_amdgcn_readlane(incl, 63);
}

template <int TM>
__device__ __forceinline__ int tile_count(const int32_t* __restrict__ ends, int E, int m_cap,
                                          int n_tiles) {
  const int lane = threadIdx.x & 63;
  int ce = 0, tc = 0, cend, pend, incl;
  for (int c0 = 0; c0 < E; c0 += 64)
    tile_scan_pass<TM>(ends, E, m_cap, n_tiles, c0, lane, ce, tc, cend, pend, incl);
  return tc;
}

// (group, first row, group end, column tile) of tile t < tile_count
template <int TM>
__device__ __forceinline__ void tile_locate(const int32_t* __restrict__ ends, int E, int m_cap,
                                            int n_tiles, int t, int& e, int& m0, int& mend,
                                            int& nt) {
  const int lane = threadIdx.x & 63;
  int ce = 0, tc = 0, cend, pend, incl;
  for (int c0 = 0; c0 < E; c0 += 64) {
    tile_scan_pass<TM>(ends, E, m_cap, n_tiles, c0, lane, ce, tc, cend, pend, incl);
    if (t < tc) {
      const unsigned long long hit = __ballot(incl > t);
      const int L = __ffsll(hit) - 1;
      const int ge = __builtin_amdgcn_readlane(cend, L);
      const int gs = __builtin_amdgcn_readlane(pend, L);
      const int te = (ge - gs + TM - 1) / TM;
      const int r = t - (__builtin_amdgcn_readlane(incl, L) - te * n_tiles);
      nt = r / te;
      e = c0 + L;
      m0 = gs + (r - nt * te) * TM;
      mend = ge;
      return;
    }
  }
}

// Source rows of gathered activation rows: v holds permuted rows p on entry and
// g[p] / div on return when g is given (all loads issued before any is used, so
// a tile's prologue waits once for them, not once per row).
template <int N>
__device__ __forceinline__ void gather_rows(const int32_t* __restrict__ g, int div, int (&v)[N]) {
  if (g) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = g[v[j]];
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] /= div;
  }
}

// Up to 64 groups: one scan pass serves both the count and the lookup (one load of
// the ends per tile instead of two), kept in the lane registers.
struct TileScan64 {
  int cend, pend, incl, total;
};
template <int TM>
__device__ __forceinline__ TileScan64 tile_scan64(const int32_t* __restrict__ ends, int E, int m_cap,
                                                  int n_tiles) {
  const int lane = threadIdx.x & 63;
  int ce = 0, tc = 0;
  TileScan64 s;
  tile_scan_pass<TM>(ends, E, m_cap, n_tiles, 0, lane, ce, tc, s.cend, s.pend, s.incl);
  s.total = tc;
  return s;
}
// tile_locate from a scan taken with n_scanned column tiles, for n_used column tiles
// (every group's tile count is a multiple of n_scanned, so the division is exact)
template <int TM>
__device__ __forceinline__ void tile_locate64(const TileScan64& s, int n_scanned, int n_used, int t,
                                              int& e, int& m0, int& mend, int& nt) {
  const int inc = s.incl / n_scanned * n_used;
  const unsigned long long hit = __ballot(inc > t);
  const int L = __ffsll(hit) - 1;
  const int ge = __builtin_amdgcn_readlane(s.cend, L);
  const int gs = __builtin_amdgcn_readlane(s.pend, L);
  const int te = (ge - gs + TM - 1) / TM;
  const int r = t - (__builtin_amdgcn_readlane(inc, L) - te * n_used);
  nt = r / te;
  e = L;
  m0 = gs + (r - nt * te) * TM;
  mend = ge;
}

template <int TM>
__device__ __forceinline__ bool deal_tile(const int32_t* __restrict__ ends, int E, int m_cap,
                                          int n_tiles, int& e, int& m0, int& mend, int& nt) {
  if (E <= 64) {
    const TileScan64 s = tile_scan64<TM>(ends, E, m_cap, n_tiles);
    const int per = (s.total + 7) >> 3;
    const int slot = (int)(blockIdx.x >> 3);
    const int t = (int)(blockIdx.x & 7) * per + slot;
    if (slot >= per || t >= s.total) return false;
    tile_locate64<TM>(s, n_tiles, n_tiles, t, e, m0, mend, nt);
    return true;
  }
  const int total = tile_count<TM>(ends, E, m_cap, n_tiles);
  const int per = (total + 7) >> 3;
  const int slot = (int)(blockIdx.x >> 3);
  const int t = (int)(blockIdx.x & 7) * per + slot;
  if (slot >= per || t >= total) return false;
  tile_locate<TM>(ends, E, m_cap, n_tiles, t, e, m0, mend, nt);
  return true;
}

}  // namespace moe
