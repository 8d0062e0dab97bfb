// Stable, unpadded counting sort of routes by local expert ("moe_sort").
//
// Grouped-GEMM page, intro: groups are consecutive row ranges described by
// cumulative end offsets (or m_indptr with a leading zero); no padding.
// StepFun page, "Prepared launches": expanded_idx_to_permuted_idx maps the
// expanded index i = t*top_k + s to its row in the expert-sorted order.
// SM90 fused-MoE page, Parameters: the EP shard holds num_local_experts experts
// from global id local_expert_offset; other routes contribute nothing.
//
// Up to 16384 routes (and per-wave histograms that fit in 64 KB of LDS): one
// workgroup does it all (k_sort_block); one launch wins while the routes are few.
// Beyond that, three launches over chunks of CHUNK routes (one 256-thread
// workgroup per chunk, wave w owning the chunk's w-th quarter):
//  1. k_sort_count:   per-chunk histogram of local experts -> cnt[chunk][e]
//                     (one coalesced row per chunk)
//  2. k_sort_scan:    per expert, the exclusive prefix of cnt[*][e] over the
//                     chunks (in place) and the expert total; 16 experts per
//                     workgroup, each column split over 64 slices of chunks
//  3. k_sort_scatter: an exclusive scan of the totals -> expert start rows; each
//                     wave counts its quarter, then walks its routes in order, 64
//                     at a time, ranking equal keys with ballots (stable), and
//                     writes e2p / p2e.
// The result is a pure function of the ids: no atomics decide any position.
#include "common.h"

namespace moe {
namespace {

constexpr int SORT_STEPS = 16;
constexpr int SORT_WAVES = 4;
constexpr int CHUNK = 64 * SORT_STEPS * SORT_WAVES;  // routes per 256-thread chunk

__device__ __forceinline__ int local_key(int32_t id, int E, int L, int off) {
  int loc = id - off;
  bool ok = (id >= 0) && (id < E) && (loc >= 0) && (loc < L);
  return ok ? loc : L;  // L = foreign
}

__global__ __launch_bounds__(256) void k_sort_count(const int32_t* __restrict__ ids, int64_t n,
                                                    int E, int L, int off,
                                                    int32_t* __restrict__ cnt) {
  extern __shared__ int32_t hist[];
  const int tid = threadIdx.x;
  for (int e = tid; e < L; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t base = (int64_t)blockIdx.x * CHUNK;
  int key[SORT_STEPS];  // all of the thread's ids are requested before any is used
#pragma unroll
  for (int step = 0; step < SORT_STEPS; ++step) {
    const int64_t i = base + step * 256 + tid;
    key[step] = i < n ? local_key(ids[i], E, L, off) : L;
  }
#pragma unroll
  for (int step = 0; step < SORT_STEPS; ++step)
    if (key[step] < L) atomicAdd(&hist[key[step]], 1);
  __syncthreads();
  int32_t* row = cnt + (int64_t)blockIdx.x * L;
  for (int e = tid; e < L; e += 256) row[e] = hist[e];
}

// Inclusive wave64 scan of an int.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(v, d);
    if (lane >= d) v += o;
  }
  return v;
}

// Column prefixes of cnt [nb][L]: workgroup b owns experts SCAN_E b .. SCAN_E b +
// SCAN_E - 1; thread (slice s, expert lane) sums chunks [s * per, (s + 1) * per) of its
// column, the slice sums are combined through LDS, and a second pass writes the
// exclusive prefix. Few experts per workgroup and many slices keep the dependent
// loads per thread short (the kernel is latency-bound).
constexpr int SCAN_E = 16;
constexpr int SCAN_SLICES = 1024 / SCAN_E;
__global__ __launch_bounds__(1024) void k_sort_scan(int32_t* __restrict__ cnt, int nb, int L,
                                                    int32_t* __restrict__ total,
                                                    int32_t* __restrict__ zero, int n_zero) {
  __shared__ int ssum[SCAN_SLICES][SCAN_E];
  const int tid = threadIdx.x, el = tid % SCAN_E, sl = tid / SCAN_E;
  if (blockIdx.x == 0)  // a buffer the caller wants cleared before the GEMMs (no extra launch)
    for (int i = tid; i < n_zero; i += 1024) zero[i] = 0;
  const int e = blockIdx.x * SCAN_E + el;
  const int per = (nb + SCAN_SLICES - 1) / SCAN_SLICES;
  const int c0 = sl * per, c1 = min(nb, c0 + per);
  int part = 0;
  if (e < L)
    for (int c = c0; c < c1; ++c) part += cnt[(int64_t)c * L + e];
  ssum[sl][el] = part;
  __syncthreads();
  int run = 0;
  for (int s2 = 0; s2 < sl; ++s2) run += ssum[s2][el];
  if (e < L) {
    for (int c = c0; c < c1; ++c) {
      int32_t* p = cnt + (int64_t)c * L + e;
      const int v = *p;
      *p = run;
      run += v;
    }
    if (sl == SCAN_SLICES - 1) total[e] = run;
  }
}

// Up to SB_MAX routes: the whole sort in one workgroup of 16 waves (one launch;
// for decode-sized inputs the three launches below cost more than the work).
// Wave w owns the contiguous routes [w * seg, (w + 1) * seg): its per-expert
// counts go to cnt[w][e]; a pass over the experts turns them into each wave's
// first row per expert (expert start + the counts of earlier waves); then every
// wave walks its routes in order, 64 at a time, ranking equal keys with ballots.
constexpr int SB_WAVES = 16;
constexpr int SB_MAX = 16384;

__global__ __launch_bounds__(1024) void k_sort_block(
    const int32_t* __restrict__ ids, int n, int E, int L, int off, int32_t* __restrict__ offs,
    int32_t* __restrict__ m_indptr, int32_t* __restrict__ n_local, int32_t* __restrict__ e2p,
    int32_t* __restrict__ p2e, int32_t* __restrict__ zero, int n_zero) {
  extern __shared__ int32_t sm[];
  int32_t* cnt = sm;                  // [SB_WAVES][L]
  int32_t* start = sm + SB_WAVES * L; // [L]
  int32_t* wsum = start + L;          // [SB_WAVES]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int i = tid; i < n_zero; i += 1024) zero[i] = 0;
  for (int i = tid; i < SB_WAVES * L; i += 1024) cnt[i] = 0;
  __syncthreads();
  const int seg = ((n + SB_WAVES - 1) / SB_WAVES + 63) / 64 * 64;
  const int b0 = w * seg, b1 = min(n, b0 + seg);
  for (int i = b0 + lane; i < b1; i += 64) {
    const int key = local_key(ids[i], E, L, off);
    if (key < L) atomicAdd(&cnt[w * L + key], 1);
  }
  __syncthreads();
  // per expert: counts of earlier waves (exclusive, in place) and the total
  for (int e = tid; e < L; e += 1024) {
    int run = 0;
    for (int v = 0; v < SB_WAVES; ++v) {
      const int c = cnt[v * L + e];
      cnt[v * L + e] = run;
      run += c;
    }
    start[e] = run;
  }
  __syncthreads();
  // exclusive scan of the expert totals (L <= 1024: one expert per thread)
  const int tot = tid < L ? start[tid] : 0;
  const int inc = wave_incl_scan(tot);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int before = 0;
  for (int v = 0; v < w; ++v) before += wsum[v];
  if (tid < L) {
    const int st = before + inc - tot;
    offs[tid] = st + tot;
    if (m_indptr) m_indptr[tid + 1] = st + tot;
    start[tid] = st;
  }
  if (tid == 0) {
    int all = 0;
    for (int v = 0; v < SB_WAVES; ++v) all += wsum[v];
    *n_local = all;
    if (m_indptr) m_indptr[0] = 0;
  }
  __syncthreads();
  for (int i = tid; i < SB_WAVES * L; i += 1024) cnt[i] += start[i % L];
  __syncthreads();
  // stable scatter: wave w only touches its own row cnt[w][*]
  int bits = 1;
  while ((1 << bits) <= L) ++bits;  // keys 0..L fit
  const uint64_t lt = (1ull << lane) - 1ull;
  int32_t* run = cnt + w * L;
  for (int base = b0; base < b1; base += 64) {
    const int i = base + lane;
    const bool valid = i < b1;
    const int key = valid ? local_key(ids[i], E, L, off) : L;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    const bool local = valid && key < L;
    const int pos = local ? run[key] + rank : -1;
    if (local && rank == 0) run[key] += __popcll(peers);
    if (valid) {
      e2p[i] = pos;
      if (pos >= 0) p2e[pos] = i;
    }
  }
}

// Chunk c's scatter. Every workgroup scans the L expert totals itself (L <= 1024,
// four per thread): cheaper than another launch.
__global__ __launch_bounds__(256) void k_sort_scatter(
    const int32_t* __restrict__ ids, int64_t n, int E, int L, int off,
    const int32_t* __restrict__ cnt, const int32_t* __restrict__ total,
    int32_t* __restrict__ offs, int32_t* __restrict__ m_indptr, int32_t* __restrict__ n_local,
    int32_t* __restrict__ e2p, int32_t* __restrict__ p2e) {
  extern __shared__ int32_t sm[];
  int32_t* run = sm;                        // [SORT_WAVES][L]: next row per wave and expert
  int32_t* start = sm + SORT_WAVES * L;     // [L]
  __shared__ int wsum[SORT_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = (int64_t)blockIdx.x * CHUNK + (int64_t)w * (CHUNK / SORT_WAVES);
  int keys[SORT_STEPS];  // all of the wave's ids are requested before any is used
#pragma unroll
  for (int step = 0; step < SORT_STEPS; ++step) {
    const int64_t i = base + step * 64 + lane;
    keys[step] = i < n ? local_key(ids[i], E, L, off) : L;
  }
  for (int i = tid; i < SORT_WAVES * L; i += 256) run[i] = 0;
  // exclusive scan of the expert totals: thread tid owns experts [4 tid, 4 tid + 4)
  int tv[4], part = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    tv[j] = e < L ? total[e] : 0;
    part += tv[j];
  }
  const int inc = wave_incl_scan(part);
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  int excl = inc - part;
  for (int v = 0; v < w; ++v) excl += wsum[v];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = 4 * tid + j;
    if (e < L) {
      start[e] = excl;
      if (blockIdx.x == 0) {
        offs[e] = excl + tv[j];
        if (m_indptr) m_indptr[e + 1] = excl + tv[j];
      }
    }
    excl += tv[j];
  }
  if (blockIdx.x == 0 && tid == 255) {
    *n_local = excl;  // the last thread ends with the grand total
    if (m_indptr) m_indptr[0] = 0;
  }
  // each wave's count of its quarter, per expert
#pragma unroll
  for (int step = 0; step < SORT_STEPS; ++step)
    if (keys[step] < L) atomicAdd(&run[w * L + keys[step]], 1);
  __syncthreads();
  // first row of each (wave, expert): expert start + chunk prefix + earlier waves
  const int32_t* pre = cnt + (int64_t)blockIdx.x * L;
  for (int e = tid; e < L; e += 256) {
    int acc = start[e] + pre[e];
#pragma unroll
    for (int v = 0; v < SORT_WAVES; ++v) {
      const int h = run[v * L + e];
      run[v * L + e] = acc;
      acc += h;
    }
  }
  __syncthreads();
  int bits = 1;
  while ((1 << bits) <= L) ++bits;  // keys 0..L fit
  const uint64_t lt = (1ull << lane) - 1ull;
  int32_t* myrun = run + w * L;
#pragma unroll
  for (int step = 0; step < SORT_STEPS; ++step) {
    const int64_t i = base + step * 64 + lane;
    const bool valid = i < n;
    const int key = keys[step];
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < bits; ++b) {
      const uint64_t m = __ballot((key >> b) & 1);
      peers &= ((key >> b) & 1) ? m : ~m;
    }
    const int rank = __popcll(peers & lt);
    int pos = -1;
    if (valid && key < L) pos = myrun[key] + rank;
    // the wave alone uses its run row: its LDS accesses take effect in order
    if (valid && key < L && rank == 0) myrun[key] += __popcll(peers);
    if (valid) {
      e2p[i] = pos;
      if (pos >= 0) p2e[pos] = (int32_t)i;
    }
  }
}

__global__ void k_sort_empty(int L, int32_t* offs, int32_t* m_indptr, int32_t* n_local) {
  for (int e = threadIdx.x; e < L; e += blockDim.x) {
    offs[e] = 0;
    if (m_indptr) m_indptr[e + 1] = 0;
  }
  if (threadIdx.x == 0) {
    *n_local = 0;
    if (m_indptr) m_indptr[0] = 0;
  }
}

inline int64_t n_chunks(int64_t n) { return (n + CHUNK - 1) / CHUNK; }

}  // namespace

size_t sort_workspace_bytes(int64_t T, int32_t k, int32_t L) {
  int64_t nb = n_chunks(T * (int64_t)k);
  return align_up((size_t)(L * nb + L) * sizeof(int32_t), 256);
}

moe_status sort_enqueue(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t L,
                        int32_t off, int32_t* offs, int32_t* m_indptr, int32_t* e2p,
                        int32_t* p2e, int32_t* n_local, void* ws, hipStream_t st, int32_t* zero,
                        int n_zero) {
  const int64_t n = T * (int64_t)k;
  if (n == 0) {
    k_sort_empty<<<1, 256, 0, st>>>(L, offs, m_indptr, n_local);
    return launch_status();
  }
  const size_t sb_lds = (size_t)(SB_WAVES * L + L + SB_WAVES) * sizeof(int32_t);
  if (n <= SB_MAX && sb_lds <= 65536) {
    k_sort_block<<<1, 1024, sb_lds, st>>>(ids, (int)n, E, L, off, offs, m_indptr, n_local, e2p, p2e,
                                          zero, zero ? n_zero : 0);
    return launch_status();
  }
  const int64_t nb = n_chunks(n);
  int32_t* cnt = reinterpret_cast<int32_t*>(ws);
  int32_t* total = cnt + L * nb;
  k_sort_count<<<(unsigned)nb, 256, (size_t)L * sizeof(int32_t), st>>>(ids, n, E, L, off, cnt);
  k_sort_scan<<<(unsigned)((L + SCAN_E - 1) / SCAN_E), 1024, 0, st>>>(cnt, (int)nb, L, total, zero,
                                                          zero ? n_zero : 0);
  k_sort_scatter<<<(unsigned)nb, 256, (size_t)(SORT_WAVES + 1) * L * sizeof(int32_t), st>>>(
      ids, n, E, L, off, cnt, total, offs, m_indptr, n_local, e2p, p2e);
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_sort_workspace_size(int64_t T, int32_t top_k, int32_t L) {
  if (T < 0 || top_k < 1 || L < 1) return 0;
  return sort_workspace_bytes(T, top_k, L);
}

extern "C" moe_status moe_sort(const int32_t* topk_ids, int64_t T, int32_t top_k, int32_t E,
                               int32_t L, int32_t off, int32_t* offs, int32_t* m_indptr,
                               int32_t* e2p, int32_t* p2e, int32_t* n_local, void* ws,
                               size_t ws_bytes, void* stream) {
  if (T < 0 || top_k < 1 || top_k > 16 || E < 1 || E > 1024 || L < 1 || off < 0 || L + off > E)
    return MOE_ERR_SHAPE;
  if (!offs || !n_local) return MOE_ERR_NULL;
  if (T > 0 && (!topk_ids || !e2p || !p2e)) return MOE_ERR_NULL;
  if (T * (int64_t)top_k > (int64_t)INT32_MAX) return MOE_ERR_SHAPE;
  if (T > 0 && (!ws || ws_bytes < sort_workspace_bytes(T, top_k, L))) return MOE_ERR_WORKSPACE;
  return sort_enqueue(topk_ids, T, top_k, E, L, off, offs, m_indptr, e2p, p2e, n_local, ws,
                      as_stream(stream), nullptr, 0);
}
