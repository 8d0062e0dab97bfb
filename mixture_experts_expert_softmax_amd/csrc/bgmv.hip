// BGMV MoE-LoRA shrink + expand over routed (token, expert) pairs.
//
// BGMV page ("flashinfer.fused_moe.prepare_bgmv_moe"), signature, Parameters and
// description: per pair p with token t = sorted_token_ids[p], expert e =
// expert_ids[p] and LoRA l = lora_indices[t],
//   shrink  s[p, :] = x[t] @ A[l, e].T           (rank values, stored in bf16)
//   expand  y[t, :] = sum over t's pairs, ascending p, of w[p] * (s[p] @ B[l, e].T)
// with y in float32. Every output has one owner that sums its routes in that fixed
// order, so results are the same on every run. Few pairs: the shrink splits the
// hidden dimension over extra workgroups and a second launch sums each pair's fp32
// partials in split order.
//
// Both steps stream LoRA weights (cache- / HBM-bound GEMV work): one workgroup per
// (pair, hidden split) for the shrink -- the x segment staged in LDS, each wave
// owning rank rows and each lane 16-byte chunks of a row, butterfly-reduced -- and
// one per (token, 256 output columns) for the expand, each thread one column whose
// B row (rank values) it reads with 16-byte loads. The shrink publishes each pair in
// a 16-slot token -> pair index; the expand sorts a token's slots ascending, or
// scans all pairs in order for a token with more than 16.
//
// Grouped pipeline (BGMV page, Parameters: grouped), for many routes per (LoRA,
// expert) bin: the pairs are grouped by bin (one workgroup up to 4096 pairs, else
// moe_sort's kernels with one bin per (LoRA, expert)); the shrink and the expand then
// run on bf16 MFMAs over tiles of 32 routes of one bin (x rows gathered through the routes' tokens against the
// bin's A, K = hidden; shrink rows against the bin's B, K = rank), so each bin's
// weights are streamed once per tile of routes rather than once per pair. Both keep
// their operands in registers: the rank (8-64) is far narrower than the 256-wide
// tiles of the layer GEMMs. The expand writes w[p] times its fp32 result as pair p's
// partial row, and a per-token combine sums a token's partials in ascending pair
// order.
#include <type_traits>
#include <algorithm>

#include "common.h"

namespace moe {
// defined in sort.hip / gemm_bf16.hip
size_t sort_workspace_bytes(int64_t T, int32_t k, int32_t L);
moe_status sort_enqueue(const int32_t* ids, int64_t T, int32_t k, int32_t E, int32_t L,
                        int32_t off, int32_t* offs, int32_t* m_indptr, int32_t* e2p,
                        int32_t* p2e, int32_t* n_local, void* ws, hipStream_t st,
                        int32_t* zero, int n_zero);

namespace {

constexpr int BG_SLOTS = 16;
constexpr int BG_SPLIT_MAX = 8;
constexpr int BG_XSEG = 2048;   // 16-byte x chunks staged per shrink workgroup (32 KB)

struct BgArgs {
  const uint4* x;              // [T][H/8]
  const uint4* A;              // [nl][E][r][H/8]
  const uint4* B;              // [nl][E][N][r/8]
  const int32_t* tok;          // [P]
  const int32_t* ex;           // [P]
  const int32_t* lidx;         // [T]
  const float* w;              // [P]
  uint16_t* s;                 // [P][r] bf16
  float* y;                    // [T][ldy]
  int64_t ldy;
  int32_t* cnt;                // [T] routes published per token
  int32_t* ri;                 // [T][BG_SLOTS]
  float* part;                 // [P][S][r]
  int64_t T, P;
  int H8, N, r, nl, E, S;
};

__device__ __forceinline__ bool pair_ok(const BgArgs& a, int64_t p, int& t, int& e, int& l) {
  t = a.tok[p];
  e = a.ex[p];
  if (t < 0 || t >= a.T || e < 0 || e >= a.E) return false;
  l = a.lidx[t];
  return l >= 0 && l < a.nl;
}

__device__ __forceinline__ float dot8(uint4 u, uint4 v, float acc) {
  const uint32_t a[4] = {u.x, u.y, u.z, u.w};
  const uint32_t b[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    acc = fmaf(__uint_as_float(a[q] << 16), __uint_as_float(b[q] << 16), acc);
    acc = fmaf(__uint_as_float(a[q] & 0xFFFF0000u), __uint_as_float(b[q] & 0xFFFF0000u), acc);
  }
  return acc;
}

__global__ __launch_bounds__(256) void k_bgmv_zero(int32_t* __restrict__ cnt, int64_t T) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < T) cnt[i] = 0;
}

// Workgroup (pair p, split sp) of the shrink; wave w owns rank rows w + 4i (RPW of
// them). A lane walks its chunks c = lane, lane + 64, ... and loads chunk c of all its
// rows together (independent loads, one latency for all rows), keeping one fp32 sum per
// row in chunk order; the rows are then reduced across the wave by butterflies.
template <int RPW>
__global__ __launch_bounds__(256) void k_bgmv_shrink(BgArgs a) {
  __shared__ uint4 xs[BG_XSEG];
  const int64_t p = blockIdx.x / a.S;
  const int sp = (int)(blockIdx.x - p * a.S);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  int t, e, l;
  if (!pair_ok(a, p, t, e, l)) {   // contributes nothing; its shrink row reads as zeros
    if (sp == 0 && tid < a.r) a.s[p * a.r + tid] = 0;
    return;
  }
  if (sp == 0 && tid == 0) {
    const int slot = atomicAdd(a.cnt + t, 1);
    if (slot < BG_SLOTS) a.ri[(int64_t)t * BG_SLOTS + slot] = (int32_t)p;
  }
  const int c0 = (int)((int64_t)a.H8 * sp / a.S), c1 = (int)((int64_t)a.H8 * (sp + 1) / a.S);
  const int nc = c1 - c0;
  for (int c = tid; c < nc; c += 256) xs[c] = a.x[(int64_t)t * a.H8 + c0 + c];
  __syncthreads();
  const uint4* Ab = a.A + (((int64_t)l * a.E + e) * a.r + wid) * a.H8 + c0;
  float acc[RPW];
#pragma unroll
  for (int i = 0; i < RPW; ++i) acc[i] = 0.f;
  for (int c = lane; c < nc; c += 64) {
    uint4 v[RPW];
#pragma unroll
    for (int i = 0; i < RPW; ++i) v[i] = Ab[(int64_t)(4 * i) * a.H8 + c];
    const uint4 xv = xs[c];
#pragma unroll
    for (int i = 0; i < RPW; ++i) acc[i] = dot8(xv, v[i], acc[i]);
  }
#pragma unroll
  for (int i = 0; i < RPW; ++i) {
    float v = acc[i];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    acc[i] = v;
  }
  if (lane == 0) {
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int j = wid + 4 * i;
      if (a.S == 1)
        a.s[p * a.r + j] = (uint16_t)(pack_bf16x2(acc[i], 0.f) & 0xFFFFu);
      else
        a.part[(p * a.S + sp) * a.r + j] = acc[i];
    }
  }
}

// Split shrink, second launch: s[p, j] = bf16 of the sum of pair p's S fp32 partials
// in split order (the launch boundary orders the partials' stores before these loads;
// a cross-workgroup release at agent scope, which writes back the XCD's L2, cost more
// than the rest of the shrink). Thread = (pair, rank row).
__global__ __launch_bounds__(256) void k_bgmv_split_sum(BgArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.P * a.r) return;
  const int64_t p = i / a.r;
  int t, e, l;
  if (!pair_ok(a, p, t, e, l)) return;   // its row was zeroed by the shrink
  float v = 0.f;
  for (int q = 0; q < a.S; ++q) v += a.part[p * a.S * a.r + q * a.r + (i - p * a.r)];
  a.s[i] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
}

// Workgroup (token t, 256-column tile) of the expand; thread = output column. The
// token's pairs are taken in ascending order in batches of up to 16: their shrink
// rows, weights and experts are staged in LDS (shared by all columns), then each
// thread loads the B rows of 4 pairs at a time (independent loads) and adds the
// pairs' terms in order. RC = rank / 8 (16-byte chunks of a row).
template <int RC>
__global__ __launch_bounds__(256) void k_bgmv_expand(BgArgs a, int col_tiles) {
  __shared__ int32_t plist[256];
  __shared__ uint4 ssh[BG_SLOTS][RC];
  __shared__ float wsh[BG_SLOTS];
  __shared__ int esh[BG_SLOTS];
  __shared__ int nlist;
  __shared__ int wcount[4];
  const int64_t t = blockIdx.x / col_tiles;
  const int ct = (int)(blockIdx.x - t * col_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = ct * 256 + tid;
  const bool col_ok = c < a.N;
  const int l = a.lidx[t];
  float acc = 0.f;
  // pairs plist[i0 .. i0 + nb), nb <= 16, in order
  auto run_batch = [&](int i0, int nb) {
    if (tid < nb * RC) {
      const int u = tid / RC, q = tid - u * RC;
      const int64_t p = plist[i0 + u];
      ssh[u][q] = reinterpret_cast<const uint4*>(a.s + p * a.r)[q];
      if (q == 0) {
        wsh[u] = a.w[p];
        esh[u] = a.ex[p];
      }
    }
    __syncthreads();
    const int64_t cc = col_ok ? c : 0;
    for (int u0 = 0; u0 < nb; u0 += 4) {
      uint4 bv[4][RC];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u0 + u < nb) {
          const uint4* bp = a.B + (((int64_t)l * a.E + esh[u0 + u]) * a.N + cc) * RC;
#pragma unroll
          for (int q = 0; q < RC; ++q) bv[u][q] = bp[q];
        }
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (u0 + u < nb) {
          float d = 0.f;
#pragma unroll
          for (int q = 0; q < RC; ++q) d = dot8(ssh[u0 + u][q], bv[u][q], d);
          acc = fmaf(wsh[u0 + u], d, acc);
        }
    }
    __syncthreads();
  };
  const int n = a.cnt[t];
  if (n <= BG_SLOTS) {
    // the published slots in ascending order: slot i goes to its rank among the n
    // (pair indices are distinct)
    if (tid < n) {
      const int v = a.ri[t * BG_SLOTS + tid];
      int rank = 0;
      for (int k = 0; k < n; ++k) rank += a.ri[t * BG_SLOTS + k] < v;
      plist[rank] = v;
    }
    __syncthreads();
    if (n > 0) run_batch(0, n);
  } else {   // more than 16 routes: scan every pair in order, 256 at a time
    for (int64_t base = 0; base < a.P; base += 256) {
      const int64_t p = base + tid;
      int tt = -1, ee = 0, ll = 0;
      const bool hit = p < a.P && pair_ok(a, p, tt, ee, ll) && tt == t;
      const uint64_t m = __ballot(hit);
      if (lane == 0) wcount[wid] = __popcll(m);
      __syncthreads();
      const int before = (wid > 0 ? wcount[0] : 0) + (wid > 1 ? wcount[1] : 0) + (wid > 2 ? wcount[2] : 0);
      if (hit) plist[before + __popcll(m & ((1ull << lane) - 1))] = (int32_t)p;
      if (tid == 0) nlist = wcount[0] + wcount[1] + wcount[2] + wcount[3];
      __syncthreads();
      const int nl = nlist;
      for (int i = 0; i < nl; i += BG_SLOTS) run_batch(i, nl - i < BG_SLOTS ? nl - i : BG_SLOTS);
      __syncthreads();   // wcount / nlist / plist are rewritten by the next chunk
    }
  }
  if (col_ok) a.y[t * a.ldy + c] = acc;
}

// Grouped pipeline, step 1: each valid pair's bin (LoRA * E + expert; -1 for a pair
// that contributes nothing) and its slot in the token -> pair index.
__global__ __launch_bounds__(256) void k_bgmv_bins(BgArgs a, int32_t* __restrict__ bins) {
  const int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= a.P) return;
  int t, e, l;
  if (!pair_ok(a, p, t, e, l)) {   // contributes nothing; its shrink row reads as zeros
    bins[p] = -1;
    for (int j = 0; j < a.r; ++j) a.s[p * a.r + j] = 0;
    return;
  }
  bins[p] = l * a.E + e;
  const int slot = atomicAdd(a.cnt + t, 1);
  if (slot < BG_SLOTS) a.ri[(int64_t)t * BG_SLOTS + slot] = (int32_t)p;
}

// Grouped pipeline, step 1 for up to GP_MAX_PAIRS pairs, in place of the index clear,
// k_bgmv_bins and the sort: one workgroup clears the token index, bins every pair
// (publishing it in the index), counts each bin in LDS, scans the counts into the bin
// ends and places every valid pair in its bin. The order within a bin is whatever the
// LDS atomics give: the shrink and the expand compute a route the same way wherever it
// sits in its tile and the combine adds by pair index, so the results do not depend
// on it.
// Measured (hidden 3072, rank 32, 32 bins, cold cache, whole grouped call): 4096
// pairs 76.3 -> 69.4 us, 2048 pairs 60.2 -> 52.6 us; at 16384 pairs one workgroup is
// too little (204.8 -> 220.3 us with 16 pairs per thread), so the three launches stay
// there.
constexpr int GP_THREADS = 1024;
constexpr int GP_PER_THREAD = 4;
constexpr int GP_MAX_PAIRS = GP_THREADS * GP_PER_THREAD;

__global__ __launch_bounds__(GP_THREADS) void k_bgmv_prep(BgArgs a, int L, int32_t* __restrict__ offs,
                                                        int32_t* __restrict__ p2e) {
  __shared__ int cntb[1024];   // per-bin counts, then starts (L <= 1024)
  __shared__ int wsum[GP_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  for (int i = tid; i < L; i += GP_THREADS) cntb[i] = 0;
  // cleared with atomic stores, on the same path as the atomic increments after the
  // barrier
  for (int64_t t = tid; t < a.T; t += GP_THREADS)
    __hip_atomic_store(a.cnt + t, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  // each stage for all of the thread's pairs before the next (loads, then the
  // dependent loads, then the atomics), so their latencies overlap
  int tk[GP_PER_THREAD], ek[GP_PER_THREAD], lk[GP_PER_THREAD], bin[GP_PER_THREAD],
      slot[GP_PER_THREAD], ts[GP_PER_THREAD];
#pragma unroll
  for (int k = 0; k < GP_PER_THREAD; ++k) {
    const int p = tid + k * GP_THREADS;
    tk[k] = p < a.P ? a.tok[p] : -1;
    ek[k] = p < a.P ? a.ex[p] : -1;
  }
#pragma unroll
  for (int k = 0; k < GP_PER_THREAD; ++k) {
    const bool ok = tk[k] >= 0 && tk[k] < a.T && ek[k] >= 0 && ek[k] < a.E;
    lk[k] = ok ? a.lidx[tk[k]] : -1;
  }
#pragma unroll
  for (int k = 0; k < GP_PER_THREAD; ++k) {
    const int p = tid + k * GP_THREADS;
    const bool valid = tk[k] >= 0 && tk[k] < a.T && ek[k] >= 0 && ek[k] < a.E && lk[k] >= 0 &&
                       lk[k] < a.nl;
    bin[k] = valid ? lk[k] * a.E + ek[k] : -1;
    if (valid) {
      slot[k] = atomicAdd(&cntb[bin[k]], 1);
      ts[k] = atomicAdd(a.cnt + tk[k], 1);
    } else if (p < a.P) {   // contributes nothing; its shrink row reads as zeros
      for (int j = 0; j < a.r; ++j) a.s[(int64_t)p * a.r + j] = 0;
    }
  }
#pragma unroll
  for (int k = 0; k < GP_PER_THREAD; ++k)
    if (bin[k] >= 0 && ts[k] < BG_SLOTS)
      a.ri[(int64_t)tk[k] * BG_SLOTS + ts[k]] = tid + k * GP_THREADS;
  __syncthreads();
  // bin ends: inclusive scan of the counts (waves, then the wave totals)
  const int v = tid < L ? cntb[tid] : 0;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(incl, d);
    if (lane >= d) incl += u;
  }
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  for (int w = 0; w < wv; ++w) incl += wsum[w];
  if (tid < L) {
    offs[tid] = incl;
    cntb[tid] = incl - v;   // the bin's start (only this thread read its count)
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < GP_PER_THREAD; ++k)
    if (bin[k] >= 0) p2e[cntb[bin[k]] + slot[k]] = (int32_t)(tid + k * GP_THREADS);
}

// Grouped pipeline, step 2 (after the sort by bin), the shrink: s[p] = bf16(x[tok[p]] . A[bin]^T) for the routes of each bin in
// sorted order, 32 routes (one MFMA column block) per workgroup, dealt XCD by XCD so a
// bin's workgroups share its A slice in one L2. The rank is only 8-64 wide, so the
// 256 x 256 GEMM tile would spend most of its MFMAs on masked columns; here the
// operands go straight from global memory into registers. Lane l takes route / A row
// l % 32 and, of every 64-value block of the contraction, the 32 values from
// 32 (l / 32): four 16-byte loads, fed to four MFMA steps in that order (the same
// permutation of the contraction on both operands). The 8 waves take every 8th block
// and their sums meet in LDS, added in wave order.
constexpr int GS_WAVES = 8;

template <int NCB>
__global__ __launch_bounds__(GS_WAVES * 64) void k_bgmv_gshrink(BgArgs a,
                                                              const int32_t* __restrict__ offs,
                                                              int L, const int32_t* __restrict__ p2e,
                                                              int ks, float* __restrict__ hs) {
  // 64-value blocks a wave loads before it multiplies (all of them issued before the
  // first MFMA: one memory round trip per batch; hidden 3072 is one batch below rank 64)
  constexpr int GS_BATCH = 6 / NCB;
  __shared__ float red[GS_WAVES][NCB][16][64];
  int e, m0, mend, nt;
  // nt: the tile's part of the contraction (ks parts; ks = 2 when the tiles would
  // occupy at most half the CUs -- each part then leaves fp32 sums that the expand adds)
  if (!deal_tile<32>(offs, L, (int)a.P, ks, e, m0, mend, nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  // wave-uniform in a scalar register: the contraction loop below is then not a
  // lane-masked loop (an MFMA must run with every lane of the wave)
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int i = m0 + j < mend ? m0 + j : mend - 1;   // rows past the bin repeat a valid one
  const int tok = a.tok[p2e[i]];
  // element offsets from the argument pointers (global loads, kept in flight together;
  // a lane outside the operands loads chunk 0 of its row and zeroes the value)
  const int64_t xo = (int64_t)tok * a.H8;
  int64_t wo[NCB];
  bool wok[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int wrow = cb * 32 + j;
    wok[cb] = wrow < a.r;
    wo[cb] = ((int64_t)e * a.r + (wok[cb] ? wrow : 0)) * a.H8;
  }
  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
  const int nb = (a.H8 + 7) >> 3;
  const int cbeg = nb * nt / ks, cend = nb * (nt + 1) / ks;   // this part's 64-value blocks
  const uint4 z = make_uint4(0, 0, 0, 0);
  for (int c0 = cbeg + wid; c0 < cend; c0 += GS_WAVES * GS_BATCH) {
    uint4 xv[GS_BATCH][4], wv[GS_BATCH][NCB][4];
#pragma unroll
    for (int g = 0; g < GS_BATCH; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k8 = 8 * (c0 + GS_WAVES * g) + 4 * h + u;   // 16-byte chunk of the row
        const bool ok = c0 + GS_WAVES * g < cend && k8 < a.H8;
        const int kk = ok ? k8 : 0;
        xv[g][u] = a.x[xo + kk];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) wv[g][cb][u] = a.A[wo[cb] + kk];
      }
    __builtin_amdgcn_sched_barrier(0);   // keep the batch's loads ahead of its MFMAs
#pragma unroll
    for (int g = 0; g < GS_BATCH; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int k8 = 8 * (c0 + GS_WAVES * g) + 4 * h + u;
        const bool ok = c0 + GS_WAVES * g < cend && k8 < a.H8;
        const uint4 xq = ok ? xv[g][u] : z;
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8, ok && wok[cb] ? wv[g][cb][u] : z),
              __builtin_bit_cast(bf16x8, xq), acc[cb], 0, 0, 0);
      }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int v = 0; v < 16; ++v) red[wid][cb][v][lane] = acc[cb][v];
  __syncthreads();
  if (wid != 0 || m0 + j >= mend) return;
  // lane holds A rows 8 q + 4 h + 0..3 (accumulator entries 4 q + 0..3) of route j
  const int64_t pj = p2e[m0 + j];
  uint16_t* out = a.s + pj * a.r;
  float* hout = hs + (pj * ks + nt) * a.r;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = cb * 32 + 8 * q + 4 * h;
      if (c >= a.r) continue;
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float t = red[0][cb][4 * q + r][lane];
#pragma unroll
        for (int w = 1; w < GS_WAVES; ++w) t += red[w][cb][4 * q + r][lane];
        f[r] = t;
      }
      if (ks == 1)
        *reinterpret_cast<uint2*>(out + c) = make_uint2(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]));
      else
        *reinterpret_cast<float4*>(hout + c) = make_float4(f[0], f[1], f[2], f[3]);
    }
}

// Step 3, the expand: part[p] = w[p] * (s[p] . B[bin]^T) in fp32 for the sorted routes
// of each bin: 32 routes x 512 output columns per workgroup, each wave 128 columns (4
// MFMA blocks), contraction = the rank (one or more 16-value MFMA steps). The routes
// are the MFMA's row operand and the B rows its column operand, so lane l holds output
// column l % 32 of routes 8 q + 4 (l / 32) + 0..3 and every store instruction writes 2
// routes x 32 adjacent floats (two whole 128-byte lines). Little LDS: several
// workgroups share a CU.
constexpr int GX_COLS = 512;

template <int R>
__global__ __launch_bounds__(256) void k_bgmv_gexpand(BgArgs a, const int32_t* __restrict__ offs,
                                                      int L, const int32_t* __restrict__ p2e,
                                                      float* __restrict__ part, int col_tiles,
                                                      int ks, const float* __restrict__ hs) {
  constexpr int NS = (R + 15) / 16;   // MFMA steps
  constexpr int RC = R / 8;           // 16-byte chunks per rank row
  __shared__ int rmap[32];
  __shared__ float wmap[32];
  int e, m0, mend, nt;
  if (!deal_tile<32>(offs, L, (int)a.P, col_tiles, e, m0, mend, nt)) return;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  if (tid < 32) {
    const int p = m0 + tid < mend ? p2e[m0 + tid] : -1;
    rmap[tid] = p;
    wmap[tid] = p >= 0 ? a.w[p] : 0.f;
  }
  const uint4 z = make_uint4(0, 0, 0, 0);
  const uint4* S4 = reinterpret_cast<const uint4*>(a.s);
  const int i = m0 + j < mend ? m0 + j : mend - 1;   // rows past the bin repeat a valid one
  const int64_t pi = p2e[i];
  const int64_t so = pi * RC;
  uint4 sv[NS], bv[4][NS];
#pragma unroll
  for (int u = 0; u < NS; ++u) {
    const int k8 = 2 * u + h;
    const int kk = k8 < RC ? k8 : 0;
    if (ks == 1) {
      sv[u] = S4[so + kk];
    } else {
      // a shrink cut in two parts: s = bf16(part 0 + part 1), written out by the
      // route's first column tile
      const float4* h0 = reinterpret_cast<const float4*>(hs + pi * 2 * R) + 2 * kk;
      const float4* h1 = h0 + R / 4;
      const float4 a0 = h0[0], a1 = h0[1], b0 = h1[0], b1 = h1[1];
      sv[u] = make_uint4(pack_bf16x2(a0.x + b0.x, a0.y + b0.y), pack_bf16x2(a0.z + b0.z, a0.w + b0.w),
                         pack_bf16x2(a1.x + b1.x, a1.y + b1.y), pack_bf16x2(a1.z + b1.z, a1.w + b1.w));
      if (nt == 0 && m0 + j < mend && k8 < RC) reinterpret_cast<uint4*>(a.s)[so + k8] = sv[u];
    }
  }
  const int c0 = nt * GX_COLS + wid * 128;
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int col = c0 + cb * 32 + j;
    const int64_t bo = ((int64_t)e * a.N + (col < a.N ? col : a.N - 1)) * RC;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int k8 = 2 * u + h;
      bv[cb][u] = a.B[bo + (k8 < RC ? k8 : 0)];
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[cb][v] = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const bool ok = 2 * u + h < RC;   // rank 8: the upper half of the step is padding
      acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          __builtin_bit_cast(bf16x8, ok ? sv[u] : z), __builtin_bit_cast(bf16x8, ok ? bv[cb][u] : z),
          acc[cb], 0, 0, 0);
    }
  }
  __syncthreads();   // rmap / wmap
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) {
    const int col = c0 + cb * 32 + j;
    if (col >= a.N) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ri = 8 * q + 4 * h + r;
        const int p = rmap[ri];
        if (p >= 0) part[(int64_t)p * a.N + col] = wmap[ri] * acc[cb][4 * q + r];
      }
  }
}

// Last step: y[t, c] = sum over t's valid pairs, ascending p, of part[p, c]. One
// workgroup per (token, 256 x CPT columns), thread = CPT adjacent columns (4 when y's
// rows are 16-byte aligned: 16-byte loads and stores); a token's pairs come from the
// index (ranked ascending) or, beyond 16 pairs, from a scan of all pairs in order.
template <int CPT>
__global__ __launch_bounds__(256) void k_bgmv_combine(BgArgs a, const float* __restrict__ part,
                                                      int col_tiles) {
  using V = typename std::conditional<CPT == 4, float4, float>::type;
  __shared__ int32_t plist[256];
  __shared__ int nlist;
  __shared__ int wcount[4];
  const int64_t t = blockIdx.x / col_tiles;
  const int ct = (int)(blockIdx.x - t * col_tiles);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int c = (ct * 256 + tid) * CPT;
  const bool col_ok = c < a.N;   // N is a multiple of 8
  float acc[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) acc[u] = 0.f;
  auto add_list = [&](int nb) {   // plist[0 .. nb), loads first, then the ordered sum
    for (int i0 = 0; i0 < nb; i0 += 8) {
      V v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (i0 + u < nb && col_ok) v[u] = *reinterpret_cast<const V*>(part + (int64_t)plist[i0 + u] * a.N + c);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (!(i0 + u < nb && col_ok)) continue;
        const float* f = reinterpret_cast<const float*>(&v[u]);
#pragma unroll
        for (int q = 0; q < CPT; ++q) acc[q] += f[q];
      }
    }
  };
  const int n = a.cnt[t];
  if (n <= BG_SLOTS) {
    if (tid < n) {
      const int v = a.ri[t * BG_SLOTS + tid];
      int rank = 0;
      for (int k = 0; k < n; ++k) rank += a.ri[t * BG_SLOTS + k] < v;
      plist[rank] = v;
    }
    __syncthreads();
    add_list(n);
  } else {   // more than 16 routes: scan every pair in order, 256 at a time
    for (int64_t base = 0; base < a.P; base += 256) {
      const int64_t p = base + tid;
      int tt = -1, ee = 0, ll = 0;
      const bool hit = p < a.P && pair_ok(a, p, tt, ee, ll) && tt == t;
      const uint64_t m = __ballot(hit);
      if (lane == 0) wcount[wid] = __popcll(m);
      __syncthreads();
      const int before = (wid > 0 ? wcount[0] : 0) + (wid > 1 ? wcount[1] : 0) + (wid > 2 ? wcount[2] : 0);
      if (hit) plist[before + __popcll(m & ((1ull << lane) - 1))] = (int32_t)p;
      if (tid == 0) nlist = wcount[0] + wcount[1] + wcount[2] + wcount[3];
      __syncthreads();
      add_list(nlist);
      __syncthreads();   // wcount / nlist / plist are rewritten by the next chunk
    }
  }
  if (col_ok) {
    V o;
    float* f = reinterpret_cast<float*>(&o);
#pragma unroll
    for (int q = 0; q < CPT; ++q) f[q] = acc[q];
    *reinterpret_cast<V*>(a.y + t * a.ldy + c) = o;
  }
}

}  // namespace

// The grouped pipeline serves at most this many (LoRA, expert) bins (moe_sort's limit).
constexpr int BG_GROUP_MAX_BINS = 1024;

bool bgmv_grouped(int mode, int64_t P, int nl, int E) {
  const int64_t bins = (int64_t)nl * E;
  if (bins > BG_GROUP_MAX_BINS || P == 0) return false;
  if (mode == MOE_BGMV_GROUPED) return true;
  if (mode == MOE_BGMV_PER_PAIR) return false;
  // measured crossover (hidden 3072, rank 32, 4 LoRAs x 8 experts on MI355X, cold
  // cache): per pair / grouped 47.6 / 60.0 us at 32 routes per bin, 64.4 / 61.4 at 48,
  // 77.6 / 62.2 at 64
  return P >= 48 * bins;
}

struct BgGroupLayout {
  size_t cnt, ri, bins, offs, e2p, p2e, n_sorted, s, hs, part, sort_ws, total;
};

BgGroupLayout bgmv_group_layout(int64_t T, int64_t P, int r, int N, int nl, int E) {
  BgGroupLayout g{};
  const int L = nl * E;
  size_t o = 0;
  g.cnt = o;      o += align_up((size_t)T * 4, 256);
  g.ri = o;       o += align_up((size_t)T * BG_SLOTS * 4, 256);
  g.bins = o;     o += align_up((size_t)P * 4, 256);
  g.offs = o;     o += align_up((size_t)L * 4, 256);
  g.e2p = o;      o += align_up((size_t)P * 4, 256);
  g.p2e = o;      o += align_up((size_t)P * 4, 256);
  g.n_sorted = o; o += 256;
  g.s = o;        o += align_up((size_t)P * r * 2, 256);
  g.hs = o;       o += align_up((size_t)P * 2 * r * 4, 256);   // two-part shrink sums
  g.part = o;     o += align_up((size_t)P * N * 4, 256);
  g.sort_ws = o;  o += align_up(sort_workspace_bytes(P, 1, L), 256);
  g.total = o;
  return g;
}

size_t bgmv_workspace_bytes(int64_t T, int64_t P, int r) {
  size_t o = 0;
  o += align_up((size_t)T * 4, 256);                       // cnt
  o += align_up((size_t)T * BG_SLOTS * 4, 256);            // ri
  o += align_up((size_t)P * BG_SPLIT_MAX * r * 4, 256);    // split partials
  o += align_up((size_t)P * r * 2, 256);                   // shrink rows (if not the caller's)
  return o;
}

// The grouped pipeline: bins + token index, stable sort by bin, the shrink (32 routes
// of a bin per workgroup), the expand grouped GEMM, the per-token combine.
moe_status bgmv_group_enqueue(const void* x, const void* A, const void* B, const int32_t* tok,
                              const int32_t* ex, const int32_t* lidx, const float* w,
                              void* shrink, float* y, int64_t ldy, int64_t T, int64_t P, int H,
                              int N, int r, int nl, int E, void* ws, hipStream_t st) {
  const BgGroupLayout g = bgmv_group_layout(T, P, r, N, nl, E);
  char* wp = reinterpret_cast<char*>(ws);
  const int L = nl * E;
  BgArgs a{};
  a.tok = tok;
  a.ex = ex;
  a.lidx = lidx;
  a.w = w;
  a.y = y;
  a.ldy = ldy;
  a.T = T;
  a.P = P;
  a.H8 = H / 8;
  a.N = N;
  a.r = r;
  a.nl = nl;
  a.E = E;
  a.cnt = reinterpret_cast<int32_t*>(wp + g.cnt);
  a.ri = reinterpret_cast<int32_t*>(wp + g.ri);
  int32_t* bins = reinterpret_cast<int32_t*>(wp + g.bins);
  int32_t* offs = reinterpret_cast<int32_t*>(wp + g.offs);
  int32_t* e2p = reinterpret_cast<int32_t*>(wp + g.e2p);
  int32_t* p2e = reinterpret_cast<int32_t*>(wp + g.p2e);
  int32_t* n_sorted = reinterpret_cast<int32_t*>(wp + g.n_sorted);
  void* s = shrink ? shrink : (void*)(wp + g.s);
  a.s = reinterpret_cast<uint16_t*>(s);
  float* part = reinterpret_cast<float*>(wp + g.part);
  moe_status st_ = MOE_OK;
  if (P <= GP_MAX_PAIRS) {
    k_bgmv_prep<<<1, GP_THREADS, 0, st>>>(a, L, offs, p2e);
    if ((st_ = launch_status()) != MOE_OK) return st_;
  } else {
    k_bgmv_zero<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(a.cnt, T);
    if ((st_ = launch_status()) != MOE_OK) return st_;
    k_bgmv_bins<<<(unsigned)((P + 255) / 256), 256, 0, st>>>(a, bins);
    if ((st_ = launch_status()) != MOE_OK) return st_;
    // stable sort of the pairs by bin (invalid pairs are foreign)
    st_ = sort_enqueue(bins, P, 1, L, L, 0, offs, nullptr, e2p, p2e, n_sorted, wp + g.sort_ws, st,
                       nullptr, 0);
    if (st_ != MOE_OK) return st_;
  }
  // shrink: s[p2e[i]] = bf16(x[tok[p2e[i]]] @ A[bin].T) for the sorted rows i of each bin
  a.x = reinterpret_cast<const uint4*>(x);
  a.A = reinterpret_cast<const uint4*>(A);
  const int64_t chunks = P / 32 + std::min<int64_t>(L, P);   // 32-row tiles over L bins
  // at most half as many tiles as CUs: cut each tile's contraction in two (twice the
  // workgroups, each moving half the bytes, still one round of one per CU). Measured
  // (hidden 3072, rank 32, 32 bins, cold cache): 1024 tokens 62.3 -> 60.4 us, 512
  // tokens 60.1 -> 56.2 us; at 2048 tokens the doubled grid takes a second round and
  // the shrink went from 19 to 31 us.
  const int ks = 2 * chunks <= device_cu_count() ? 2 : 1;
  float* hs = reinterpret_cast<float*>(wp + g.hs);
  const unsigned gsg = (unsigned)((chunks * ks + 7) / 8 * 8);
  if (r == 64)
    k_bgmv_gshrink<2><<<gsg, GS_WAVES * 64, 0, st>>>(a, offs, L, p2e, ks, hs);
  else
    k_bgmv_gshrink<1><<<gsg, GS_WAVES * 64, 0, st>>>(a, offs, L, p2e, ks, hs);
  if ((st_ = launch_status()) != MOE_OK) return st_;
  // expand: part[p2e[i]] = w[p2e[i]] * (s[p2e[i]] @ B[bin].T), fp32
  a.B = reinterpret_cast<const uint4*>(B);
  const int xt = (N + GX_COLS - 1) / GX_COLS;
  const unsigned gxg = (unsigned)((chunks * xt + 7) / 8 * 8);
  switch (r) {
    case 8: k_bgmv_gexpand<8><<<gxg, 256, 0, st>>>(a, offs, L, p2e, part, xt, ks, hs); break;
    case 16: k_bgmv_gexpand<16><<<gxg, 256, 0, st>>>(a, offs, L, p2e, part, xt, ks, hs); break;
    case 32: k_bgmv_gexpand<32><<<gxg, 256, 0, st>>>(a, offs, L, p2e, part, xt, ks, hs); break;
    default: k_bgmv_gexpand<64><<<gxg, 256, 0, st>>>(a, offs, L, p2e, part, xt, ks, hs); break;
  }
  if ((st_ = launch_status()) != MOE_OK) return st_;
  // 4 columns per thread where every row of y starts 16-byte aligned
  const bool vec = reinterpret_cast<uintptr_t>(y) % 16 == 0 && ldy % 4 == 0;
  const int col_tiles = (N + (vec ? 1023 : 255)) / (vec ? 1024 : 256);
  if (T * col_tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  if (vec)
    k_bgmv_combine<4><<<(unsigned)(T * col_tiles), 256, 0, st>>>(a, part, col_tiles);
  else
    k_bgmv_combine<1><<<(unsigned)(T * col_tiles), 256, 0, st>>>(a, part, col_tiles);
  return launch_status();
}

moe_status bgmv_enqueue(const void* x, const void* A, const void* B, const int32_t* tok,
                        const int32_t* ex, const int32_t* lidx, const float* w, void* shrink,
                        float* y, int64_t ldy, int64_t T, int64_t P, int H, int N, int r, int nl,
                        int E, void* ws, hipStream_t st) {
  if (T == 0) return MOE_OK;
  char* wp = reinterpret_cast<char*>(ws);
  BgArgs a{};
  a.x = reinterpret_cast<const uint4*>(x);
  a.A = reinterpret_cast<const uint4*>(A);
  a.B = reinterpret_cast<const uint4*>(B);
  a.tok = tok;
  a.ex = ex;
  a.lidx = lidx;
  a.w = w;
  a.y = y;
  a.ldy = ldy;
  a.T = T;
  a.P = P;
  a.H8 = H / 8;
  a.N = N;
  a.r = r;
  a.nl = nl;
  a.E = E;
  size_t o = 0;
  a.cnt = reinterpret_cast<int32_t*>(wp + o);  o += align_up((size_t)T * 4, 256);
  a.ri = reinterpret_cast<int32_t*>(wp + o);   o += align_up((size_t)T * BG_SLOTS * 4, 256);
  a.part = reinterpret_cast<float*>(wp + o);   o += align_up((size_t)P * BG_SPLIT_MAX * r * 4, 256);
  a.s = shrink ? reinterpret_cast<uint16_t*>(shrink) : reinterpret_cast<uint16_t*>(wp + o);
  // hidden splits: enough workgroups for two per CU, each split at least 64 chunks
  // per lane row pass and at most BG_XSEG chunks (its x segment lives in LDS)
  const int cu = device_cu_count();
  int S = 1;
  if (P > 0) {
    S = (int)std::min<int64_t>((2 * cu + P - 1) / P, BG_SPLIT_MAX);
    S = std::min(S, std::max(1, a.H8 / 64));
  }
  while ((a.H8 + S - 1) / S > BG_XSEG) ++S;
  if (S > BG_SPLIT_MAX) return MOE_ERR_UNSUPPORTED;
  a.S = S;
  k_bgmv_zero<<<(unsigned)((T + 255) / 256), 256, 0, st>>>(a.cnt, T);
  moe_status s = launch_status();
  if (s != MOE_OK) return s;
  if (P > 0) {
    if (P * S > INT32_MAX) return MOE_ERR_UNSUPPORTED;
    const unsigned g = (unsigned)(P * S);
    if (r == 8)
      k_bgmv_shrink<2><<<g, 256, 0, st>>>(a);
    else if (r == 16)
      k_bgmv_shrink<4><<<g, 256, 0, st>>>(a);
    else if (r == 32)
      k_bgmv_shrink<8><<<g, 256, 0, st>>>(a);
    else
      k_bgmv_shrink<16><<<g, 256, 0, st>>>(a);
    s = launch_status();
    if (s != MOE_OK) return s;
    if (S > 1) {
      k_bgmv_split_sum<<<(unsigned)((P * r + 255) / 256), 256, 0, st>>>(a);
      s = launch_status();
      if (s != MOE_OK) return s;
    }
  }
  const int col_tiles = (N + 255) / 256;
  if (T * col_tiles > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  const unsigned ge = (unsigned)(T * col_tiles);
  if (r == 8)
    k_bgmv_expand<1><<<ge, 256, 0, st>>>(a, col_tiles);
  else if (r == 16)
    k_bgmv_expand<2><<<ge, 256, 0, st>>>(a, col_tiles);
  else if (r == 32)
    k_bgmv_expand<4><<<ge, 256, 0, st>>>(a, col_tiles);
  else
    k_bgmv_expand<8><<<ge, 256, 0, st>>>(a, col_tiles);
  return launch_status();
}

}  // namespace moe

using namespace moe;

static moe_status check_bgmv(const moe_bgmv_desc* d) {
  if (!d) return MOE_ERR_NULL;
  if (d->num_tokens < 0 || d->num_pairs < 0 || d->num_pairs > INT32_MAX) return MOE_ERR_SHAPE;
  if (d->hidden < 8 || d->hidden % 8 || d->feat_out < 8 || d->feat_out % 8) return MOE_ERR_SHAPE;
  if (d->rank != 8 && d->rank != 16 && d->rank != 32 && d->rank != 64) return MOE_ERR_SHAPE;
  if (d->num_loras < 1 || d->num_experts < 1) return MOE_ERR_SHAPE;
  if (d->mode < MOE_BGMV_AUTO || d->mode > MOE_BGMV_GROUPED) return MOE_ERR_DTYPE;
  if (d->mode == MOE_BGMV_GROUPED && (int64_t)d->num_loras * d->num_experts > BG_GROUP_MAX_BINS)
    return MOE_ERR_UNSUPPORTED;
  if (d->hidden / 8 > BG_XSEG * BG_SPLIT_MAX) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

static size_t bgmv_ws_bytes(const moe_bgmv_desc* d) {
  if (bgmv_grouped(d->mode, d->num_pairs, d->num_loras, d->num_experts))
    return bgmv_group_layout(d->num_tokens, d->num_pairs, d->rank, d->feat_out, d->num_loras,
                             d->num_experts).total;
  return bgmv_workspace_bytes(d->num_tokens, d->num_pairs, d->rank);
}

extern "C" size_t moe_bgmv_workspace_size(const moe_bgmv_desc* d) {
  if (check_bgmv(d) != MOE_OK) return 0;
  return bgmv_ws_bytes(d);
}

extern "C" moe_status moe_bgmv(const moe_bgmv_desc* d, const void* x, const void* lora_a,
                               const void* lora_b, const int32_t* sorted_token_ids,
                               const int32_t* expert_ids, const int32_t* lora_indices,
                               const float* topk_weights, void* shrink_out, float* y_accum,
                               int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_bgmv(d);
  if (s != MOE_OK) return s;
  if (d->num_tokens == 0) return MOE_OK;
  if (ldy < d->feat_out) return MOE_ERR_SHAPE;
  if (!x || !lora_indices || !y_accum) return MOE_ERR_NULL;
  if (d->num_pairs > 0 && (!lora_a || !lora_b || !sorted_token_ids || !expert_ids || !topk_weights))
    return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(lora_a) || !aligned16(lora_b) ||
      (shrink_out && !aligned16(shrink_out)))
    return MOE_ERR_ALIGN;
  if (!ws || ws_bytes < bgmv_ws_bytes(d) || !aligned16(ws)) return MOE_ERR_WORKSPACE;
  if (bgmv_grouped(d->mode, d->num_pairs, d->num_loras, d->num_experts)) {
    if ((int64_t)d->num_tokens * d->hidden >= ((int64_t)1 << 32) ||
        (int64_t)d->num_pairs * d->feat_out >= ((int64_t)1 << 31))
      return MOE_ERR_UNSUPPORTED;
    return bgmv_group_enqueue(x, lora_a, lora_b, sorted_token_ids, expert_ids, lora_indices,
                              topk_weights, shrink_out, y_accum, ldy, d->num_tokens,
                              d->num_pairs, d->hidden, d->feat_out, d->rank, d->num_loras,
                              d->num_experts, ws, as_stream(stream));
  }
  return bgmv_enqueue(x, lora_a, lora_b, sorted_token_ids, expert_ids, lora_indices, topk_weights,
                      shrink_out, y_accum, ldy, d->num_tokens, d->num_pairs, d->hidden, d->feat_out,
                      d->rank, d->num_loras, d->num_experts, ws, as_stream(stream));
}
