// Ragged bf16 grouped GEMMs on gfx950 MFMA: fwd, dgrad, wgrad, and the MoE
// FC1 (SwiGLU / SwiGLUStep epilogue) and FC2 (row store or fused finalize).
//
// Grouped-GEMM page, operation table:
//   fwd    Y[rows of e]  = X[rows of e] @ W[e].T
//   dgrad  dX[rows of e] = G[rows of e] @ W[e]      (W read in place)
//   wgrad  dW[e]         = G[rows of e].T @ X[rows of e]   (empty group -> zeros)
// with groups given by cumulative end offsets read on the device, fp32
// accumulation and no atomics. SM90 fused-MoE page, formula: FC1 computes
// x @ w1[e].T for the up and gate rows and applies silu(gate) * up in the
// epilogue; FC2 computes act @ w2[e].T. StepFun page: SwiGLUStep clamps with a
// per-expert limit. SM90 page, use_fused_finalize: the FC2 epilogue may add
// the route-weighted rows straight into a zeroed output with bf16 atomics.
//
// Design (gfx950, wave64):
//  * Workgroup tile 256 (weight rows) x 256 (activation rows) x 64 (contraction),
//    256 threads = 4 waves arranged 2 x 2; each wave owns a 128 x 128 block held
//    as 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16 (256 fp32 per lane).
//  * The MFMA "A" operand is the weight side and "B" the activation side, so a
//    lane's accumulator holds 4 consecutive output columns of one output row:
//    epilogue stores are 8-byte (bf16) or 16-byte (fp32) runs.
//  * Whole 64-deep contractions (every case but a ragged fwd K): operands are
//    copied straight from global memory into LDS (global_load_lds_dwordx4, or a
//    buffer copy whose record count zero-fills past a ragged group or a matrix
//    edge) in four slots of 32-deep stages, three stages ahead; row-major tiles
//    are [256 rows][4 chunks of 16 B] swizzled by (row >> 2) & 3, K-major tiles
//    [32 contraction rows][32 chunks] swizzled by (row & 3) << 2 and read with
//    transposing ds_read_b64_tr_b16. Otherwise the tiles are staged through
//    registers as [256 rows][8 chunks] swizzled by (row >> 1) & 7, double buffered.
//  * Ragged groups: an upper bound of M tiles is launched (no host sync); each
//    workgroup decodes its (expert, row block) from the device offsets, clamps
//    row reads inside its group and masks stores. Rows of a partial contraction
//    tile are zero-filled.
//  * blockIdx -> tile: consecutive workgroups land on different XCDs, so every
//    XCD is given a contiguous range of the real tiles (counted on the device),
//    ordered expert-major, column tile, row block: the row blocks sharing a
//    weight tile run together on one XCD and read it from HBM once.
#include <type_traits>

#include "common.h"

namespace moe {
namespace {

constexpr int TB = 256;        // tile rows on each side
constexpr int TK = 64;         // contraction per stage
constexpr int NTHREADS = 256;  // 4 waves
constexpr int TILE_U4 = TB * TK * 2 / 16;  // uint4 slots per operand tile (2048)

enum Epi { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_SWIGLU_STEP = 2, EPI_FUSED = 3 };
constexpr int SPLIT_MAX = 8;   // parts a split tile is cut into at most
// The forward GEMMs take the work-queue kernel (k_gemm_nt_q) for at least QUEUE_GROUPS
// groups of at most QUEUE_ROWS expected rows each: there about half the groups end in a
// short tile and the tiles take many rounds. Measured (ms, queue / one tile per
// workgroup with the split last round): expert shard (32 of 256 experts, ~256 rows
// each) FC1 0.741 / 0.755, FC2 0.342 / 0.366; Mixtral T = 2048 (8 experts, ~512 rows)
// FC2 0.617 / 0.513 -- its last round is better cut along K; grouped fwd (16 groups,
// ~512 rows) 0.195 / 0.185.
constexpr int QUEUE_ROWS = 384;
constexpr int QUEUE_GROUPS = 16;

struct NtArgs {
  const uint16_t* A;         // activation rows, row stride K
  const int32_t* a_gather;   // optional: row p reads A row a_gather[p] / a_div
  int a_div;
  const uint16_t* B;         // weights [E][NB][K]
  int64_t b_stride;          // elements per expert
  const int32_t* ends;       // [E] cumulative group ends
  int E;
  int m_cap;                 // rows available in A / C (clamp for offsets)
  int NB;                    // weight rows per expert
  int N;                     // output columns
  int K;
  int n_tiles;
  int m_tiles;               // launched upper bound on row blocks
  uint16_t* C;               // bf16 output, row stride ldc
  int64_t ldc;
  int I;                     // FC1: act width; gate rows start at I
  const float* limits;       // FC1 step: [E] or NULL
  float def_limit;
  const float* route_w;      // fused finalize: topk weights [T*k]
  const int32_t* p2e;        // fused finalize: route of permuted row
  int top_k;
  float* h_out;              // FC1 (optional): fp32 pre-activations [rows][2I], up then gate
  float* split_ws;           // split tiles: fp32 partial tiles [SPLIT_SLOTS][TB * TB]
  int32_t* split_cnt;        // split tiles: arrival counters, 0 between launches
  int n_res;                 // workgroups resident at once (0: never split)
  bool mmajor;               // deal tiles column tile first (deal_tile_split)
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Tile (and contraction range, in units of ktiles) of this workgroup in the NT and
// dgrad kernels. With n_res resident workgroups, total tiles take total / n_res full rounds; when the
// remainder rem would leave most of the last round idle, each of those rem tiles
// is cut along K into S = min(n_res / rem, SPLIT_MAX) parts instead, which run
// side by side. The whole tiles are dealt as in deal_tile; part p of remainder
// tile i is workgroup full + 8 * ((i / 8) * S + p) + i % 8, so all parts of a
// tile share one XCD. slot = i * S + p indexes the partial-tile buffer, cidx = i
// the arrival counter.
// With mmajor the tiles are numbered column tile first (every group's row blocks of
// column tile 0, then of column tile 1, ...) instead of group first, so that the
// workgroups in flight on an XCD cover one band of output columns.
template <int TM = TB>
__device__ __forceinline__ bool deal_tile_split(const int32_t* ends, int E, int m_cap, int n_tiles,
                                                int n_res, int ktiles, int& e, int& m0, int& mend,
                                                int& nt, int& k0, int& nk, int& part, int& S,
                                                int& slot, int& cidx, bool mmajor = false) {
  const bool one_pass = E <= 64;   // a single scan serves count and lookup
  TileScan64 sc{};
  if (one_pass) sc = tile_scan64<TM>(ends, E, m_cap, n_tiles);
  const int total = one_pass ? sc.total : tile_count<TM>(ends, E, m_cap, n_tiles);
  const int b = (int)blockIdx.x;
  int full = total, rem = 0;
  S = 1;
  part = 0;
  if (n_res > 0) {
    full = total / n_res * n_res;
    rem = total - full;
    if (rem > 0) {
      S = n_res / rem;
      S = S < SPLIT_MAX ? S : SPLIT_MAX;
      S = S < ktiles ? S : ktiles;
    }
  }
  int t;
  if (S < 2) {
    S = 1;
    const int per = (total + 7) >> 3;
    t = (b & 7) * per + (b >> 3);
    if ((b >> 3) >= per || t >= total) return false;
  } else if (b < full) {
    t = (b & 7) * (full >> 3) + (b >> 3);
    S = 1;  // a whole tile
  } else {
    const int u = b - full, w = u >> 3;
    const int i = (w / S) * 8 + (u & 7);
    if (i >= rem) return false;
    part = w % S;
    t = full + i;
    slot = i * S + part;
    cidx = i;
  }
  if (mmajor) {
    const int rb = total / n_tiles;   // row blocks over all groups
    int unused;
    if (one_pass)
      tile_locate64<TM>(sc, n_tiles, 1, t % rb, e, m0, mend, unused);
    else
      tile_locate<TM>(ends, E, m_cap, 1, t % rb, e, m0, mend, unused);
    nt = t / rb;
  } else if (one_pass) {
    tile_locate64<TM>(sc, n_tiles, n_tiles, t, e, m0, mend, nt);
  } else {
    tile_locate<TM>(ends, E, m_cap, n_tiles, t, e, m0, mend, nt);
  }
  k0 = ktiles * part / S;
  nk = ktiles * (part + 1) / S - k0;
  return true;
}

// Which of a wave's 16 32x32 accumulator blocks (bit i * 4 + j of the result) hold
// results: block rows r0 + j * 32 (j < jn) below rend, block columns c0 + i * 32 below cend.
__device__ __forceinline__ int block_mask(int r0, int rend, int jn, int c0, int cend) {
  int m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (j < jn && r0 + j * 32 < rend && c0 + i * 32 < cend) m |= 1 << (i * 4 + j);
  return m;
}

// Part `part` of S of a split tile publishes its fp32 partial into slot `slot` of
// the split workspace; the last of the S parts to arrive (counter cidx) sums all of
// them in part order -- the same result whichever part arrives last -- into acc and
// returns true (it goes on to the epilogue); the others return false. Only the blocks
// in the wave's mask vmask (wave-uniform, the same for every part) are written and
// summed. The sum is a single workgroup's job and bound by the loads it keeps in
// flight: it takes the parts two at a time, with all of one accumulator row's loads
// of both issued before any is used.
__device__ __forceinline__ bool split_reduce(f32x16 (&acc)[4][4], float* split_ws, int32_t* split_cnt,
                                             int slot, int part, int S, int cidx, uint4* smem,
                                             int tid, int vmask) {
  constexpr int TILE_F4 = TB * TB / 4;
  float4* mine = reinterpret_cast<float4*>(split_ws) + (size_t)slot * TILE_F4;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (!(vmask >> (i * 4 + j) & 1)) continue;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        mine[((i * 4 + j) * 4 + q) * NTHREADS + tid] =
            make_float4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2],
                        acc[i][j][4 * q + 3]);
    }
  __syncthreads();
  int* flag = reinterpret_cast<int*>(smem);
  if (tid == 0) {
    const int old = __hip_atomic_fetch_add(split_cnt + cidx, 1, __ATOMIC_ACQ_REL,
                                           __HIP_MEMORY_SCOPE_AGENT);
    flag[0] = old == S - 1;
    if (old == S - 1) split_cnt[cidx] = 0;  // ready for the next launch
  }
  __syncthreads();
  if (!flag[0]) return false;
  const float4* first = reinterpret_cast<const float4*>(split_ws) + (size_t)(slot - part) * TILE_F4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!(vmask >> (i * 4) & 15)) continue;
    for (int p = 0; p < S; p += 2) {
      const bool two = p + 1 < S;
      const float4* s0 = first + (size_t)p * TILE_F4;
      const float4* s1 = two ? s0 + TILE_F4 : s0;   // never past the last part
      float4 w0[4][4], w1[4][4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!(vmask >> (i * 4 + j) & 1)) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int idx = ((i * 4 + j) * 4 + q) * NTHREADS + tid;
          w0[j][q] = s0[idx];
          w1[j][q] = two ? s1[idx] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (!(vmask >> (i * 4 + j) & 1)) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 a0 = w0[j][q], a1 = w1[j][q];
          if (p == 0) {   // ((p0 + p1) + p2) + ...: part order
            acc[i][j][4 * q] = a0.x;
            acc[i][j][4 * q + 1] = a0.y;
            acc[i][j][4 * q + 2] = a0.z;
            acc[i][j][4 * q + 3] = a0.w;
          } else {
            acc[i][j][4 * q] += a0.x;
            acc[i][j][4 * q + 1] += a0.y;
            acc[i][j][4 * q + 2] += a0.z;
            acc[i][j][4 * q + 3] += a0.w;
          }
          if (two) {
            acc[i][j][4 * q] += a1.x;
            acc[i][j][4 * q + 1] += a1.y;
            acc[i][j][4 * q + 2] += a1.z;
            acc[i][j][4 * q + 3] += a1.w;
          }
        }
      }
    }
  }
  return true;
}

// One 64-deep stage of MFMAs: wave (wn, wm) multiplies its 128 weight rows by its
// 128 activation rows.
__device__ __forceinline__ void mma_stage(const uint4* __restrict__ Ws, const uint4* __restrict__ Xs,
                                          int wn, int wm, int lane, f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int ch = ((kk << 1) + (lane >> 5)) ^ ((lane >> 1) & 7);
    bf16x8 wf[4], xf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) wf[i] = as_bf16x8(Ws[(wn * 128 + i * 32 + (lane & 31)) * 8 + ch]);
#pragma unroll
    for (int j = 0; j < 4; ++j) xf[j] = as_bf16x8(Xs[(wm * 128 + j * 32 + (lane & 31)) * 8 + ch]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[i], xf[j], acc[i][j], 0, 0, 0);
  }
}

// Tile rows that are contiguous along the contraction: thread tid owns rows
// (tid>>3) + 32j, 16-byte chunk (tid&7) of every 64-wide stage.
struct RowLoader {
  const uint16_t* base;
  uint32_t off[8];
  int K;
  int ch;
  uint4 r[8];
  __device__ __forceinline__ void load(int kt) {
    const int k0 = kt * TK + ch * 8;
    const bool ok = k0 < K;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      r[j] = ok ? *reinterpret_cast<const uint4*>(base + off[j] + k0) : make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void store(uint4* __restrict__ lds, int tid) const {
    const int row = tid >> 3;
    const int pc = ch ^ ((row >> 1) & 7);
#pragma unroll
    for (int j = 0; j < 8; ++j) lds[(row + 32 * j) * 8 + pc] = r[j];
  }
};

typedef short v4i16 __attribute__((ext_vector_type(4)));

// MFMA fragment of a K-major LDS tile: lane L gets output column
// cb + L % 32 and contraction values 16 kk + 8 (L / 32) + 0..7. ds_read_b64_tr_b16
// works on groups of 16 lanes: lane 4j + a of a group addresses contraction row
// kb + j, columns 4a .. 4a + 3 of the group's 16 columns, and lane i of the group
// receives column i at rows kb .. kb + 3 (established on the device with an
// index-valued tile). Two reads give the 8 contraction values.
__device__ __forceinline__ bf16x8 ktile_frag(const uint4* __restrict__ lds, int kk, int cb, int lane) {
  typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
  const int g = lane >> 4, i = lane & 15;
  const int col = cb + 16 * (g & 1) + 4 * (i & 3);
  const int row = kk * 16 + 8 * (g >> 1) + (i >> 2);
  const int chunk = col >> 3, half = (col >> 2) & 1;
  char* t = const_cast<char*>(reinterpret_cast<const char*>(lds));
  const int o0 = row * 512 + ((chunk ^ ((row & 3) << 2)) << 4) + half * 8;
  const int o1 = (row + 4) * 512 + ((chunk ^ (((row + 4) & 3) << 2)) << 4) + half * 8;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + o0));
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(t + o1));
  typedef short v8i16 __attribute__((ext_vector_type(8)));
  const v8i16 both{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  return __builtin_bit_cast(bf16x8, both);
}

__device__ __forceinline__ void zero_acc(f32x16 (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
}

__device__ __forceinline__ void atomic_add_bf16x2_bits(uint16_t* p, uint32_t bits) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  __builtin_amdgcn_global_atomic_fadd_v2bf16(reinterpret_cast<bf16x2_t*>(p),
                                             __builtin_bit_cast(bf16x2_t, bits));
}

// Direct-to-LDS copy of one 16-byte chunk per lane: the chunk at g lands at LDS byte
// address lds + 16 * lane (lds goes to M0). The compiler does not see this LDS
// write, so the loop below counts copies in flight itself (vmcnt) before each barrier
// that publishes a stage.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// The backward products' full-K main loop (mainloop_dma_g below; the forward's is
// mainloop_fwd64) is a pipeline of 32-deep stages fetched straight into LDS without
// passing through registers (32 KB a stage: the 256 activation rows, then the 256
// weight rows; 64 bytes of a row-major operand's row). Stage s + DMA_DIST is requested
// while stage s is consumed, so a copy has about two stages of MFMA work to land, and
// each copy is issued right after one fragment read so the copies go out spread over
// the stage's MFMAs (issued back to back, they stall the wave on the address unit
// ahead of its MFMAs). A row-major row's four 16-byte chunks are stored at
// chunk ^ ((row / 4) % 4), which keeps the 32-row fragment reads free of bank
// conflicts; copy j of wave w covers rows 64 j + 16 w + lane / 4, so lane l fetches
// global chunk (l % 4) ^ ((l / 16) % 4). The loop is rotated by one 16-deep step: the
// last step of a stage runs after the barrier, under the first fragment reads of the
// next. Stages past the end re-load the last one into a slot nobody reads, which keeps
// the copy count uniform.
constexpr int DMA_SLOTS = 4;
constexpr int DMA_DIST = DMA_SLOTS - 1;   // stages between a copy and its use
constexpr int DMA_STAGE_U4 = 2 * TB * 32 * 2 / 16;   // uint4 slots per 32-deep stage
constexpr int LDS_U4 = DMA_SLOTS * DMA_STAGE_U4;      // 128 KB: dgrad / wgrad
constexpr int LDS_FWD_U4 = 5 * TB * 128 / 16;                    // 160 KB: mainloop_fwd64
static_assert(LDS_U4 >= 4 * TILE_U4, "the partial-K path's two 64-deep stages fit");


// Copy of one 16-byte chunk per lane through a buffer resource: lands at LDS byte
// address lds + 16 * lane; offsets at or past the resource's record count read as
// zeros, which is how the copies below end ragged contractions and matrix edges.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r), "{m0}"(lds) : "memory");
}

// Copy sources of the backward kernels' operands, for the same four-slot pipeline of
// 32-deep stages (activation side in the first 16 KB of a stage, weight side in the
// second). A copy instruction of wave w fills LDS bytes 4096 j + 1024 w .. + 1023
// of its half, i.e.
//  - row-major (contraction contiguous): rows 64 j + 16 w + lane / 4, 64 bytes
//    each, chunk swizzle (row / 4) % 4 -- as in the forward loop;
//  - K-major (contraction rows of 256 output columns, 512 bytes): contraction
//    rows 8 j + 2 w + lane / 32, chunk (lane % 32) ^ ((row % 4) << 2) -- the
//    layout the transposing fragment reads expect.
struct RmSrc {              // row-major operand
  const uint16_t* base;
  uint32_t off[4];          // element offsets of the thread's 4 rows
  int gch;                  // global chunk the lane fetches
  __device__ __forceinline__ void init(int tid) {
    const int lane = tid & 63;
    gch = (lane & 3) ^ ((lane >> 4) & 3);
  }
};
struct KmSrc {              // K-major operand: contraction row 0, first output column
  const char* base;
  int64_t ld2;              // bytes per contraction row
  int rows;                 // valid contraction rows from base
  int cols2;                // valid bytes of a row from base
  uint32_t voff[4];         // byte offsets of the thread's chunks within a stage
  __device__ __forceinline__ void init(int tid) {
    const int lane = tid & 63, w = tid >> 6;
    const int c = (lane & 31) ^ (((2 * w + (lane >> 5)) & 3) << 2);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      voff[j] = (uint32_t)((8 * j + 2 * w + (lane >> 5)) * ld2) + (uint32_t)c * 16u;
  }
  // resource over stage `sub` (< ceil(rows / 32), so at least one valid row): records
  // end at the last valid byte of the operand. A stage reads at most 31 rows past its
  // first plus one row, so counting at most 33 rows keeps the count exact in 32 bits.
  __device__ __forceinline__ __amdgpu_buffer_rsrc_t stage(int sub) const {
    int left = rows - sub * 32;
    left = left < 33 ? left : 33;
    const int n = (left - 1) * (int)ld2 + cols2;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base + (int64_t)sub * 32 * ld2),
                                             (short)0, n, 0x00020000);
  }
};

// Backward main loop: the direct-to-LDS pipeline above (four 32-deep slots, copies
// three stages ahead interleaved with fragment reads, rotated by one step) for a
// K-major weight side and an activation side in either layout. A = weight side (output columns), B = activation
// side (output rows); kbase is the row-major operand's first contraction element.
// JN = 32-row activation blocks per wave: 4 for the whole 256-row tile; 1 (row-major
// activation side only) for a tile of at most 64 rows, where row-wave wm takes rows
// 32 wm .. 32 wm + 31, each wave issues only its first activation copy (rows 0..63)
// and a step has 4 MFMAs instead of 16 -- the ragged last tile of a group.
template <bool A_K, bool B_K, int JN, class SA, class SB>
__device__ __forceinline__ void mainloop_dma_g(const SA& sa, const SB& sb, uint4* smem, int kbase,
                                               int nsub, int tid, int lane, int wn, int wm,
                                               f32x16 (&acc)[4][4]) {
  static_assert(A_K, "the forward (both operands row-major) runs mainloop_fwd64");
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem + (uint32_t)w * 1024u;
  const int rsel = lane & 31, kg = lane >> 5, sw = (rsel >> 2) & 3;
  constexpr uint32_t STAGE_B = DMA_STAGE_U4 * 16, HALF_B = STAGE_B / 2;
  constexpr int NCOPY = 4 + (B_K ? 4 : JN);   // copies per wave per stage
  // the 4 copies of one operand's part of stage `sub` into LDS half at byte d
  auto copy_rm = [&](const RmSrc& src, int sub, uint32_t d, int j) {
    dma16(src.base + src.off[j] + kbase + sub * 32 + src.gch * 8, d + j * 4096u);
  };

  bf16x8 wf[2][4], xf[2][4];
  auto rd_a = [&](const uint4* As, int kk, int set, int i) {
    if constexpr (A_K) wf[set][i] = ktile_frag(As, kk, wn * 128 + i * 32, lane);
    else wf[set][i] = as_bf16x8(As[(wn * 128 + i * 32 + rsel) * 4 + (((kk << 1) + kg) ^ sw)]);
  };
  auto rd_b = [&](const uint4* Bs, int kk, int set, int j) {
    if constexpr (B_K) xf[set][j] = ktile_frag(Bs, kk, wm * 128 + j * 32, lane);
    else xf[set][j] = as_bf16x8(Bs[(wm * JN * 32 + j * 32 + rsel) * 4 + (((kk << 1) + kg) ^ sw)]);
  };
  // fragment reads of step kk of the stage in `slot`, each of the first four
  // followed by one copy of operand H (0: B, 1: A) of stage `sub` into slot `dslot`
  auto rd_issue = [&](int slot, int kk, int set, int sub, int dslot, auto hsel) {
    constexpr int H = decltype(hsel)::value;
    constexpr bool KM = H == 0 ? B_K : A_K;
    const uint4* Bs = smem + slot * DMA_STAGE_U4;
    const uint4* As = Bs + DMA_STAGE_U4 / 2;
    const uint32_t d = lds0 + (uint32_t)dslot * STAGE_B + (uint32_t)H * HALF_B;
    const auto& src = [&]() -> const auto& {
      if constexpr (H == 0) return sb; else return sa;
    }();
    if constexpr (KM) {
      const __amdgpu_buffer_rsrc_t r = src.stage(sub);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rd_a(As, kk, set, i);
        dma16_buf(r, src.voff[i], d + i * 4096u);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) rd_b(Bs, kk, set, j);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rd_a(As, kk, set, i);
        copy_rm(src, sub, d, i);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) rd_b(Bs, kk, set, j);
    }
  };
  auto mm = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[set][i], xf[set][j], acc[i][j], 0, 0, 0);
  };
  auto issue = [&](int sub, int slot) {
    const uint32_t d = lds0 + (uint32_t)slot * STAGE_B;
    if constexpr (B_K) {
      const __amdgpu_buffer_rsrc_t r = sb.stage(sub);
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_buf(r, sb.voff[j], d + j * 4096u);
    } else {
#pragma unroll
      for (int j = 0; j < JN; ++j) copy_rm(sb, sub, d, j);
    }
    if constexpr (A_K) {
      const __amdgpu_buffer_rsrc_t r = sa.stage(sub);
#pragma unroll
      for (int j = 0; j < 4; ++j) dma16_buf(r, sa.voff[j], d + HALF_B + j * 4096u);
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) copy_rm(sa, sub, d + HALF_B, j);
    }
  };
  auto body = [&](int sub, bool first) {
    const int slot = sub % DMA_SLOTS;
    const int nxt = sub + DMA_DIST < nsub ? sub + DMA_DIST : nsub - 1;
    const int dslot = (sub + DMA_DIST) % DMA_SLOTS;
    rd_issue(slot, 0, 0, nxt, dslot, std::integral_constant<int, 0>{});
    if (!first) mm(1);
    rd_issue(slot, 1, 1, nxt, dslot, std::integral_constant<int, 1>{});
    mm(0);
    // a step's NR fragment reads (two transposing reads per K-major fragment) go
    // between the previous step's 16 MFMAs
    constexpr int NR = (A_K ? 8 : 4) + (B_K ? 8 : JN);
    constexpr int NM = 4 * JN;
    if (first) __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
    for (int q = 0; q < (first ? 1 : 2); ++q) {
      for (int r = 0; r < (NM > NR ? NM : NR); ++r) {
        if (r < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (r < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCOPY * (DMA_DIST - 1)) : "memory");
    __syncthreads();
  };
#pragma unroll
  for (int q = 0; q < DMA_DIST; ++q) issue(q < nsub ? q : nsub - 1, q);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NCOPY * (DMA_DIST - 1)) : "memory");
  __syncthreads();
  body(0, true);
  for (int sub = 1; sub < nsub; ++sub) body(sub, false);
  mm(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Forward main loop over 64-deep stages with whole 128-byte rows for both operands:
// each lane group of 8 copies one row's 128 bytes (a whole cache line), and a row's 8
// chunks sit at chunk ^ ((row / 2) % 8) in LDS, which keeps the 32-row fragment reads
// (16 lanes at a time, 16 bytes each) on distinct banks. The five 32 KB slots of LDS
// (160 KB) hold NWS weight slots and 5 - NWS activation slots (64 JN rows each); a
// ring of n slots has its stage m + n - 1 copied while stage m is consumed. Iteration
// m copies the shorter ring's next stage in its first half and the longer ring's in
// its second half, and ends with one barrier after waiting for all but the longer
// ring's copies, so both rings' next stages have landed. Two weight and three
// activation slots measured best (the activation rows, gathered or shared by many
// column tiles, come from L2 and the Infinity Cache and gain from the longer lead;
// expert shard -4%, the Mixtral layer unchanged). Copy j of wave w covers rows
// 32 j + 8 w + lane / 8 of either operand (woff, xoff: row offsets in elements; gch:
// the global chunk lane l fetches, (l % 8) ^ ((row / 2) % 8)).
template <int JN>
__device__ __forceinline__ void mainloop_fwd64(const uint16_t* wbase, const uint32_t (&woff)[8],
                                               const uint16_t* xbase, const uint32_t (&xoff)[8], int gch,
                                               uint4* smem, int kbase, int nst, int tid, int lane, int wn,
                                               int wm, f32x16 (&acc)[4][4]) {
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem + (uint32_t)w * 1024u;
  // weight / activation slots (a ring of n slots copies its stages n - 1 ahead): the
  // activation slot holds 64 JN rows, so smaller tiles get more of them
  constexpr uint32_t SLOT_B = TB * 128, XSLOT_B = 64 * JN * 128;
  constexpr int NWS = JN == 4 ? 2 : 3;
  constexpr int NXS = (int)((5 * SLOT_B - NWS * SLOT_B) / XSLOT_B);
  constexpr uint32_t XRING_B = NWS * SLOT_B;
  static_assert(NWS >= 2 && NXS >= 2, "both rings need a slot beside the one being read");
  static_assert(NWS * SLOT_B + NXS * XSLOT_B <= 5 * SLOT_B, "the rings exceed 160 KB");
  constexpr int DW = NWS - 1, DX = NXS - 1;   // copy lead of each ring, in stages
  constexpr int NXC = 2 * JN;     // activation copies per wave per stage (64 JN rows)
  const int rsel = lane & 31, kg = lane >> 5, sw = (rsel >> 1) & 7;
  auto copy_w = [&](int m, int slot, int j) {
    dma16(wbase + woff[j] + kbase + m * 64 + gch * 8, lds0 + (uint32_t)slot * SLOT_B + j * 4096u);
  };
  auto copy_x = [&](int m, int slot, int j) {
    dma16(xbase + xoff[j] + kbase + m * 64 + gch * 8, lds0 + XRING_B + (uint32_t)slot * XSLOT_B + j * 4096u);
  };
  bf16x8 wf[2][4], xf[2][4];
  // fragment reads of 16-deep step q of stage m into register set `set`; copy c of
  // the step's 4 (after every second read) is activation copy 4 q + c of stage xs
  // (steps 0 and 1) or weight copy 4 (q - 2) + c of stage ws (steps 2 and 3)
  auto rd_issue = [&](int m, auto qsel, int set, int xs, int xsl, int ws, int wsl) {
    constexpr int Q = decltype(qsel)::value;
    const uint4* Ws = smem + (size_t)(m % NWS) * (SLOT_B / 16);
    const uint4* Xs = smem + (XRING_B + (size_t)(m % NXS) * XSLOT_B) / 16;
    auto cp = [&](int c) {   // the ring with the shorter distance is copied first
      constexpr bool XFIRST = NXS <= NWS;
      constexpr int QX = XFIRST ? 0 : 2, QW = XFIRST ? 2 : 0;
      if constexpr (Q >= QX && Q < QX + 2) {
        if (4 * (Q - QX) + c < NXC) copy_x(xs, xsl, 4 * (Q - QX) + c);
      } else {
        copy_w(ws, wsl, 4 * (Q - QW) + c);
      }
    };
    // read order wf[0], xf[0 .. JN-1], wf[1 .. 3]: the order in which the next step's
    // MFMAs (weight fragment outer) first need them, so that each read is issued at
    // least six MFMAs before its first use; a copy follows every second read
    auto rd = [&](int r) {
      if (r == 0) {
        wf[set][0] = as_bf16x8(Ws[(wn * 128 + rsel) * 8 + (((Q << 1) + kg) ^ sw)]);
      } else if (r <= JN) {
        const int j = r - 1;
        xf[set][j] = as_bf16x8(Xs[(wm * JN * 32 + j * 32 + rsel) * 8 + (((Q << 1) + kg) ^ sw)]);
      } else {
        const int i = r - JN;
        wf[set][i] = as_bf16x8(Ws[(wn * 128 + i * 32 + rsel) * 8 + (((Q << 1) + kg) ^ sw)]);
      }
    };
    constexpr int NRD = 4 + JN;
#pragma unroll
    for (int r = 0; r < NRD; ++r) {
      rd(r);
      if ((r & 1) && (r >> 1) < 4) cp(r >> 1);
    }
#pragma unroll
    for (int c = NRD / 2; c < 4; ++c) cp(c);
  };
  auto mm = [&](int set) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[set][i], xf[set][j], acc[i][j], 0, 0, 0);
  };
  auto interleave = [&](int nsteps) {
    constexpr int NR = 4 + JN, NM = 4 * JN;
    for (int q = 0; q < nsteps; ++q) {
      if constexpr (JN == 4) {   // 8 reads: one between each pair of MFMAs
        for (int r = 0; r < 8; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        }
      } else {
        for (int r = 0; r < (NM > NR ? NM : NR); ++r) {
          if (r < NM) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (r < NR) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
  };
  // iteration m: the reads of step q + 1 go between the MFMAs of step q; the first
  // MFMAs finish the previous stage's last step (rotated loop)
  auto body = [&](int m, bool first) {
    const int xs = m + NXS - 1 < nst ? m + NXS - 1 : nst - 1;
    const int ws = m + NWS - 1 < nst ? m + NWS - 1 : nst - 1;
    const int xsl = (m + NXS - 1) % NXS, wsl = (m + NWS - 1) % NWS;
    rd_issue(m, std::integral_constant<int, 0>{}, 0, xs, xsl, ws, wsl);
    if (!first) mm(1);
    rd_issue(m, std::integral_constant<int, 1>{}, 1, xs, xsl, ws, wsl);
    mm(0);
    rd_issue(m, std::integral_constant<int, 2>{}, 0, xs, xsl, ws, wsl);
    mm(1);
    rd_issue(m, std::integral_constant<int, 3>{}, 1, xs, xsl, ws, wsl);
    mm(0);
    if (first) __builtin_amdgcn_sched_group_barrier(0x100, 4 + JN, 0);
    interleave(first ? 3 : 4);
    __builtin_amdgcn_sched_barrier(0);
    // only the copies of the ring with the longer distance, issued last, stay in flight
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NXS <= NWS ? 8 : NXC) : "memory");
    __syncthreads();
  };
  // prologue: the stages before each ring's first in-loop copy, in stage order; then
  // wait for stage 0 of both (all copies of later stages may stay in flight)
#pragma unroll
  for (int st = 0; st < (DW > DX ? DW : DX); ++st) {
    if (st < DW) {
#pragma unroll
      for (int j = 0; j < 8; ++j) copy_w(st < nst ? st : nst - 1, st, j);
    }
    if (st < DX) {
#pragma unroll
      for (int j = 0; j < NXC; ++j) copy_x(st < nst ? st : nst - 1, st, j);
    }
  }
  constexpr int LATER = 8 * (DW - 1) + NXC * (DX - 1);
  static_assert(LATER + 8 + NXC <= 63, "copies in flight exceed the vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LATER) : "memory");
  __syncthreads();
  body(0, true);
  for (int m = 1; m < nst; ++m) body(m, false);
  mm(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// ---------------------------------------------------------------------------
// fwd / FC1 / FC2: both operands contiguous along the contraction.
// ---------------------------------------------------------------------------
// TM: activation rows per tile, 256 or (full-K path only) 128 -- the family for few
// rows per expert, where each row-wave takes 64 rows (two 32-row blocks).
// One tile of the forward kernels: rows [m0, mend) of group e, column tile nt,
// contraction stages [k0, k0 + nk) (a part of a split tile when S > 1), computed by
// the whole workgroup (t: the thread index) and stored by the epilogue.
template <int EPI, bool KFULL, int TM>
__device__ __forceinline__ void nt_tile(const NtArgs& a, uint4* smem, int e, int m0, int mend,
                                        int nt, int k0, int nk, int part, int S, int slot,
                                        int cidx, int t) {
  const int ktiles = (a.K + TK - 1) / TK;
  (void)ktiles;
  const int tid = t, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int lrow = tid >> 3;

  RowLoader la, lb;
  la.base = a.A;
  la.K = a.K;
  la.ch = tid & 7;
  lb.base = a.B + (int64_t)e * a.b_stride;
  lb.K = a.K;
  lb.ch = tid & 7;
  // source rows of the activation copies: the gathered indices are loaded together
  // (one wait for all eight, not one per row)
  int src[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int p = m0 + lrow + 32 * j;
    src[j] = p < mend ? p : mend - 1;
  }
  gather_rows(a.a_gather, a.a_div, src);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    la.off[j] = (uint32_t)src[j] * (uint32_t)a.K;
    const int R = lrow + 32 * j;
    int wrow;
    if (EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_STEP) {
      int c = nt * 128 + (R >> 7) * 64 + (R & 63);
      // rows past the edge load distinct valid rows (their results are masked): many
      // copies of one row in a stage serialize on its cache line
      c = c < a.I ? c : c % a.I;
      wrow = ((R >> 6) & 1) * a.I + c;
    } else {
      wrow = nt * TB + R;
      wrow = wrow < a.NB ? wrow : wrow % a.NB;
    }
    lb.off[j] = (uint32_t)wrow * (uint32_t)a.K;
  }

  f32x16 acc[4][4];
  zero_acc(acc);
  int jn = 4;   // 32-row blocks per wave

  if (KFULL) {
    // rows lrow + 32 j of both operands (la.off, lb.off), whole 128-byte rows per copy
    const int wgch = (lane & 7) ^ ((4 * wid + (lane >> 4)) & 7);
    // a short last tile of its group (at most 64 rows) runs one 32-row block per row
    // wave and copies only its first 64 activation rows
    const int rows = mend - m0;
    if (rows <= 64) {
      jn = 1;
      mainloop_fwd64<1>(lb.base, lb.off, la.base, la.off, wgch, smem, k0 * TK, nk, tid, lane, wn, wm, acc);
    } else if (TM == 128) {
      jn = 2;
      mainloop_fwd64<2>(lb.base, lb.off, la.base, la.off, wgch, smem, k0 * TK, nk, tid, lane, wn, wm, acc);
    } else {
      mainloop_fwd64<4>(lb.base, lb.off, la.base, la.off, wgch, smem, k0 * TK, nk, tid, lane, wn, wm, acc);
    }
    // a part of a split tile: the last of its parts to arrive finishes the tile
    if (S > 1 && !split_reduce(acc, a.split_ws, a.split_cnt, slot, part, S, cidx, smem, tid,
                               block_mask(m0 + wm * jn * 32, mend, jn, nt * TB + wn * 128,
                                          EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_STEP ? TB * a.n_tiles
                                                                                      : a.N)))
      return;
  } else {
    la.load(0);
    lb.load(0);
    la.store(smem, tid);
    lb.store((smem + TILE_U4), tid);
    __syncthreads();
    for (int kt = 0; kt < ktiles; ++kt) {
      const int s = kt & 1;
      const bool more = kt + 1 < ktiles;
      if (more) {
        la.load(kt + 1);
        lb.load(kt + 1);
      }
      mma_stage((smem + TILE_U4 + s * 2 * TILE_U4), (smem + s * 2 * TILE_U4), wn, wm, lane, acc);
      if (more) {
        la.store((smem + (s ^ 1) * 2 * TILE_U4), tid);
        lb.store((smem + TILE_U4 + (s ^ 1) * 2 * TILE_U4), tid);
      }
      __syncthreads();
    }
  }

  // ---- epilogue: lane holds rows m, 4 consecutive columns per (i, q); row block j
  // of wave row wm starts at row 32 (wm jn + j) of the tile
  const int hi4 = (lane >> 5) * 4;
  constexpr bool FC1 = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_STEP;
  {
    // Staged through LDS (free once every wave is past the loop): in registers a lane
    // holds 4 columns of one row, so stores straight from registers would put 32 rows
    // x 8 bytes in each instruction -- 32 partial cache lines, whose write requests
    // then bound the epilogue (about 10 us per 256 x 256 tile with every CU storing at
    // once). The tile goes to LDS in rows (16-byte chunks XOR-swizzled by row, so the
    // 32 rows of a write and the chunks of a read fall on distinct banks) and leaves
    // in whole rows: 16 bytes per lane, each instruction covering whole 128-byte
    // lines. Every output pointer is 16-byte aligned and every row stride a multiple
    // of 16 bytes (the entry points' rules).
    constexpr int TC = FC1 ? 128 : TB;   // output columns of the tile
    constexpr int NCH = TC / 8;          // 16-byte bf16 chunks per tile row
    constexpr int RSB = TC * 2;          // LDS bytes per bf16 tile row
    constexpr int NI = FC1 ? 2 : 4;      // 32-column blocks per wave
    constexpr int CW = TC / 2;           // tile columns per wave
    char* lds = reinterpret_cast<char*>(smem);
    const int rows = mend - m0 < 64 * jn ? mend - m0 : 64 * jn;
    float lim = 0.f;
    if (EPI == EPI_SWIGLU_STEP) lim = a.limits ? a.limits[e] : a.def_limit;
    float wgt[4] = {1.f, 1.f, 1.f, 1.f};
    if (EPI == EPI_FUSED) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int p = m0 + wm * jn * 32 + j * 32 + (lane & 31);
        wgt[j] = (j < jn && p < mend) ? a.route_w[a.p2e[p]] : 0.f;
      }
    }
    __syncthreads();   // no wave still reads a stage or has a copy in flight
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j >= jn) continue;
      const int R = wm * jn * 32 + j * 32 + (lane & 31);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * CW + i * 32 + q * 8 + hi4;
          float v[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (FC1) {
              float u = acc[i][j][q * 4 + r];
              float g = acc[i + 2][j][q * 4 + r];
              if (EPI == EPI_SWIGLU_STEP) {
                u = fminf(fmaxf(u, -lim), lim);
                g = fminf(fmaxf(g, -lim), lim);
              }
              v[r] = silu_f32(g) * u;
            } else {
              v[r] = EPI == EPI_FUSED ? wgt[j] * acc[i][j][q * 4 + r] : acc[i][j][q * 4 + r];
            }
          }
          const uint32_t off = (uint32_t)(R * RSB + ((((c >> 3) ^ (R % NCH)) << 4) | (hi4 << 1)));
          *reinterpret_cast<uint2*>(lds + off) =
              make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
        }
    }
    __syncthreads();
    {
      // read back: lane k of a row's NCH lanes takes chunk k; 64 / NCH rows per read
      constexpr int RPI = 64 / NCH;
      const int k = lane % NCH;
      const int col = nt * TC + k * 8;
      if (col < (FC1 ? a.I : a.N)) {
#pragma unroll 4
        for (int r0 = wid * RPI; r0 < rows; r0 += 4 * RPI) {
          const int R = r0 + lane / NCH;
          if (R >= rows) continue;
          const uint4 v = *reinterpret_cast<const uint4*>(lds + R * RSB + ((k ^ (R % NCH)) << 4));
          const int p = m0 + R;
          if (EPI == EPI_FUSED) {
            uint16_t* d = a.C + (int64_t)(a.p2e[p] / a.top_k) * a.ldc + col;
            atomic_add_bf16x2_bits(d, v.x);
            atomic_add_bf16x2_bits(d + 2, v.y);
            atomic_add_bf16x2_bits(d + 4, v.z);
            atomic_add_bf16x2_bits(d + 6, v.w);
          } else {
            *reinterpret_cast<uint4*>(a.C + (int64_t)p * a.ldc + col) = v;
          }
        }
      }
    }
    if constexpr (FC1) {
      // the training forward also keeps the fp32 pre-activations h = [up | gate]
      // (exactly the values the activation above saw): two more passes of
      // [256 rows][128 floats], up then gate, each leaving in whole rows
      if (a.h_out) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          __syncthreads();   // the previous pass's reads are done
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j >= jn) continue;
            const int R = wm * jn * 32 + j * 32 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int c = wn * 64 + i * 32 + q * 8 + hi4;   // 4 floats: one chunk
                const f32x16& s4 = acc[i + 2 * half][j];
                *reinterpret_cast<float4*>(lds + R * 512 + (((c >> 2) ^ (R & 31)) << 4)) =
                    make_float4(s4[q * 4 + 0], s4[q * 4 + 1], s4[q * 4 + 2], s4[q * 4 + 3]);
              }
          }
          __syncthreads();
          const int k = lane & 31;   // 16-byte chunk of a 512-byte row; 2 rows per read
          const int col = nt * 128 + k * 4;
          if (col < a.I) {
#pragma unroll 4
            for (int r0 = wid * 2; r0 < rows; r0 += 8) {
              const int R = r0 + (lane >> 5);
              if (R >= rows) continue;
              const float4 v = *reinterpret_cast<const float4*>(lds + R * 512 + ((k ^ (R & 31)) << 4));
              *reinterpret_cast<float4*>(a.h_out + (int64_t)(m0 + R) * 2 * a.I + half * a.I + col) = v;
            }
          }
        }
      }
    }
  }
}

// Work-queue form of the whole-stage forward kernel, for groups of few rows, whose
// short last tiles (at most 64 rows: a quarter of the MFMAs) finish well before the
// others. Workgroups reach the XCDs in a fixed order, so with one workgroup per tile a
// CU freed early waits until every XCD has a free CU; here one workgroup per CU takes
// tiles until none are left. The tiles are dealt as in deal_tile -- XCD x owns the
// contiguous range [x per, (x + 1) per) of the group-major order, so the row blocks
// that share a weight tile run on one XCD -- and handed out in range order by a
// counter per XCD; a workgroup whose range is used up takes tiles from the other
// ranges (x + 1, x + 2, ...). Every tile runs its whole contraction: the results are
// those of the one-tile-per-workgroup kernel without a split, bit for bit, whichever
// workgroup computes a tile. The counters (q[0..7] per range, q[8] finished
// workgroups) are zero at launch -- callers clear them as they clear the split-tile
// counters -- and the last workgroup to finish sets them back to zero.
template <int EPI, int TM>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_nt_q(NtArgs a) {
  __shared__ uint4 smem[LDS_FWD_U4];
  const int ktiles = (a.K + TK - 1) / TK;
  const bool one_pass = a.E <= 64;
  TileScan64 sc{};
  if (one_pass) sc = tile_scan64<TM>(a.ends, a.E, a.m_cap, a.n_tiles);
  const int total = one_pass ? sc.total : tile_count<TM>(a.ends, a.E, a.m_cap, a.n_tiles);
  const int per = (total + 7) >> 3;
  const int x = (int)(blockIdx.x & 7);
  int* q = a.split_cnt;
  int* flag = reinterpret_cast<int*>(smem);
  for (;;) {
    // thread index through an opaque move per tile: address arithmetic derived from it
    // is redone per tile instead of being held across the loop
    int t = (int)threadIdx.x;
    asm volatile("" : "+v"(t));
    __syncthreads();   // the previous tile's epilogue has read LDS
    if (t == 0) {
      int tile = -1;
      for (int d = 0; d < 8 && tile < 0; ++d) {
        const int xx = (x + d) & 7;
        const int cnt = total - xx * per < per ? total - xx * per : per;
        if (cnt <= 0) continue;
        const int i = __hip_atomic_fetch_add(q + xx, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (i < cnt) tile = xx * per + i;
      }
      flag[0] = tile;
    }
    __syncthreads();
    const int tile = flag[0];
    __syncthreads();   // read by every wave before the tile's copies rewrite LDS
    if (tile < 0) break;
    int e, m0, mend, nt;
    if (one_pass)
      tile_locate64<TM>(sc, a.n_tiles, a.n_tiles, tile, e, m0, mend, nt);
    else
      tile_locate<TM>(a.ends, a.E, a.m_cap, a.n_tiles, tile, e, m0, mend, nt);
    nt_tile<EPI, true, TM>(a, smem, e, m0, mend, nt, 0, ktiles, 0, 1, 0, 0, t);
  }
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(q + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {   // every other workgroup has taken its last tile
#pragma unroll
      for (int i = 0; i < 9; ++i) __hip_atomic_store(q + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

template <int EPI, bool KFULL, int TM = TB>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_nt(NtArgs a) {
  static_assert(TM == TB || (TM == 128 && KFULL), "128-row tiles need whole 64-deep stages");
  // 160 KB: the five 32 KB slots of mainloop_fwd64, or the partial-K path's two stages
  __shared__ uint4 smem[LDS_FWD_U4];
  const int ktiles = (a.K + TK - 1) / TK;
  int e, m0, mend, nt, k0 = 0, nk = ktiles, part = 0, S = 1, slot = 0, cidx = 0;
  if (KFULL) {
    if (!deal_tile_split<TM>(a.ends, a.E, a.m_cap, a.n_tiles, a.n_res, ktiles, e, m0, mend, nt,
                             k0, nk, part, S, slot, cidx, a.mmajor))
      return;
  } else {
    if (!deal_tile<TB>(a.ends, a.E, a.m_cap, a.n_tiles, e, m0, mend, nt)) return;
  }
  nt_tile<EPI, KFULL, TM>(a, smem, e, m0, mend, nt, k0, nk, part, S, slot, cidx, (int)threadIdx.x);
}

// ---------------------------------------------------------------------------
// Epilogue staging of the backward products (LDS_U4 = 128 KB, free once every wave
// is past its main loop; callers barrier before and after). A lane holds 4 columns
// of one row per (i, q), so stores straight from registers would put 32 rows x 8 or
// 16 bytes in each instruction (32 partial cache lines); staged, the tile leaves in
// whole rows. Row R of the staged tile is 512 bytes whose 16-byte chunk c sits at
// chunk c ^ (R % 32), so the 32 rows of a write and the chunks of a read fall on
// distinct banks.
// The whole 256 x 256 tile as bf16 (chunk = 8 columns).
__device__ __forceinline__ void stage_tile_bf16(const f32x16 (&acc)[4][4], char* lds, int wn, int wm,
                                                int lane) {
  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = wm * 128 + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = wn * 128 + i * 32 + q * 8 + hi4;
        *reinterpret_cast<uint2*>(lds + R * 512 + ((((c >> 3) ^ (R & 31)) << 4) | (hi4 << 1))) =
            make_uint2(pack_bf16x2(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1]),
                       pack_bf16x2(acc[i][j][q * 4 + 2], acc[i][j][q * 4 + 3]));
      }
  }
}
// Tile columns [128 h, 128 h + 128) as fp32 (chunk = 4 columns); the two waves that
// hold them (wn == h) write.
__device__ __forceinline__ void stage_half_f32(const f32x16 (&acc)[4][4], char* lds, int h, int wn,
                                               int wm, int lane) {
  if (wn != h) return;
  const int hi4 = (lane >> 5) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int R = wm * 128 + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int c = i * 32 + q * 8 + hi4;
        *reinterpret_cast<float4*>(lds + R * 512 + (((c >> 2) ^ (R & 31)) << 4)) =
            make_float4(acc[i][j][q * 4 + 0], acc[i][j][q * 4 + 1], acc[i][j][q * 4 + 2],
                        acc[i][j][q * 4 + 3]);
      }
  }
}
// 16-byte chunk k (lane % 32) of staged row R (two rows per read: R = r0 + lane / 32)
__device__ __forceinline__ uint4 staged_chunk(const char* lds, int R, int k) {
  return *reinterpret_cast<const uint4*>(lds + R * 512 + ((k ^ (R & 31)) << 4));
}

// ---------------------------------------------------------------------------
// dgrad: dX[m, k] = sum_n G[m, n] W[e, n, k]. Weight side = k (read transposed
// from W rows n), activation side = G rows m, contraction n.
// ---------------------------------------------------------------------------
struct DgradArgs {
  const uint16_t* G; const uint16_t* W; const int32_t* ends; int E; int m_cap;
  int N; int K; int n_tiles; int m_tiles; uint16_t* DX;
  // activation backward (ACT > 0): DX is dh [rows][2K] = [du | dg], from the fp32
  // pre-activations h [rows][2K] = [u | g] and the clamp limits of SwiGLUStep
  const float* h; const float* limits; float def_limit;
  // optional split of the last round's tiles along N, as in the forward
  float* split_ws; int32_t* split_cnt; int n_res;
};

// dgrad: dX[m, k] = sum_n G[m, n] W[e, n, k]; ACT 0 stores dX, ACT 1 / 2 treat dX as
// da, the gradient of the SwiGLU / SwiGLUStep output, and store dh = act'(h) da.
template <int ACT>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_dgrad(DgradArgs a) {
  __shared__ uint4 smem[LDS_U4];
  // nt: tile of K (output columns); [k0, k0 + nk): this workgroup's 32-deep stages of N
  int e, m0, mend, nt, k0, nk, part, S, slot = 0, cidx = 0;
  if (!deal_tile_split(a.ends, a.E, a.m_cap, a.n_tiles, a.n_res, a.N / 32, e, m0, mend, nt, k0, nk,
                       part, S, slot, cidx))
    return;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int c0 = nt * TB;

  f32x16 acc[4][4];
  zero_acc(acc);
  // (the contraction N is a multiple of 32: whole 32-deep stages)
  KmSrc sw;   // weight side: W[e] rows n (contraction), columns k
  sw.base = reinterpret_cast<const char*>(a.W + ((int64_t)e * a.N + (int64_t)k0 * 32) * a.K + c0);
  sw.ld2 = 2 * (int64_t)a.K;
  sw.rows = nk * 32;
  sw.cols2 = 2 * (a.K - c0);
  sw.init(tid);
  RmSrc sg;   // activation side: G rows, contraction along N
  sg.base = a.G;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int p = m0 + (tid >> 2) + 64 * j;
    p = p < mend ? p : mend - 1;
    sg.off[j] = (uint32_t)p * (uint32_t)a.N;
  }
  sg.init(tid);
  mainloop_dma_g<true, false, 4>(sw, sg, smem, k0 * 32, nk, tid, lane, wn, wm, acc);
  if (S > 1 && !split_reduce(acc, a.split_ws, a.split_cnt, slot, part, S, cidx, smem, tid,
                             block_mask(m0 + wm * 128, mend, 4, c0 + wn * 128, a.K)))
    return;
  char* lds = reinterpret_cast<char*>(smem);
  const int rows = mend - m0 < TB ? mend - m0 : TB;
  const int k = lane & 31;
  if constexpr (ACT == 0) {
    __syncthreads();   // no wave still reads a stage or has a copy in flight
    stage_tile_bf16(acc, lds, wn, wm, lane);
    __syncthreads();
    const int col = c0 + k * 8;
    if (col < a.K) {
#pragma unroll 4
      for (int r0 = wid * 2; r0 < rows; r0 += 8) {
        const int R = r0 + (lane >> 5);
        if (R >= rows) continue;
        *reinterpret_cast<uint4*>(a.DX + (int64_t)(m0 + R) * a.K + col) = staged_chunk(lds, R, k);
      }
    }
  } else {
    // activation backward, one column half of the tile at a time: a lane takes 4
    // consecutive da of a row from LDS, loads the matching fp32 u and g (16 bytes each,
    // whole lines across the row's lanes) and writes du and dg
    float lim = 0.f;
    if (ACT == 2) lim = a.limits ? a.limits[e] : a.def_limit;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();   // the main loop's (or the previous half's) LDS reads are done
      stage_half_f32(acc, lds, h, wn, wm, lane);
      __syncthreads();
      const int col = c0 + h * 128 + k * 4;
      if (col < a.K) {
#pragma unroll 4
        for (int r0 = wid * 2; r0 < rows; r0 += 8) {
          const int R = r0 + (lane >> 5);
          if (R >= rows) continue;
          const int p = m0 + R;
          const uint4 dv = staged_chunk(lds, R, k);
          const float* hrow = a.h + (int64_t)p * 2 * a.K;
          const float4 u4 = *reinterpret_cast<const float4*>(hrow + col);
          const float4 g4 = *reinterpret_cast<const float4*>(hrow + a.K + col);
          const float das[4] = {__uint_as_float(dv.x), __uint_as_float(dv.y), __uint_as_float(dv.z),
                                __uint_as_float(dv.w)};
          const float us[4] = {u4.x, u4.y, u4.z, u4.w};
          const float gs[4] = {g4.x, g4.y, g4.z, g4.w};
          float du[4], dg[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float da = das[r];
            float u = us[r], g = gs[r];
            float mu = 1.f, mg = 1.f;
            if (ACT == 2) {   // the clamp passes the gradient where -L <= v <= L
              mu = (u >= -lim && u <= lim) ? 1.f : 0.f;
              mg = (g >= -lim && g <= lim) ? 1.f : 0.f;
              u = fminf(fmaxf(u, -lim), lim);
              g = fminf(fmaxf(g, -lim), lim);
            }
            const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
            du[r] = da * (g * sg) * mu;
            dg[r] = da * u * (sg * (1.0f + g * (1.0f - sg))) * mg;
          }
          uint16_t* crow = a.DX + (int64_t)p * 2 * a.K;
          *reinterpret_cast<uint2*>(crow + col) =
              make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
          *reinterpret_cast<uint2*>(crow + a.K + col) =
              make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// wgrad: dW[e, n, k] = sum over rows m of group e of G[m, n] X[m, k].
// Weight side = k (X read transposed), activation side = n (G read transposed),
// contraction over the group's rows, zero-filled past the group end.
// ---------------------------------------------------------------------------
struct WgradArgs {
  const uint16_t* G; const uint16_t* X; const int32_t* ends; int E; int m_cap;
  int N; int K; int n_tiles; int k_tiles; void* DW;
  int chunk;   // consecutive tiles an XCD takes at a time
};
constexpr int WG_KG = 8;       // k tiles per group in the blocked tile order

template <bool OUT_F32>
__global__ __launch_bounds__(NTHREADS, 1) void k_gemm_wgrad(WgradArgs a) {
  __shared__ uint4 smem[LDS_U4];
  // A tile's cost is its group's row count. Within a group the tiles are ordered in
  // groups of WG_KG k tiles: all n tiles of k tiles 0..7, then of 8..15, ..., so a run
  // of consecutive tiles is a compact block (4 n x 8 k for a chunk of 32) whose G and
  // X slices the XCD's L2 shares (a run of one n row would re-read every X slice for
  // each n). Chunks of a.chunk consecutive tiles go round-robin over the 8 XCDs, so
  // every XCD works through its share of each group at the same time: contiguous
  // ranges would hand whole groups to single XCDs, and the XCDs with small groups
  // would idle while the one with the largest group still takes new workgroups.
  const int x = (int)(blockIdx.x & 7), s = (int)(blockIdx.x >> 3);
  const int per_e = a.n_tiles * a.k_tiles;
  const int t = ((s / a.chunk) * 8 + x) * a.chunk + s % a.chunk;
  const int e = t / per_e;
  if (e >= a.E) return;
  const int rem = t - e * per_e;
  const int full_kg = a.k_tiles / WG_KG, per_full = a.n_tiles * WG_KG;
  int kg, kgs, q;
  if (rem < full_kg * per_full) {
    kg = rem / per_full;
    kgs = WG_KG;
    q = rem - kg * per_full;
  } else {   // the last, narrower group of k tiles
    kg = full_kg;
    kgs = a.k_tiles - full_kg * WG_KG;
    q = rem - full_kg * per_full;
  }
  const int ntile = q / kgs;   // rows n of dW
  const int ktile = kg * WG_KG + q % kgs;
  int start = 0;
  for (int g = 0; g < e; ++g) {
    int v = a.ends[g];
    v = v < start ? start : (v > a.m_cap ? a.m_cap : v);
    start = v;
  }
  int end = a.ends[e];
  end = end < start ? start : (end > a.m_cap ? a.m_cap : end);
  const int rows = end - start;
  const int n0 = ntile * TB, c0 = ktile * TB;

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;

  // both operands K-major (contraction = the group's rows); copies past the group's
  // last row or a matrix edge read as zeros
  KmSrc sx;   // weight side: output columns k from X rows
  sx.base = reinterpret_cast<const char*>(a.X + (int64_t)start * a.K + c0);
  sx.ld2 = 2 * (int64_t)a.K;
  sx.rows = rows;
  sx.cols2 = 2 * (a.K - c0);
  sx.init(tid);
  KmSrc sgd;  // activation side: output rows n from G rows
  sgd.base = reinterpret_cast<const char*>(a.G + (int64_t)start * a.N + n0);
  sgd.ld2 = 2 * (int64_t)a.N;
  sgd.rows = rows;
  sgd.cols2 = 2 * (a.N - n0);
  sgd.init(tid);

  f32x16 acc[4][4];
  zero_acc(acc);
  const int nsub = (rows + 31) / 32;
  if (nsub > 0) mainloop_dma_g<true, true, 4>(sx, sgd, smem, 0, nsub, tid, lane, wn, wm, acc);
  // staged through LDS (an empty group stages its zero tile like any other)
  char* lds = reinterpret_cast<char*>(smem);
  const int nrows = a.N - n0 < TB ? a.N - n0 : TB;
  const int k = lane & 31;
  if (OUT_F32) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      __syncthreads();
      stage_half_f32(acc, lds, h, wn, wm, lane);
      __syncthreads();
      const int col = c0 + h * 128 + k * 4;
      if (col < a.K) {
#pragma unroll 4
        for (int r0 = wid * 2; r0 < nrows; r0 += 8) {
          const int R = r0 + (lane >> 5);
          if (R >= nrows) continue;
          float* d = reinterpret_cast<float*>(a.DW) + ((int64_t)e * a.N + n0 + R) * a.K + col;
          *reinterpret_cast<uint4*>(d) = staged_chunk(lds, R, k);
        }
      }
    }
  } else {
    __syncthreads();
    stage_tile_bf16(acc, lds, wn, wm, lane);
    __syncthreads();
    const int col = c0 + k * 8;
    if (col < a.K) {
#pragma unroll 4
      for (int r0 = wid * 2; r0 < nrows; r0 += 8) {
        const int R = r0 + (lane >> 5);
        if (R >= nrows) continue;
        uint16_t* d = reinterpret_cast<uint16_t*>(a.DW) + ((int64_t)e * a.N + n0 + R) * a.K + col;
        *reinterpret_cast<uint4*>(d) = staged_chunk(lds, R, k);
      }
    }
  }
}

// Zero fill of n 16-byte words (graph-safe replacement for a memset node).
__global__ __launch_bounds__(256) void k_zero16(uint4* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

inline int round_up8(int64_t v) { return (int)((v + 7) / 8 * 8); }

}  // namespace

// Upper bound on the row blocks of ragged groups: sum_e ceil(m_e/256) <= floor(M/256) + E.
// Row blocks over E groups holding M rows in all: at most one partial block per
// non-empty group, and there are at most min(E, M) of those.
int row_block_bound(int64_t M, int E, int tm = TB) { return (int)(M / tm + (M < E ? M : E)); }

moe_status zero_fill(void* p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return MOE_OK;
  const int64_t n = (int64_t)(bytes / 16);
  const int blocks = (int)std::min<int64_t>((n + 255) / 256, 8192);
  k_zero16<<<blocks, 256, 0, st>>>(reinterpret_cast<uint4*>(p), n);
  return launch_status();
}

// C[rows, N] (bf16) = rows of A [*, K] times W[e]^T for ragged groups, with an epilogue.
// tm: activation rows per tile, 256 or 128 (128 only when K is a multiple of 64;
// otherwise 256 is used)
moe_status gemm_nt_enqueue(int epi, const void* A, const int32_t* a_gather, int a_div,
                           const void* B, int NB, int E, const int32_t* ends, int64_t M, int N,
                           int K, void* C, int64_t ldc, int I, const float* limits,
                           float def_limit, const float* route_w, const int32_t* p2e, int top_k,
                           hipStream_t st, void* split_ws, int32_t* split_cnt, void* h_out,
                           int tm, int rows_hint) {
  if (M == 0) return MOE_OK;
  NtArgs a;
  a.A = reinterpret_cast<const uint16_t*>(A);
  a.a_gather = a_gather;
  a.a_div = a_div > 0 ? a_div : 1;
  a.B = reinterpret_cast<const uint16_t*>(B);
  a.b_stride = (int64_t)NB * K;
  a.ends = ends;
  a.E = E;
  a.m_cap = (int)M;
  a.NB = NB;
  a.N = N;
  a.K = K;
  const bool fc1 = (epi == EPI_SWIGLU || epi == EPI_SWIGLU_STEP);
  a.n_tiles = fc1 ? (I + 127) / 128 : (N + TB - 1) / TB;
  const bool kfull = (K % TK) == 0;
  if (tm != 128 || !kfull) tm = TB;
  a.m_tiles = row_block_bound(M, E, tm);
  a.C = reinterpret_cast<uint16_t*>(C);
  a.ldc = ldc;
  a.I = I;
  a.limits = limits;
  a.def_limit = def_limit;
  a.route_w = route_w;
  a.p2e = p2e;
  a.top_k = top_k;
  a.h_out = reinterpret_cast<float*>(h_out);
  a.split_ws = reinterpret_cast<float*>(split_ws);
  a.split_cnt = split_cnt;
  a.n_res = 0;
  // SM90 fused-MoE page, Parameters (gemm2_raster_along_m): the fused finalize deals its
  // tiles column tile first when the output it scatters into is large and the
  // contraction short -- at least 32 MiB for I <= 192, 64 MiB for I <= 384 -- so that
  // the workgroups in flight add into one band of output columns. At the layer shapes
  // here (I >= 2048) the rule never applies; at the Mixtral shape dealing column tile
  // first measured the same as group first (1.27 vs 1.26 ms).
  const size_t out_bytes = (size_t)(M / (top_k > 0 ? top_k : 1)) * N * 2;
  a.mmajor = epi == EPI_FUSED && ((K <= 192 && out_bytes >= (32u << 20)) ||
                                  (K <= 384 && out_bytes >= (64u << 20)));
  if (split_ws && split_cnt && kfull) {
    const int cu = device_cu_count();
    a.n_res = (cu < SPLIT_SLOTS ? cu : SPLIT_SLOTS) & ~7;  // one 128 KB-LDS workgroup per CU
  }
  const int64_t tiles = (int64_t)a.m_tiles * a.n_tiles;
  // parts of split tiles take at most n_res + 8 * SPLIT_MAX workgroups past the whole ones
  int grid = round_up8(tiles + (a.n_res > 0 ? a.n_res + 8 * SPLIT_MAX : 0));
  // few rows per group (the caller's estimate): the work-queue kernel, one workgroup
  // per CU, whole contractions (no split), counters in the split-tile counter area
  const bool queue = kfull && tm == TB && split_cnt && rows_hint > 0 && rows_hint <= QUEUE_ROWS &&
                     E >= QUEUE_GROUPS &&
                     (epi == EPI_STORE || epi == EPI_SWIGLU || epi == EPI_SWIGLU_STEP ||
                      epi == EPI_FUSED);
  if (queue) {
    a.n_res = 0;
    const int pers = std::max(8, device_cu_count() & ~7);
    grid = grid < pers ? grid : pers;
  }
#define MOE_LAUNCH_NT(E_)                                                  \
  (tm == 128 ? k_gemm_nt<E_, true, 128><<<grid, NTHREADS, 0, st>>>(a)      \
   : kfull   ? k_gemm_nt<E_, true><<<grid, NTHREADS, 0, st>>>(a)           \
             : k_gemm_nt<E_, false><<<grid, NTHREADS, 0, st>>>(a))
#define MOE_LAUNCH_NTQ(E_)                                                                     \
  (queue ? k_gemm_nt_q<E_, TB><<<grid, NTHREADS, 0, st>>>(a) : MOE_LAUNCH_NT(E_))
  switch (epi) {
    case EPI_STORE: MOE_LAUNCH_NTQ(EPI_STORE); break;
    case EPI_SWIGLU: MOE_LAUNCH_NTQ(EPI_SWIGLU); break;
    case EPI_SWIGLU_STEP: MOE_LAUNCH_NTQ(EPI_SWIGLU_STEP); break;
    case EPI_FUSED: MOE_LAUNCH_NTQ(EPI_FUSED); break;
    default: return MOE_ERR_DTYPE;
  }
#undef MOE_LAUNCH_NTQ
#undef MOE_LAUNCH_NT
  return launch_status();
}

// act: 0 plain dgrad into DX [M, K]; 1 / 2 (SwiGLU / SwiGLUStep backward): DX is dh
// [M, 2K] and h [M, 2K] the saved fp32 pre-activations.
moe_status gemm_dgrad_enqueue(const void* G, const void* W, const int32_t* ends, int E, int64_t M,
                              int N, int K, void* DX, hipStream_t st, int act, const void* h,
                              const float* limits, float def_limit, void* split_ws,
                              int32_t* split_cnt) {
  if (M == 0) return MOE_OK;
  DgradArgs a{reinterpret_cast<const uint16_t*>(G), reinterpret_cast<const uint16_t*>(W), ends, E,
              (int)M, N, K, (K + TB - 1) / TB, row_block_bound(M, E),
              reinterpret_cast<uint16_t*>(DX), reinterpret_cast<const float*>(h), limits,
              def_limit, reinterpret_cast<float*>(split_ws), split_cnt, 0};
  if (split_ws && split_cnt) {
    const int cu = device_cu_count();
    a.n_res = (cu < SPLIT_SLOTS ? cu : SPLIT_SLOTS) & ~7;  // one 128 KB-LDS workgroup per CU
  }
  // parts of split tiles take at most n_res + 8 * SPLIT_MAX workgroups past the whole ones
  const int grid = round_up8((int64_t)a.m_tiles * a.n_tiles +
                             (a.n_res > 0 ? a.n_res + 8 * SPLIT_MAX : 0));
  if (act == 1)
    k_gemm_dgrad<1><<<grid, NTHREADS, 0, st>>>(a);
  else if (act == 2)
    k_gemm_dgrad<2><<<grid, NTHREADS, 0, st>>>(a);
  else
    k_gemm_dgrad<0><<<grid, NTHREADS, 0, st>>>(a);
  return launch_status();
}

moe_status gemm_wgrad_enqueue(const void* G, const void* X, const int32_t* ends, int E, int64_t M,
                              int N, int K, void* DW, bool out_f32, hipStream_t st) {
  WgradArgs a{reinterpret_cast<const uint16_t*>(G), reinterpret_cast<const uint16_t*>(X), ends, E,
              (int)M, N, K, (N + TB - 1) / TB, (K + TB - 1) / TB, DW, 0};
  // chunks of up to 32 tiles, but at least 8 chunks per group so that every XCD takes
  // a share of every group (group sizes differ: a group's tiles cost its row count)
  const int per_e = a.n_tiles * a.k_tiles;
  a.chunk = std::max(1, std::min(32, per_e / 8));
  // every XCD holds ceil(chunks / 8) chunks; the excess exits
  const int64_t chunks = ((int64_t)E * per_e + a.chunk - 1) / a.chunk;
  const int grid = (int)(8 * ((chunks + 7) / 8) * a.chunk);
  if (out_f32)
    k_gemm_wgrad<true><<<grid, NTHREADS, 0, st>>>(a);
  else
    k_gemm_wgrad<false><<<grid, NTHREADS, 0, st>>>(a);
  return launch_status();
}

}  // namespace moe
