// fp8-activation grouped GEMMs on gfx950 scaled MFMA: FC1 with the activation and
// the fp8 requantization in its epilogue, FC2 to bf16 rows. Three weight families:
//   MXFP4  e2m1 pairs, one UE8M0 scale per 32 values along the contraction;
//   MXFP8  e4m3 bytes, same scales (activations MXFP8 in both MX families);
//   FP8    e4m3 bytes with one fp32 scale per expert matrix, activations e4m3 with
//          one fp32 scale for the tensor (StepFun page, intro: the per-tensor fp8 weight family).
//          The MFMA runs with unit block scales and the per-tensor factors are
//          applied in the epilogue; the FC1 output is requantized with a given
//          per-tensor scale, saturating at +-448.
//
// W4A8 page ("flashinfer.fused_moe.cake / cake_cute (MXFP4 SiTU routed MoE)"),
// Host plan, Inputs: activations are float8_e4m3fn with one UE8M0 scale per 32 values
// along H; the expert bank is MXFP4 (two e2m1 values per byte) with UE8M0
// block-32 scales, w1 holding the up rows then the gate rows. Intro: fp32
// accumulation, and the FC1 output requantized with UE8M0 scales rounded up
// before FC2.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 contract (checked on the device with exact
// small-integer operands): with the e2m1 operand in the A slot, lane l supplies
// row l%32, k = 32*(l/32) + e as nibble e (low nibble first) of 4 VGPRs; the
// e4m3 operand in the B slot supplies column l%32 with bytes 0..15 at
// k = 16*(l/32) + b and bytes 16..31 at k = 32 + 16*(l/32) + (b-16); the UE8M0
// scale of 32-block kb of a row/column comes from byte 0 of the scale VGPR of
// lane (row + 32*kb); D uses the usual 32x32 layout. An e4m3 operand in the A slot
// (cbsz=0, MXFP8 weights) packs its bytes exactly as in the B slot.
//
// Tile: 256 weight rows x 256 activation rows, 4 waves of 128 x 128 (4 x 4
// accumulators), weights as the A operand so a lane holds 4 consecutive output
// columns; a tile that holds fewer rows (a small expert, an expert's tail) copies
// and multiplies only its 32-row blocks that hold rows. Operands are copied straight from global memory into LDS, several stages
// ahead. MXFP4: 128-deep stages of activation codes [256][8 x 16 B], weight codes
// [256][4 x 16 B] and both operands' 4 scale bytes per row (50 KB), three slots.
// MXFP8 / FP8: 64-deep stages of activation and weight codes [256][4 x 16 B] each
// (plus the scale words for MXFP8), four slots. Tiles are dealt out as in the bf16
// kernels (device-counted, XCD-balanced, expert-major).
#include <type_traits>

#include "common.h"

namespace moe {
// recorded tile choices (tune.hip): 1 streaming, 0 256-row, -1 none
int tune_lookup(int stage, int wf, int K, int NB, int L, int64_t R);

namespace {

constexpr int MTB = 256;          // tile rows on each side
constexpr int MTK = 128;          // contraction per stage
constexpr int MNT = 256;          // threads
// activation codes of a 128-deep MXFP4 stage of a tile with JV 32-row blocks per
// row-wave (64 JV rows), in uint4
template <int JV> constexpr int xt_u4() { return JV * 64 * MTK / 16; }

// Weight formats (the order of MOE_WFMT_MXFP4, MOE_WFMT_MXFP8, MOE_WFMT_FP8 minus 1).
constexpr int WF_MXFP4 = 0, WF_MXFP8 = 1, WF_FP8 = 2;
template <int WF> constexpr int wbits() { return WF == WF_MXFP4 ? 4 : 8; }
template <int WF> constexpr bool block_scaled() { return WF != WF_FP8; }
// 16-byte chunks per weight row and stage, and the stage size in uint4
template <int WF> constexpr int wch() { return MTK * wbits<WF>() / 8 / 16; }
// SG: the block scales come in groups of four stages (16 bytes per row, their own
// two-group LDS ring of 16 KB) instead of one 4-byte word per row and stage
template <int WF, int JV, bool SG = false> constexpr int stage_u4() {
  return xt_u4<JV>() + MTB * wch<WF>() + (block_scaled<WF>() && !SG ? 2 * MTB / 4 : 0);
}
constexpr int MX_SG_U4 = 2 * 2 * MTB;   // two groups of x and w scales, [256][16 B] each
// scaled-MFMA format code of the weight (A-slot) operand
template <int WF> constexpr int a_fmt() { return WF == WF_MXFP4 ? 4 : 0; }
constexpr int UNIT_SCALE = 127;              // UE8M0 code of 1.0
constexpr uint32_t UNIT_SCALE4 = 0x7F7F7F7Fu;

enum MxEpi { MX_FC1_SWIGLU = 0, MX_FC1_STEP = 1, MX_FC2 = 2 };

typedef int v8i __attribute__((ext_vector_type(8)));

// Direct-to-LDS copies (MXFP4 256-row kernel): lane l's 16 (4) bytes from g land at
// LDS byte address lds + 16 l (4 l). The compiler does not see these LDS writes; the
// loop counts the copies in flight itself (vmcnt) before each barrier.
__device__ __forceinline__ void mx_dma16(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void mx_dma4(const void* g, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// MXFP4 stages in LDS: three slots (up to 150 KB) two stages ahead, or four slots
// three stages ahead when the tile has at most 128 activation rows (34 KB a stage)
template <int JV> constexpr int mx_dma_slots() { return JV <= 2 ? 4 : 3; }
// 8-bit weight families: four slots of 64-deep stages (activation codes 64 JV x 64 B,
// weight codes 16 KB, then both operands' scale words for MXFP8), copies three
// stages ahead
constexpr int MX8_SLOTS = 4;
template <int WF, int JV, bool SG = false> constexpr int mx8_stage_u4() {
  return JV * 256 + 1024 + (WF == 2 || SG ? 0 : 2 * 64);
}
// LDS of the 256-row kernel: the largest layout over JV = 1..4
constexpr int mx_lds_u4_max(int wf) {
  return wf == 0 ? 3 * (4 * 512 + 1024) + MX_SG_U4 : MX8_SLOTS * (4 * 256 + 1024) + MX_SG_U4;
}

struct MxArgs {
  const uint8_t* A;        // activation codes [rows][K]
  const uint8_t* A_sf;     // [rows][K/32]
  const int32_t* a_gather; // optional: row p reads A row a_gather[p] / a_div
  int a_div;
  const uint8_t* B;        // weight codes [E][NB][K/2] (MXFP4) or [E][NB][K] (MXFP8)
  const uint8_t* B_sf;     // [E][NB][K/32]
  const int32_t* ends;
  int E, m_cap, NB, N, K, n_tiles;
  uint16_t* C;             // FC2: bf16 rows [rows][ldc]
  int64_t ldc;
  int32_t* qcnt;           // work-queue counters [9], zero at launch, or NULL (no queue)
  uint8_t* Cq;             // FC1: e4m3 act [rows][I]
  uint8_t* Cq_sf;          // FC1: [rows][I/32] (MX families)
  int I;
  const float* limits;
  float def_limit;
  // FP8 family: A-operand tensor scale [1], weight scales [E], FC1 output scale [1]
  const float* a_scale;
  const float* w_scale;
  const float* q_scale;
};

// Per-tensor factor of an output element (FP8 family): a_scale * w_scale[e].
template <int WF>
__device__ __forceinline__ float pt_alpha(const MxArgs& a, int e) {
  return block_scaled<WF>() ? 1.f : a.a_scale[0] * a.w_scale[e];
}

// e4m3 code input of a requantized FC1 value v * inv: the MX families' block scale
// keeps it within +-448 by construction; the per-tensor scale may not, so it saturates.
template <int WF>
__device__ __forceinline__ float q_in(float v, float inv) {
  const float y = v * inv;
  return block_scaled<WF>() ? y : fminf(fmaxf(y, -448.f), 448.f);
}

// Round-up UE8M0 code of a block maximum: the smallest e with amax <= 448 * 2^e,
// as e + 127. With amax = (1+f) * 2^E, 448 = 1.75 * 2^8: e = E - 8 when
// 1+f <= 1.75, else E - 7. An all-zero block takes code 0.
__device__ __forceinline__ uint32_t ue8m0_round_up_448(float amax) {
  const uint32_t bits = __float_as_uint(amax);
  const int ex = (int)((bits >> 23) & 0xFF);
  if (amax == 0.f) return 0u;
  int c = ex - 8 + ((bits & 0x7FFFFF) > 0x600000 ? 1 : 0);
  c = c < 0 ? 0 : (c > 253 ? 253 : c);
  return (uint32_t)c;
}

// Issue order for the scheduler: NM MFMAs (group 0x008), each followed by its even
// share of NR LDS reads (group 0x100).
template <int NM, int NR>
__device__ __forceinline__ void sched_mfma_reads() {
  static_assert(NR <= 5 * NM, "at most five reads per MFMA");
#pragma unroll
  for (int r = 0; r < NM; ++r) {
    const int c = ((r + 1) * NR) / NM - (r * NR) / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (c > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (c > 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (c > 2) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (c > 3) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (c > 4) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// One tile of up to 256 activation rows, of which the first 64 JV exist: the
// activation rows come in 32-row blocks, block b = 2 j + wm going to row-wave wm
// (j < JV), so the two row-waves share the tile's rows evenly and a tile holding the
// few rows of a small expert, or an expert's tail, copies and multiplies only
// those (JV = 4: the whole 256-row tile). Every output element takes the same MFMA
// sequence whatever JV is.
template <int EPI, int WF, int JV, bool SG>
__device__ __forceinline__ void mx_tile(const MxArgs& a, uint4* smem, int e, int m0, int mend,
                                        int nt, int t) {
  static_assert(!SG || block_scaled<WF>(), "scale groups: block-scaled weights only");
  constexpr int WB = wbits<WF>();
  constexpr bool BS = block_scaled<WF>();
  constexpr int JN = JV;             // 32-row activation blocks per wave
  constexpr int XROWS = 64 * JV;     // activation rows copied
  constexpr int XT_U4 = xt_u4<JV>();
  constexpr int WCH = wch<WF>(), WT_U4 = MTB * WCH, STAGE_U4 = stage_u4<WF, JV, SG>();
  constexpr int WLD = WT_U4 / MNT;   // weight loads per thread and stage (4 or 8)
  constexpr int NSLOT = mx_dma_slots<JV>();
  static_assert((WF == WF_MXFP4 ? NSLOT * STAGE_U4 : MX8_SLOTS * mx8_stage_u4<WF, JV, SG>()) +
                        (SG ? MX_SG_U4 : 0) <=
                    mx_lds_u4_max(WF == WF_MXFP4 ? 0 : 1),
                "stage layout exceeds the kernel's LDS");
  const int tid = t, lane = tid & 63, wid = tid >> 6;
  const int wn = wid & 1, wm = wid >> 1;
  const int rsel = lane & 31, g = lane >> 5;
  const int K = a.K, ks = K >> 5;   // bytes per scale row
  const bool fc1 = EPI != MX_FC2;

  // per-thread source rows: activation codes rows (tid>>3)+32j, weight codes rows
  // tid/WCH + (256/WCH)j (the MXFP4 copies use these rows), scales: row tid of each
  // operand (activation rows taken modulo XROWS)
  const int xr = tid >> 3, xc = tid & 7, wr = tid / WCH, wc = tid % WCH;
  const uint32_t kw = (uint32_t)K * WB / 8;   // weight bytes per row
  uint32_t xoff[XROWS / 32], woff[WLD];
  // source rows, gathered together: the MXFP4 copy rows xr + 32 j, the 8-bit copy
  // rows (tid >> 2) + 64 j, and the scale row tid % XROWS
  constexpr int NXR = WF == WF_MXFP4 ? XROWS / 32 : JV;
  int src[NXR + 1];
#pragma unroll
  for (int j = 0; j < NXR; ++j) {
    const int p = m0 + (WF == WF_MXFP4 ? xr + 32 * j : (tid >> 2) + 64 * j);
    src[j] = p < mend ? p : mend - 1;
  }
  {
    const int p = m0 + tid % XROWS;
    src[NXR] = p < mend ? p : mend - 1;
  }
  gather_rows(a.a_gather, a.a_div, src);
  if constexpr (WF == WF_MXFP4) {
#pragma unroll
    for (int j = 0; j < XROWS / 32; ++j) xoff[j] = (uint32_t)src[j] * (uint32_t)K + xc * 16;
  }
  auto wrow_of = [&](int R) {
    if (fc1) {
      int c = nt * 128 + (R >> 7) * 64 + (R & 63);
      c = c < a.I ? c : a.I - 1;
      return ((R >> 6) & 1) * a.I + c;
    }
    const int r = nt * MTB + R;
    return r < a.NB ? r : a.NB - 1;
  };
  const uint8_t* Bb = a.B + (int64_t)e * a.NB * kw;
  const uint8_t* Bs = a.B_sf + (int64_t)e * a.NB * ks;
#pragma unroll
  for (int j = 0; j < WLD; ++j) woff[j] = (uint32_t)wrow_of(wr + (MTB / WLD) * j) * kw + wc * 16;
  uint32_t xsoff, wsoff;
  xsoff = (uint32_t)src[NXR] * (uint32_t)ks;
  wsoff = (uint32_t)wrow_of(tid) * (uint32_t)ks;
  f32x16 acc[4][JN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int ktiles = K / MTK;
  if constexpr (WF == WF_MXFP4) {
    // MXFP4: stages copied straight into LDS, NSLOT slots, NSLOT - 1 stages ahead.
    // Copy j of wave w: activation rows 32 j + 8 w + lane / 8 (whole 128-byte rows,
    // global chunk (lane % 8) ^ ((row / 2) % 8)); weight rows 64 j + 16 w + lane / 4
    // (64-byte rows, chunk (lane % 4) ^ ((row / 4) % 4)); scale words of rows
    // 64 w + lane (activation rows modulo XROWS). These are the layouts the fragment
    // reads below expect. The loop is rotated by one step: a stage's second step runs
    // after the barrier, under the first fragment reads of the next stage.
    // SG: no scale words in the stages; instead, with the copies of every fourth stage
    // 4g, each wave first copies 16 bytes of scales (stages 4g .. 4g+3) for its 64
    // activation and 64 weight rows into group buffer g % 2 ([256 rows][16 B] each of
    // x and w). Those two copies precede the stage's own, so a barrier that has seen a
    // stage's copies land has seen its scale group land too.
    constexpr int XC = XROWS / 32;              // activation-row copies per wave and stage
    constexpr int NC = XC + (SG ? 4 : 6);    // + 4 weight-row copies (+ 2 scale words)
    constexpr int NC2 = NC / 2;              // issued with each step's fragment reads
    // copies allowed in flight at a barrier: the younger stages' (a scale group issued
    // with them is waited for as well, which costs little: it was issued first)
    constexpr int NWAIT = (NSLOT - 2) * NC;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem + (uint32_t)w * 1024u;
    const uint32_t lds0s = (uint32_t)(uintptr_t)smem + (uint32_t)w * 256u;
    constexpr uint32_t XT_B = XT_U4 * 16, WT_B = WT_U4 * 16, STAGE_B = STAGE_U4 * 16;
    constexpr uint32_t SG_B = NSLOT * STAGE_B;   // scale-group ring (SG)
    const int gx = (lane & 7) ^ ((4 * w + (lane >> 4)) & 7);
    const int gw = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t xrow[XC], wrowb[4];
#pragma unroll
    for (int j = 0; j < XC; ++j) xrow[j] = xoff[j] - xc * 16;
#pragma unroll
    for (int j = 0; j < 4; ++j) wrowb[j] = woff[j] - wc * 16;
    // copy c (0..NC-1) of stage q into the slot at byte offset d: XC activation-row
    // copies, 4 weight-row copies, then the two scale words
    auto cp = [&](int c, int q, uint32_t d) {
      if (c < XC) {
        mx_dma16(a.A + xrow[c] + q * MTK + gx * 16, lds0 + d + c * 4096u);
      } else if (c < XC + 4) {
        mx_dma16(Bb + wrowb[c - XC] + q * (MTK / 2) + gw * 16, lds0 + d + XT_B + (c - XC) * 4096u);
      } else if (c == XC + 4) {
        mx_dma4(a.A_sf + xsoff + q * (MTK / 32), lds0s + d + XT_B + WT_B);
      } else {
        mx_dma4(Bs + wsoff + q * (MTK / 32), lds0s + d + XT_B + WT_B + 1024u);
      }
    };
    // SG: the scale group of stage q (a multiple of 4) into buffer (q / 4) % 2
    auto cp_group = [&](int q) {
      const uint32_t gb = SG_B + (uint32_t)((q >> 2) & 1) * 8192u + (uint32_t)w * 1024u;
      mx_dma16(a.A_sf + xsoff + q * (MTK / 32), (uint32_t)(uintptr_t)smem + gb);
      mx_dma16(Bs + wsoff + q * (MTK / 32), (uint32_t)(uintptr_t)smem + gb + 4096u);
    };
    v8i wf[2][4], xf[2][JN];
    // scale words of the current stage and of the previous one (whose second step
    // runs at the start of the current stage)
    uint32_t wsr[4], xsr[JN], wsp[4], xsp[JN];
    auto rd_scales = [&](int slot, int st) {
      if (SG) {
        const uint32_t* XS = reinterpret_cast<const uint32_t*>(smem + SG_B / 16 + ((st >> 2) & 1) * 512);
        const uint32_t* WS = XS + 4 * MTB;
        const int ph = st & 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) wsr[i] = WS[(wn * 128 + i * 32 + rsel) * 4 + ph];
#pragma unroll
        for (int j = 0; j < JN; ++j) xsr[j] = XS[((2 * j + wm) * 32 + rsel) * 4 + ph];
      } else {
        const uint32_t* XS = reinterpret_cast<const uint32_t*>(smem + slot * STAGE_U4 + XT_U4 + WT_U4);
        const uint32_t* WS = XS + MTB;
#pragma unroll
        for (int i = 0; i < 4; ++i) wsr[i] = WS[wn * 128 + i * 32 + rsel];
#pragma unroll
        for (int j = 0; j < JN; ++j) xsr[j] = XS[(2 * j + wm) * 32 + rsel];
      }
    };
    // fragment reads of step kk of `slot` (4 weight, 2 JN activation), copies
    // c0..c0+NC2-1 of stage q into slot offset d among them
    auto rd_issue = [&](int slot, int kk, int set, int q, uint32_t d, int c0) {
      const uint4* X = smem + slot * STAGE_U4;
      const uint4* W = X + XT_U4;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wn * 128 + i * 32 + rsel;
        const uint4 v = W[r * 4 + ((2 * kk + g) ^ ((r >> 2) & 3))];
        wf[set][i] = v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        if (i < NC2) cp(c0 + i, q, d);
      }
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int r = (2 * j + wm) * 32 + rsel;
        const uint4 lo = X[r * 8 + ((4 * kk + g) ^ ((r >> 1) & 7))];
        if (j < NC2 - 4) cp(c0 + 4 + j, q, d);
        const uint4 hi = X[r * 8 + ((4 * kk + 2 + g) ^ ((r >> 1) & 7))];
        xf[set][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
    };
    auto mm = [&](int set, int kk, const uint32_t (&ws)[4], const uint32_t (&xs)[JN]) {
      const int sh = 8 * (2 * kk + g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf[set][i], xf[set][j], acc[i][j], a_fmt<WF>(), 0, 0, (int)((ws[i] >> sh) & 0xFF), 0,
              (int)((xs[j] >> sh) & 0xFF));
    };
    auto body = [&](int st, bool first) {
      const int slot = st % NSLOT;
      const int q = st + NSLOT - 1 < ktiles ? st + NSLOT - 1 : ktiles - 1;
      const uint32_t d = (uint32_t)((st + NSLOT - 1) % NSLOT) * STAGE_B;
      if (SG && ((st + NSLOT - 1) & 3) == 0 && st + NSLOT - 1 < ktiles) cp_group(q);
      rd_scales(slot, st);
      rd_issue(slot, 0, 0, q, d, 0);
      if (!first) mm(1, 1, wsp, xsp);   // the previous stage's second step
      rd_issue(slot, 1, 1, q, d, NC2);
      mm(0, 0, wsr, xsr);
#pragma unroll
      for (int i = 0; i < 4; ++i) wsp[i] = wsr[i];
#pragma unroll
      for (int j = 0; j < JN; ++j) xsp[j] = xsr[j];
      // issue order (0x008 MFMA, 0x100 LDS read): the 4 + JN scale reads and step 0's
      // 4 + 2 JN fragment reads, then step 1's between step 0's 4 JN MFMAs
      // (non-first: the former between the previous stage's last step)
      if (first) {
        __builtin_amdgcn_sched_group_barrier(0x100, 8 + 3 * JN, 0);
      } else if (JV == 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (r & 3) {} else __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        sched_mfma_reads<4 * JN, 8 + 3 * JN>();
      }
      if (JV == 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (r < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        sched_mfma_reads<4 * JN, 4 + 2 * JN>();
      }
      __builtin_amdgcn_sched_barrier(0);
      // copies complete in issue order: the younger stages' may still be in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NWAIT) : "memory");
      __syncthreads();
    };
#pragma unroll
    for (int q = 0; q < NSLOT - 1; ++q) {
      if (SG && (q & 3) == 0 && q < ktiles) cp_group(q);
#pragma unroll
      for (int c = 0; c < NC; ++c) cp(c, q < ktiles ? q : ktiles - 1, (uint32_t)q * STAGE_B);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NWAIT) : "memory");
    __syncthreads();
    body(0, true);
    for (int st = 1; st < ktiles; ++st) body(st, false);
    mm(1, 1, wsp, xsp);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else {
    // MXFP8 / FP8: 64-deep stages copied straight into LDS, MX8_SLOTS slots, three
    // stages ahead; each stage is one scaled-MFMA step. Copy j of wave w covers rows
    // 64 j + 16 w + lane / 4 of the activation (j < XROWS / 64) and of the weight codes
    // (64-byte rows, global chunk (lane % 4) ^ ((row / 4) % 4)); MXFP8 also copies the
    // scale word of the stage's 128-deep block for rows 64 w + lane. Loop rotated by
    // one step: the previous stage's MFMAs run under the current stage's fragment reads.
    // SG (MXFP8, K a multiple of 512): no words in the stages; with the copies of every
    // eighth stage 8g each wave first copies 16 bytes of scales (the four words of
    // stages 8g .. 8g+7) for its 64 activation and 64 weight rows into group buffer
    // g % 2, as in the MXFP4 loop.
    constexpr int XC8 = XROWS / 64;   // activation copies per wave and stage
    constexpr uint32_t XCODE_B = XROWS * 64, WCODE_B = 16384,
                       SLOT_B = mx8_stage_u4<WF, JV, SG>() * 16;
    constexpr uint32_t SG_B = MX8_SLOTS * SLOT_B;   // scale-group ring (SG)
    // Copies per wave: XC8 + 4 code copies per stage, plus (MXFP8) the 2 scale words
    // for even stages only -- both stages of a 128-deep block use the even one's words.
    // An odd-parity body issues an even stage (or, clamped at the end, a copy nobody
    // reads) and copies the words; an even-parity body does not. Any two consecutive
    // bodies therefore have NWAIT copies in flight at a barrier.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint32_t lds0 = (uint32_t)(uintptr_t)smem + (uint32_t)w * 1024u;
    const uint32_t lds0s = (uint32_t)(uintptr_t)smem + (uint32_t)w * 256u;
    const int gc = (lane & 3) ^ ((lane >> 4) & 3);
    uint32_t xrow[XC8], wrow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int R = (tid >> 2) + 64 * j;
      if (j < XC8) xrow[j] = (uint32_t)src[j] * (uint32_t)K + gc * 16;
      wrow[j] = (uint32_t)wrow_of(R) * kw + gc * 16;
    }
    const int nsub = K / 64;
    auto cp = [&](int c, int q, uint32_t d) {
      if (c < XC8) {
        mx_dma16(a.A + xrow[c] + q * 64, lds0 + d + c * 4096u);
      } else if (c < XC8 + 4) {
        mx_dma16(Bb + wrow[c - XC8] + q * 64, lds0 + d + XCODE_B + (c - XC8) * 4096u);
      } else if (c == XC8 + 4) {
        mx_dma4(a.A_sf + xsoff + (q >> 1) * 4, lds0s + d + XCODE_B + WCODE_B);
      } else {
        mx_dma4(Bs + wsoff + (q >> 1) * 4, lds0s + d + XCODE_B + WCODE_B + 1024u);
      }
    };
    // SG: the scale group of stage q (a multiple of 8) into buffer (q / 8) % 2
    auto cp_group = [&](int q) {
      const uint32_t gb = SG_B + (uint32_t)((q >> 3) & 1) * 8192u + (uint32_t)w * 1024u;
      mx_dma16(a.A_sf + xsoff + (q >> 1) * 4, (uint32_t)(uintptr_t)smem + gb);
      mx_dma16(Bs + wsoff + (q >> 1) * 4, (uint32_t)(uintptr_t)smem + gb + 4096u);
    };
    v8i wf[2][4], xf[2][JN];
    uint32_t wsr[4], xsr[JN], wsp[4], xsp[JN];
#pragma unroll
    for (int i = 0; i < 4; ++i) wsr[i] = wsp[i] = UNIT_SCALE4;
#pragma unroll
    for (int j = 0; j < JN; ++j) xsr[j] = xsp[j] = UNIT_SCALE4;
    // SG: a scale group issued with the younger stages is waited for as well (it was
    // issued first, so this costs little)
    constexpr int NWAIT = 2 * (XC8 + 4) + (BS && !SG ? 2 : 0);
    // fragment reads of stage st in `slot` (two 16-byte chunks per fragment), with
    // the copies of stage q into slot offset d spread among them
    auto rd_issue = [&](int slot, int st, int set, int q, uint32_t d) {
      const uint4* X = smem + slot * mx8_stage_u4<WF, JV, SG>();
      const uint4* W = X + XROWS * 4;
      // the two stages of a 128-deep block share their scale words: the odd stage
      // keeps the even one's in registers
      if (BS && set == 0) {
        const uint32_t* XS;
        int ws_off, stride, ph;
        if (SG) {
          XS = reinterpret_cast<const uint32_t*>(smem + SG_B / 16 + ((st >> 3) & 1) * 512);
          ws_off = 4 * MTB;
          stride = 4;
          ph = (st >> 1) & 3;
        } else {
          XS = reinterpret_cast<const uint32_t*>(W + 1024);
          ws_off = MTB;
          stride = 1;
          ph = 0;
        }
        const uint32_t* WS = XS + ws_off;
#pragma unroll
        for (int i = 0; i < 4; ++i) wsr[i] = WS[(wn * 128 + i * 32 + rsel) * stride + ph];
#pragma unroll
        for (int j = 0; j < JN; ++j) xsr[j] = XS[((2 * j + wm) * 32 + rsel) * stride + ph];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wn * 128 + i * 32 + rsel;
        const uint4 lo = W[r * 4 + (g ^ ((r >> 2) & 3))];
        const uint4 hi = W[r * 4 + ((2 + g) ^ ((r >> 2) & 3))];
        wf[set][i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        cp(i, q, d);
      }
#pragma unroll
      for (int j = 0; j < JN; ++j) {
        const int r = (2 * j + wm) * 32 + rsel;
        const uint4 lo = X[r * 4 + (g ^ ((r >> 2) & 3))];
        const uint4 hi = X[r * 4 + ((2 + g) ^ ((r >> 2) & 3))];
        xf[set][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        cp(4 + j, q, d);
      }
      if (BS && !SG && set == 1) {   // this body issues an even stage
        cp(XC8 + 4, q, d);
        cp(XC8 + 5, q, d);
      }
    };
    // MFMAs of the stage with parity sp (its scale byte is 2 (sp) + g of the word)
    auto mm = [&](int set, int sp, const uint32_t (&ws)[4], const uint32_t (&xs)[JN]) {
      const int sh = 8 * (2 * sp + g);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf[set][i], xf[set][j], acc[i][j], a_fmt<WF>(), 0, 0, (int)((ws[i] >> sh) & 0xFF), 0,
              (int)((xs[j] >> sh) & 0xFF));
    };
    // P: the stage's parity as a constant (stages come in pairs: K is a multiple of
    // 128), which picks the fragment registers and the scale byte
    auto body = [&](int st, bool first, auto pc) {
      constexpr int P = decltype(pc)::value;
      const int slot = st & (MX8_SLOTS - 1);
      const int q = st + MX8_SLOTS - 1 < nsub ? st + MX8_SLOTS - 1 : nsub - 1;
      const uint32_t d = (uint32_t)((st + MX8_SLOTS - 1) & (MX8_SLOTS - 1)) * SLOT_B;
      if (SG && ((st + MX8_SLOTS - 1) & 7) == 0 && st + MX8_SLOTS - 1 < nsub) cp_group(q);
      rd_issue(slot, st, P, q, d);
      if (!first) mm(P ^ 1, P ^ 1, wsp, xsp);   // the previous stage
#pragma unroll
      for (int i = 0; i < 4; ++i) wsp[i] = wsr[i];
#pragma unroll
      for (int j = 0; j < JN; ++j) xsp[j] = xsr[j];
      // issue order (0x008 MFMA, 0x100 LDS read): the stage's (4 + JN +) 8 + 2 JN
      // reads between the previous stage's 4 JN MFMAs
      constexpr int NR = 8 + 2 * JN + (BS && P == 0 ? 4 + JN : 0);
      if (first) {
        __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);
      } else if (JV == 4) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          if (BS && P == 0 && (r & 1) == 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      } else {
        sched_mfma_reads<4 * JN, NR>();
      }
      __builtin_amdgcn_sched_barrier(0);
      // copies complete in issue order: the two younger stages' may still be in flight
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NWAIT) : "memory");
      __syncthreads();
    };
    static_assert((MX8_SLOTS & (MX8_SLOTS - 1)) == 0, "slot index is taken with a mask");
    static_assert(MX8_SLOTS == 4, "the prologue and the wait count assume four slots");
#pragma unroll
    for (int q = 0; q < MX8_SLOTS - 1; ++q) {   // stages 0 (+words / group), 1, 2 (+words)
      if (SG && q == 0) cp_group(0);
#pragma unroll
      for (int c = 0; c < ((BS && !SG && (q & 1) == 0) ? XC8 + 6 : XC8 + 4); ++c)
        cp(c, q < nsub ? q : nsub - 1, (uint32_t)q * SLOT_B);
    }
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NWAIT) : "memory");
    __syncthreads();
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    body(0, true, P0{});
    body(1, false, P1{});
    for (int st = 2; st < nsub; st += 2) {
      body(st, false, P0{});
      body(st + 1, false, P1{});
    }
    mm(1, 1, wsp, xsp);   // the last stage (odd)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  }

  // The epilogue below stores under per-lane row conditions. The MFMAs read every
  // lane's operands, so none of them may be moved into those branches (where lanes
  // beyond the tile's rows are switched off): pass each accumulator through an
  // opaque, side-effecting asm before any branch.
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JN; ++j) asm volatile("" : "+a"(acc[i][j]));
  const int hi4 = (lane >> 5) * 4;
  const float alpha = pt_alpha<WF>(a, e);
  // Staged through LDS, as in the bf16 forward kernels: in registers a lane holds 4
  // columns of one row, so stores straight from registers would cover 32 rows x 4
  // (FC1) or 8 (FC2) bytes per instruction. The tile goes to LDS (16-byte chunks
  // XOR-swizzled by row) and leaves in whole 128-byte lines; FC1's block scale codes
  // leave as one 4-byte word per row (I is a multiple of 128, so a tile's four codes
  // of a row are one aligned word; outputs are 16-byte aligned by the entry points).
  char* lds = reinterpret_cast<char*>(smem);
  const int rows = mend - m0 < 64 * JN ? mend - m0 : 64 * JN;
  __syncthreads();   // no wave still reads a stage or has a copy in flight
  if (fc1) {
    // e4m3 tile [256 rows][128 B] at 0, scale codes [256 rows][4 B] after it
    constexpr int SC_OFF = 256 * 128;
    float lim = 0.f;
    if (EPI == MX_FC1_STEP) lim = a.limits ? a.limits[e] : a.def_limit;
    const float qinv = BS ? 1.f : 1.0f / a.q_scale[0];
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int R = (2 * j + wm) * 32 + rsel;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        float v[16];
        float amax = 0.f;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          float u = acc[i][j][q] * alpha;
          float gt = acc[i + 2][j][q] * alpha;
          if (EPI == MX_FC1_STEP) {
            u = fminf(fmaxf(u, -lim), lim);
            gt = fminf(fmaxf(gt, -lim), lim);
          }
          v[q] = silu_f32(gt) * u;
          amax = fmaxf(amax, fabsf(v[q]));
        }
        uint32_t code = 0;
        float inv = qinv;
        if (BS) {
          amax = fmaxf(amax, __shfl_xor(amax, 32));
          code = ue8m0_round_up_448(amax);
          inv = __uint_as_float((254u - code) << 23);   // 2^(127 - code)
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q_in<WF>(v[4 * q], inv),
                                                   q_in<WF>(v[4 * q + 1], inv), 0, false);
          pk = __builtin_amdgcn_cvt_pk_fp8_f32(q_in<WF>(v[4 * q + 2], inv),
                                               q_in<WF>(v[4 * q + 3], inv), pk, true);
          const int c = wn * 64 + i * 32 + q * 8 + hi4;   // byte column of the tile
          const int off = R * 128 + ((((c >> 4) ^ ((R >> 1) & 7)) << 4) | (c & 15));
          *reinterpret_cast<uint32_t*>(lds + off) = (uint32_t)pk;
        }
        if (BS && g == 0) lds[SC_OFF + R * 4 + wn * 2 + i] = (char)code;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    __syncthreads();
    const int k = lane & 7;   // 16-byte chunk of a 128-byte tile row; 8 rows per read
    const int col = nt * 128 + k * 16;
    if (col < a.I) {
#pragma unroll 2
      for (int r0 = wid * 8; r0 < rows; r0 += 32) {
        const int R = r0 + (lane >> 3);
        if (R >= rows) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + R * 128 + ((k ^ ((R >> 1) & 7)) << 4));
        *reinterpret_cast<uint4*>(a.Cq + (int64_t)(m0 + R) * a.I + col) = v;
      }
    }
    if (BS) {
      const int R = wid * 64 + lane;
      if (R < rows)
        *reinterpret_cast<uint32_t*>(a.Cq_sf + (int64_t)(m0 + R) * (a.I >> 5) + nt * 4) =
            *reinterpret_cast<const uint32_t*>(lds + SC_OFF + R * 4);
    }
  } else {
    // bf16 tile [256 rows][512 B]
#pragma unroll
    for (int j = 0; j < JN; ++j) {
      const int R = (2 * j + wm) * 32 + rsel;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int c = wn * 128 + i * 32 + q * 8 + hi4;
          const int off = R * 512 + ((((c >> 3) ^ (R & 31)) << 4) | (hi4 << 1));
          *reinterpret_cast<uint2*>(lds + off) =
              make_uint2(pack_bf16x2(acc[i][j][q * 4 + 0] * alpha, acc[i][j][q * 4 + 1] * alpha),
                         pack_bf16x2(acc[i][j][q * 4 + 2] * alpha, acc[i][j][q * 4 + 3] * alpha));
          // one block at a time: batching all blocks' values costs registers
          if (q == 3) __builtin_amdgcn_sched_barrier(0);
        }
    }
    __syncthreads();
    const int k = lane & 31;   // 16-byte chunk of a 512-byte tile row; 2 rows per read
    const int col = nt * MTB + k * 8;
    if (col < a.N) {
#pragma unroll 4
      for (int r0 = wid * 2; r0 < rows; r0 += 8) {
        const int R = r0 + (lane >> 5);
        if (R >= rows) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(lds + R * 512 + ((k ^ (R & 31)) << 4));
        *reinterpret_cast<uint4*>(a.C + (int64_t)(m0 + R) * a.ldc + col) = v;
      }
    }
  }
}

// 256-row tiles; each picks the number of 32-row blocks per row-wave that hold rows.
// SG (block-scaled weights, K a multiple of 512): block scales copied in groups of
// 512 contraction values per row.
template <int EPI, int WF, bool SG>
__device__ __forceinline__ void mx_tile_jv(const MxArgs& a, uint4* smem, int e, int m0, int mend,
                                           int nt, int t) {
  const int jv = (mend - m0 + 63) >> 6;   // 1..4
  if (jv >= 4)
    mx_tile<EPI, WF, 4, SG>(a, smem, e, m0, mend, nt, t);
  else if (jv == 3)
    mx_tile<EPI, WF, 3, SG>(a, smem, e, m0, mend, nt, t);
  else if (jv == 2)
    mx_tile<EPI, WF, 2, SG>(a, smem, e, m0, mend, nt, t);
  else
    mx_tile<EPI, WF, 1, SG>(a, smem, e, m0, mend, nt, t);
}

template <int EPI, int WF, bool SG>
__global__ __launch_bounds__(MNT, 1) void k_gemm_mx(MxArgs a) {
  __shared__ uint4 smem[mx_lds_u4_max(WF == WF_MXFP4 ? 0 : 1)];
  int e, m0, mend, nt;
  if (!deal_tile<MTB>(a.ends, a.E, a.m_cap, a.n_tiles, e, m0, mend, nt)) return;
  mx_tile_jv<EPI, WF, SG>(a, smem, e, m0, mend, nt, (int)threadIdx.x);
}

// Work-queue form (as the bf16 forward's k_gemm_nt_q): one workgroup per CU takes the
// 256-row tiles from per-XCD ranges of the dealing order, stealing from the other
// ranges at the end, so CUs freed by tiles of fewer 32-row blocks take new work
// instead of waiting for the in-order dispatch. The tiles are computed exactly as by
// k_gemm_mx. Counters a.qcnt[0..8] (per range, finished workgroups) are zero at
// launch -- the sort clears them -- and the last workgroup to finish resets them.
template <int EPI, int WF, bool SG>
__global__ __launch_bounds__(MNT, 1) void k_gemm_mx_q(MxArgs a) {
  __shared__ uint4 smem[mx_lds_u4_max(WF == WF_MXFP4 ? 0 : 1)];
  const bool one_pass = a.E <= 64;
  TileScan64 sc{};
  if (one_pass) sc = tile_scan64<MTB>(a.ends, a.E, a.m_cap, a.n_tiles);
  const int total = one_pass ? sc.total : tile_count<MTB>(a.ends, a.E, a.m_cap, a.n_tiles);
  const int per = (total + 7) >> 3;
  const int x = (int)(blockIdx.x & 7);
  int* q = a.qcnt;
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
      tile_locate64<MTB>(sc, a.n_tiles, a.n_tiles, tile, e, m0, mend, nt);
    else
      tile_locate<MTB>(a.ends, a.E, a.m_cap, a.n_tiles, tile, e, m0, mend, nt);
    mx_tile_jv<EPI, WF, SG>(a, smem, e, m0, mend, nt, t);
  }
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(q + 8, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1) {   // every other workgroup has taken its last tile
#pragma unroll
      for (int i = 0; i < 9; ++i) __hip_atomic_store(q + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Few rows per expert (decode): the cost is streaming the expert bank once. Tile:
// 32 activation rows (one MFMA column block) by 64 weight rows (FC1: 32 up rows and
// the 32 gate rows of the same output columns, i.e. one requantization block; FC2:
// 64 output columns); the 4 waves split the contraction and meet in LDS at the end.
// A wave streams its 64 rows x (its share of K) in stages of 128 weight bytes per row
// (4 steps of 64 values for MXFP4, 2 for MXFP8): each load instruction takes 8 whole
// 128-byte lines (lane l: row 8j + l / 8, 16-byte chunk l % 8). Weight stages are loaded two ahead into
// registers and pass through a private LDS slot that turns them into MFMA fragments
// (chunks swizzled by (row >> 1) & 7; one slot is enough because a wave's LDS operations
// run in order). The weight scales of the wave's range are read into LDS once at the
// start; the activation fragments come straight from global memory, one stage ahead
// (for decode most tile rows repeat the same token, so those loads are cheap). Two
// blocks share a CU.
constexpr int STB = 32;         // activation rows per tile
constexpr int SCW = 16;         // weight-scale dwords kept per row and wave
constexpr int SMAX_K = 2048;    // contraction per wave that they cover (one byte per 32)

template <int NS>
struct MxAct {
  u32x4 xl[NS], xh[NS];
  uint32_t sx[NS];
};
struct MxW {
  u32x4 v[8];
};

template <int EPI, int WF>
__global__ __launch_bounds__(256, 2) void k_gemm_mx_stream(MxArgs a) {
  constexpr int WB = wbits<WF>();
  constexpr bool BS = block_scaled<WF>();
  constexpr int NS = 128 * 8 / WB / 64;   // 64-value steps per 128-byte stage: 4 or 2
  __shared__ u32x4 ring[4][512];              // [wave][64 rows x 8 chunks]
  __shared__ uint32_t scl[4][64][SCW];        // [wave][tile row][scale dwords]
  int e, m0, mend, nt;
  if (!deal_tile<STB>(a.ends, a.E, a.m_cap, a.n_tiles, e, m0, mend, nt)) return;
  constexpr bool fc1 = EPI != MX_FC2;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 31, g = lane >> 5;
  const int K = a.K, ks = K >> 5;
  const uint32_t kh = (uint32_t)K * WB / 8;   // weight bytes per row
  // weight row (within the expert) of tile row R in [0, 64)
  auto wrow_of = [&](int R) -> int {
    if (fc1) return (R >> 5) * a.I + min(nt * 32 + (R & 31), a.I - 1);
    return min(nt * 64 + R, a.NB - 1);
  };
  const int64_t eb = (int64_t)e * a.NB;
  const uint8_t* Bw = a.B + eb * kh;
  const uint8_t* Bs = a.B_sf + eb * ks;
  // stages of NS steps of 64 values (K is a multiple of 64 NS); wave w takes stages
  // [s0, s0 + nst)
  const int nstg = K / (64 * NS);
  const int s0 = wid * nstg / 4;
  const int nst = (wid + 1) * nstg / 4 - s0;

  // weight scales of this wave's stages: 2 NS bytes per stage and row, from byte
  // 2 NS s0
  uint32_t sreg[SCW];
  if (BS) {
    const uint32_t* srow =
        reinterpret_cast<const uint32_t*>(Bs + (int64_t)wrow_of(lane) * ks + 2 * NS * s0);
#pragma unroll
    for (int d = 0; d < SCW; ++d) sreg[d] = d < NS / 2 * nst ? srow[d] : 0u;
  }

  // 32-bit per-lane offsets from stage-uniform bases. Weights: instruction j loads
  // tile row R = 8j + lane / 8, chunk (lane % 8) ^ ((R >> 1) & 7), and stores it to
  // LDS chunk lane % 8 of that row.
  uint32_t voff[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int R = 8 * j + (lane >> 3);
    voff[j] = (uint32_t)wrow_of(R) * kh + 16u * ((lane & 7) ^ ((R >> 1) & 7));
  }
  int p = m0 + r;
  p = p < mend ? p : mend - 1;
  const int src = a.a_gather ? a.a_gather[p] / a.a_div : p;
  const uint32_t xoff = (uint32_t)src * (uint32_t)K + 16u * g;
  const uint32_t xsoff = (uint32_t)src * (uint32_t)ks + g;

  // loads of stage q (clamped to the last stage: the extra copies are never used)
  auto issue_w = [&](int q, MxW& w) {
    const uint8_t* base = Bw + 128 * (s0 + min(q, nst - 1));
#pragma unroll
    for (int j = 0; j < 8; ++j) w.v[j] = *reinterpret_cast<const u32x4*>(base + voff[j]);
  };
  auto issue_a = [&](int q, MxAct<NS>& act) {
    const int st = s0 + min(q, nst - 1);
    const uint8_t* xb = a.A + 64 * NS * st;
    const uint8_t* sbp = a.A_sf + 2 * NS * st;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      act.xl[s] = *reinterpret_cast<const u32x4*>(xb + xoff + 64 * s);
      act.xh[s] = *reinterpret_cast<const u32x4*>(xb + xoff + 64 * s + 32);
      act.sx[s] = BS ? sbp[xsoff + 2 * s] : UNIT_SCALE;
    }
  };
  auto stash = [&](const MxW& w) {
    u32x4* dst = &ring[wid][0];
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[64 * j + lane] = w.v[j];
  };
  f32x16 acc0, acc1;
#pragma unroll
  for (int q = 0; q < 16; ++q) acc0[q] = acc1[q] = 0.f;
  const uint8_t* sc0 = reinterpret_cast<const uint8_t*>(&scl[wid][r][0]);
  const uint8_t* sc1 = reinterpret_cast<const uint8_t*>(&scl[wid][32 + r][0]);
  // A fragment of weight row R for step s: MXFP4 one 16-byte chunk (2s + g), MXFP8
  // the chunks 4s + g and 4s + 2 + g (k = 16g + b and 32 + 16g + b of the step)
  auto wfrag = [&](const u32x4* W, int R, int s) -> v8i {
    const int sw = (R >> 1) & 7;
    if (WF == WF_MXFP4) {
      const u32x4 v = W[R * 8 + ((2 * s + g) ^ sw)];
      return v8i{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
    }
    const u32x4 lo = W[R * 8 + ((4 * s + g) ^ sw)];
    const u32x4 hi = W[R * 8 + ((4 * s + 2 + g) ^ sw)];
    return v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
  };
  auto compute = [&](int q, const MxAct<NS>& act) {
    const u32x4* W = &ring[wid][0];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int bi = 2 * NS * q + 2 * s + g;
      const v8i f0 = wfrag(W, r, s);
      const v8i f1 = wfrag(W, 32 + r, s);
      const v8i x{(int)act.xl[s].x, (int)act.xl[s].y, (int)act.xl[s].z, (int)act.xl[s].w,
                  (int)act.xh[s].x, (int)act.xh[s].y, (int)act.xh[s].z, (int)act.xh[s].w};
      const int s0w = BS ? (int)sc0[bi] : UNIT_SCALE, s1w = BS ? (int)sc1[bi] : UNIT_SCALE;
      acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f0, x, acc0, a_fmt<WF>(), 0, 0, s0w, 0,
                                                             (int)act.sx[s]);
      acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(f1, x, acc1, a_fmt<WF>(), 0, 0, s1w, 0,
                                                             (int)act.sx[s]);
    }
  };

  if (nst > 0) {
    // issue order W(0) A(0) W(1), then per stage q: W(q + 2) A(q + 1); stage q's
    // MFMAs wait for A(q), by which time W(q + 1) is in too and goes to LDS after them
    MxW W0, W1;
    MxAct<NS> A0, A1;
    issue_w(0, W0);
    issue_a(0, A0);
    issue_w(1, W1);
    __builtin_amdgcn_sched_barrier(0);
    if (BS) {
#pragma unroll
      for (int d = 0; d < SCW; ++d) scl[wid][lane][d] = sreg[d];
    }
    stash(W0);
    // (the scheduling barriers keep the compiler from sinking loads to their uses)
    for (int q = 0; q < nst; q += 2) {
      issue_w(q + 2, W0);
      issue_a(q + 1, A1);
      __builtin_amdgcn_sched_barrier(0);
      compute(q, A0);
      if (q + 1 >= nst) break;
      stash(W1);
      issue_w(q + 3, W1);
      issue_a(q + 2, A0);
      __builtin_amdgcn_sched_barrier(0);
      compute(q + 1, A1);
      if (q + 2 >= nst) break;
      stash(W0);
    }
  }
  __syncthreads();
  float* red = reinterpret_cast<float*>(&ring[0][0]);   // [3][2][16][64]
  if (wid > 0) {
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      red[(((wid - 1) * 2 + 0) * 16 + q) * 64 + lane] = acc0[q];
      red[(((wid - 1) * 2 + 1) * 16 + q) * 64 + lane] = acc1[q];
    }
  }
  __syncthreads();
  if (wid != 0) return;
#pragma unroll
  for (int w = 0; w < 3; ++w)
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      acc0[q] += red[((w * 2 + 0) * 16 + q) * 64 + lane];
      acc1[q] += red[((w * 2 + 1) * 16 + q) * 64 + lane];
    }

  // D layout: register q of lane l holds token m0 + l % 32 and output column
  // 8 * (q / 4) + 4 * (l / 32) + q % 4 of its 32-column group
  const int hi4 = g * 4;
  const int prow = m0 + r;
  const float alpha = pt_alpha<WF>(a, e);
  if (fc1) {
    float lim = 0.f;
    if (EPI == MX_FC1_STEP) lim = a.limits ? a.limits[e] : a.def_limit;
    float v[16];
    float amax = 0.f;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      float u = acc0[q] * alpha, gt = acc1[q] * alpha;
      if (EPI == MX_FC1_STEP) {
        u = fminf(fmaxf(u, -lim), lim);
        gt = fminf(fmaxf(gt, -lim), lim);
      }
      v[q] = silu_f32(gt) * u;
      amax = fmaxf(amax, fabsf(v[q]));
    }
    uint32_t code = 0;
    float inv;
    if (BS) {
      amax = fmaxf(amax, __shfl_xor(amax, 32));
      code = ue8m0_round_up_448(amax);
      inv = __uint_as_float((254u - code) << 23);
    } else {
      inv = 1.0f / a.q_scale[0];
    }
    if (prow >= mend) return;
    uint8_t* crow = a.Cq + (int64_t)prow * a.I + nt * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int pk = __builtin_amdgcn_cvt_pk_fp8_f32(q_in<WF>(v[4 * q], inv), q_in<WF>(v[4 * q + 1], inv), 0,
                                               false);
      pk = __builtin_amdgcn_cvt_pk_fp8_f32(q_in<WF>(v[4 * q + 2], inv), q_in<WF>(v[4 * q + 3], inv), pk,
                                           true);
      *reinterpret_cast<uint32_t*>(crow + q * 8 + hi4) = (uint32_t)pk;
    }
    if (BS && g == 0) a.Cq_sf[(int64_t)prow * (a.I >> 5) + nt] = (uint8_t)code;
  } else {
    if (prow >= mend) return;
    uint16_t* crow = a.C + (int64_t)prow * a.ldc;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = nt * 64 + i * 32 + q * 8 + hi4;
        if (col >= a.N) continue;
        const f32x16& ac = i ? acc1 : acc0;
        *reinterpret_cast<uint2*>(crow + col) =
            make_uint2(pack_bf16x2(ac[q * 4 + 0] * alpha, ac[q * 4 + 1] * alpha),
                       pack_bf16x2(ac[q * 4 + 2] * alpha, ac[q * 4 + 3] * alpha));
      }
  }
}

// The decode kernel takes over while the experts hold few rows on average. The
// 256-row tiles multiply only the 32-row blocks that hold rows, so the crossover is
// low; measured at H=7168, I=2048, 64 experts (rows per expert, on average): FC1
// 3 (MXFP4), 12 (MXFP8), 24 (fp8 per-tensor); FC2 never for MXFP4 (the 256-row tile
// is faster even at one token), 2 for the 8-bit weights.
inline int mx_stream_rows(int wf, int stage) {
  if (stage == 1) return wf == WF_MXFP4 ? 3 : wf == WF_MXFP8 ? 12 : 24;
  return wf == WF_MXFP4 ? 0 : 2;
}
inline bool mx_small_fits(int K, int NB, int64_t act_rows, int wb) {
  const int stage_k = 128 * 8 / wb;
  return K % stage_k == 0 && K <= 4 * SMAX_K && (int64_t)NB * K * wb / 8 < (1LL << 31) &&
         act_rows * K < (1LL << 31);
}

// Tile family of a stage: `force` 0 / 1 picks the 256-row / streaming tile (the
// latter only where it fits), -1 a choice recorded by moe_tune for this shape and
// bucket, else the built-in rule.
inline bool mx_use_small(int64_t R, int L, int K, int NB, int64_t act_rows, int rows_per_expert,
                         int wb, int stage, int wf, int force) {
  if (!mx_small_fits(K, NB, act_rows, wb)) return false;
  if (force < 0) force = tune_lookup(stage, wf, K, NB, L, R);
  if (force >= 0) return force == 1;
  return R <= (int64_t)rows_per_expert * L;
}

// The 256-row tiles take the work-queue kernel (counters given) from MX_QUEUE_ROWS
// expected rows per expert: measured on the layer at H=7168, I=2048, 64 experts, top-8
// (all three weight formats), it is 1-3% faster at 256 and 1024 rows per expert and
// 1-8% slower at 16 and 128, where a tile is one 32-row block and the weight stream
// sets the pace.
constexpr int MX_QUEUE_ROWS = 256;

// Row tiles of tm rows over L experts holding R rows in all: at most one partial
// tile per non-empty expert, and there are at most min(L, R) of those.
inline int64_t mx_row_tiles(int64_t R, int L, int tm) { return R / tm + (R < L ? R : L); }

}  // namespace

template <int EPI, int WF>
moe_status mx_launch(const MxArgs& a, bool small, int64_t tiles, hipStream_t st) {
  int grid = (int)((tiles + 7) / 8 * 8);
  const bool sg = block_scaled<WF>() && a.K % 512 == 0;
  if (small) {
    k_gemm_mx_stream<EPI, WF><<<grid, 256, 0, st>>>(a);
  } else if (a.qcnt) {
    const int pers = std::max(8, device_cu_count() & ~7);
    grid = grid < pers ? grid : pers;
    if (sg)
      k_gemm_mx_q<EPI, WF, block_scaled<WF>()><<<grid, MNT, 0, st>>>(a);
    else
      k_gemm_mx_q<EPI, WF, false><<<grid, MNT, 0, st>>>(a);
  } else if (sg) {
    k_gemm_mx<EPI, WF, block_scaled<WF>()><<<grid, MNT, 0, st>>>(a);
  } else {
    k_gemm_mx<EPI, WF, false><<<grid, MNT, 0, st>>>(a);
  }
  return launch_status();
}

template <int EPI>
moe_status mx_launch_w(const MxArgs& a, int wf, bool small, int64_t tiles, hipStream_t st) {
  if (wf == WF_FP8) return mx_launch<EPI, WF_FP8>(a, small, tiles, st);
  if (wf == WF_MXFP8) return mx_launch<EPI, WF_MXFP8>(a, small, tiles, st);
  return mx_launch<EPI, WF_MXFP4>(a, small, tiles, st);
}

inline int wf_bits(int wf) { return wf == WF_MXFP4 ? 4 : 8; }

// Whether the streaming tile can serve a stage of this shape (for the tuner).
bool mx_small_possible(int stage, int wf, int H, int I, int64_t R) {
  return stage == 1 ? mx_small_fits(H, 2 * I, R, wf_bits(wf)) : mx_small_fits(I, H, R, wf_bits(wf));
}

// FC1: act (e4m3) = requant(activation(x[p2e[p]/k] @ w1[e].T)) for permuted rows p.
// wf: WF_MXFP4 / WF_MXFP8 (x_sf, w1_sf UE8M0 block scales; act_sf out) or WF_FP8
// (x_sf float [1], w1_sf float [L], act_scale float [1] in; act_sf unused).
moe_status mx_fc1_enqueue(int activation, int wf, const void* x, const void* x_sf,
                          const int32_t* p2e, int top_k, const void* w1, const void* w1_sf, int L,
                          const int32_t* offs, int64_t R, int H, int I, const float* limits,
                          void* act, void* act_sf, const float* act_scale, hipStream_t st,
                          int force, int32_t* qcnt, int rows_hint) {
  if (R == 0) return MOE_OK;
  if (wf != WF_MXFP4 && wf != WF_MXFP8 && wf != WF_FP8) return MOE_ERR_DTYPE;
  MxArgs a{};
  a.A = reinterpret_cast<const uint8_t*>(x);
  a.A_sf = reinterpret_cast<const uint8_t*>(x_sf);
  a.a_gather = p2e;
  a.a_div = top_k;
  a.B = reinterpret_cast<const uint8_t*>(w1);
  a.B_sf = reinterpret_cast<const uint8_t*>(w1_sf);
  a.ends = offs;
  a.E = L;
  a.m_cap = (int)R;
  a.NB = 2 * I;
  a.N = I;
  a.K = H;
  a.Cq = reinterpret_cast<uint8_t*>(act);
  a.Cq_sf = reinterpret_cast<uint8_t*>(act_sf);
  a.I = I;
  a.limits = limits;
  a.def_limit = 7.0f;
  a.a_scale = reinterpret_cast<const float*>(x_sf);
  a.w_scale = reinterpret_cast<const float*>(w1_sf);
  a.q_scale = act_scale;
  a.qcnt = rows_hint >= MX_QUEUE_ROWS ? qcnt : nullptr;
  const bool small = mx_use_small(R, L, H, 2 * I, R, mx_stream_rows(wf, 1), wf_bits(wf), 1, wf, force);
  a.n_tiles = small ? I / 32 : (I + 127) / 128;
  const int64_t tiles = mx_row_tiles(R, L, small ? STB : MTB) * a.n_tiles;
  if (activation == MOE_ACT_SWIGLU_STEP) return mx_launch_w<MX_FC1_STEP>(a, wf, small, tiles, st);
  return mx_launch_w<MX_FC1_SWIGLU>(a, wf, small, tiles, st);
}

// FC2: y[p] (bf16) = act[p] @ w2[e].T; act_sf / w2_sf as x_sf / w1_sf above (FP8:
// act_sf is the float [1] scale of act).
moe_status mx_fc2_enqueue(int wf, const void* act, const void* act_sf, const void* w2,
                          const void* w2_sf, int L, const int32_t* offs, int64_t R, int H, int I,
                          void* y, hipStream_t st, int force, int32_t* qcnt, int rows_hint) {
  if (R == 0) return MOE_OK;
  if (wf != WF_MXFP4 && wf != WF_MXFP8 && wf != WF_FP8) return MOE_ERR_DTYPE;
  MxArgs a{};
  a.A = reinterpret_cast<const uint8_t*>(act);
  a.A_sf = reinterpret_cast<const uint8_t*>(act_sf);
  a.a_gather = nullptr;
  a.a_div = 1;
  a.B = reinterpret_cast<const uint8_t*>(w2);
  a.B_sf = reinterpret_cast<const uint8_t*>(w2_sf);
  a.ends = offs;
  a.E = L;
  a.m_cap = (int)R;
  a.NB = H;
  a.N = H;
  a.K = I;
  a.C = reinterpret_cast<uint16_t*>(y);
  a.qcnt = rows_hint >= MX_QUEUE_ROWS ? qcnt : nullptr;
  a.ldc = H;
  a.a_scale = reinterpret_cast<const float*>(act_sf);
  a.w_scale = reinterpret_cast<const float*>(w2_sf);
  const bool small = mx_use_small(R, L, I, H, R, mx_stream_rows(wf, 2), wf_bits(wf), 2, wf, force);
  a.n_tiles = small ? (H + 63) / 64 : (H + MTB - 1) / MTB;
  const int64_t tiles = mx_row_tiles(R, L, small ? STB : MTB) * a.n_tiles;
  return mx_launch_w<MX_FC2>(a, wf, small, tiles, st);
}

}  // namespace moe
