// Deterministic top-k combine ("finalize").
//
// SM90 fused-MoE page, Parameters (use_fused_finalize=False): FC2 writes unscaled
// rows, then the scales are applied and the k rows of a token are combined in
// float32 in a fixed order with one final rounding. Rows are read through
// expanded_idx_to_permuted_idx (StepFun page, "Prepared launches").
//
// HBM-bound: every local FC2 row is read once and every output row written once.
// One thread owns 8 consecutive columns (16-byte loads and stores); a block of
// 256 threads sweeps 2048 columns of one token, so each y row is read as long
// coalesced runs.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void k_finalize(const uint4* __restrict__ y,
                                                  const int32_t* __restrict__ e2p,
                                                  const float* __restrict__ w, int64_t T, int k,
                                                  int H8, uint4* __restrict__ out) {
  const int64_t t = blockIdx.y + (int64_t)gridDim.y * blockIdx.z;
  if (t >= T) return;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;  // 8-column chunk
  if (c >= H8) return;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  for (int s = 0; s < k; ++s) {
    const int p = e2p[t * k + s];
    if (p < 0) continue;
    const float ws = w[t * k + s];
    const uint4 v = y[(int64_t)p * H8 + c];
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += ws * bf16_bits_to_f32(u[j] & 0xFFFFu);
      acc[2 * j + 1] += ws * bf16_bits_to_f32(u[j] >> 16);
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  out[t * H8 + c] = o;
}

}  // namespace

moe_status finalize_enqueue(const void* y, const int32_t* e2p, const float* w, int64_t T, int k,
                            int H, void* out, hipStream_t st) {
  if (T == 0) return MOE_OK;
  const int H8 = H / 8;
  const unsigned gx = (unsigned)((H8 + 255) / 256);
  const int64_t gy = T < 65535 ? T : 65535;
  const int64_t gz = (T + gy - 1) / gy;
  k_finalize<<<dim3(gx, (unsigned)gy, (unsigned)gz), 256, 0, st>>>(
      reinterpret_cast<const uint4*>(y), e2p, w, T, k, H8, reinterpret_cast<uint4*>(out));
  return launch_status();
}

}  // namespace moe

using namespace moe;

extern "C" moe_status moe_finalize(const void* y, const int32_t* e2p, const float* topk_weights,
                                   int64_t T, int32_t top_k, int32_t H, void* out, void* stream) {
  if (T < 0 || top_k < 1 || top_k > 16 || H < 8 || H % 8) return MOE_ERR_SHAPE;
  if (T == 0) return MOE_OK;
  if (!y || !e2p || !topk_weights || !out) return MOE_ERR_NULL;
  if (!aligned16(y) || !aligned16(out)) return MOE_ERR_ALIGN;
  return finalize_enqueue(y, e2p, topk_weights, T, top_k, H, out, as_stream(stream));
}
