// Recorded tile-family choices of the layer's GEMM stages.
//
// SM90 fused-MoE page, Parameters: an autotuner profiles the legal tiles of each
// GEMM per token bucket and caches the winner; the built-in tile rule goes by rows
// per local expert. Here the candidates are two tile families per stage (bf16: the
// 256-row and 128-row tiles of gemm_bf16.hip; fp8 activations: the 256-row and the
// 32-row streaming tiles of gemm_mx.hip); moe_tune (api.hip) times both on the
// caller's data and stores the faster one under the stage, weight format (-1 for
// bf16), shape and bucket = rows per local expert rounded up to a power of two.
// Host-only code; one table per process, guarded by a mutex.
#include <map>
#include <mutex>
#include <tuple>

#include "common.h"

namespace moe {
namespace {

typedef std::tuple<int, int, int, int, int, int> TuneKey;   // stage, wf, K, NB, L, bucket

std::mutex& tune_mu() {
  static std::mutex m;
  return m;
}
std::map<TuneKey, int>& tune_table() {
  static std::map<TuneKey, int> t;
  return t;
}

int bucket_of(int64_t R, int L) {
  const int64_t per = L > 0 ? (R + L - 1) / L : R;
  int b = 1;
  while (b < per && b < (1 << 30)) b <<= 1;
  return b;
}

}  // namespace

int tune_lookup(int stage, int wf, int K, int NB, int L, int64_t R) {
  std::lock_guard<std::mutex> g(tune_mu());
  const auto& t = tune_table();
  if (t.empty()) return -1;
  const auto it = t.find(TuneKey(stage, wf, K, NB, L, bucket_of(R, L)));
  return it == t.end() ? -1 : it->second;
}

void tune_store(int stage, int wf, int K, int NB, int L, int64_t R, int choice) {
  std::lock_guard<std::mutex> g(tune_mu());
  tune_table()[TuneKey(stage, wf, K, NB, L, bucket_of(R, L))] = choice;
}

}  // namespace moe

extern "C" void moe_tune_clear(void) {
  std::lock_guard<std::mutex> g(moe::tune_mu());
  moe::tune_table().clear();
}
