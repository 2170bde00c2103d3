// Host-side choice of GEMM tile and split-K, and the launch dispatch.
//
// The cost model counts, per CU, the matrix-core time of the tiles it runs
// (scaled by a per-tile efficiency: larger wave tiles need less LDS traffic
// per MFMA) plus the HBM time of the split-K partials, and takes the cheapest
// (tile, split) pair. MI355X: 256 CUs, 4096 bf16 flop/clk/CU at 2.4 GHz,
// 160 KiB LDS per CU.
#include <hip/hip_runtime.h>

#include "internal.h"

namespace tpmlp {
namespace {

constexpr int kCUs = 256;
constexpr double kFlopPerSecPerCU = 4096.0 * 2.4e9;
constexpr double kHbmBytesPerSec = 5.0e12;  // sustained, for partial traffic
constexpr double kLaunchSec = 2.0e-6;       // one extra kernel

struct PipeTile {
  TileId id;
  int bm, bn, lds_kib;
  double eff;
};
constexpr PipeTile kPipeTiles[] = {
    {kPipe256x256, 256, 256, 128, 0.85},
    {kPipe256x128, 256, 128, 96, 0.75},
    {kPipe128x256, 128, 256, 96, 0.75},
    {kPipe128x128, 128, 128, 64, 0.60},
};

double cost(int64_t M, int64_t N, int64_t K, int bm, int bn, int lds_kib, double eff, int split) {
  const int64_t tiles = (M / bm) * (N / bn) * split;
  const int64_t per_cu = 160 / lds_kib;  // workgroups resident per CU
  const int64_t rounds = (tiles + kCUs * per_cu - 1) / (kCUs * per_cu);
  const int64_t busiest = rounds * per_cu < tiles ? rounds * per_cu : tiles;  // tiles on one CU
  const double kc = static_cast<double>(K / split);
  double t = static_cast<double>(busiest) * 2.0 * bm * bn * kc / (kFlopPerSecPerCU * eff);
  if (split > 1) t += (split + 1.0) * M * N * 4.0 / kHbmBytesPerSec + kLaunchSec;
  return t;
}

}  // namespace

SplitPlan plan_gemm_bf16(int64_t M, int64_t N, int64_t K, bool allow_split) {
  SplitPlan best{kGeneral128x128, 1, K};
  double best_t = 1e30;
  static const int kSplits[] = {1, 2, 3, 4, 6, 8};
  const bool k_ok = K % 64 == 0;
  for (const PipeTile& t : kPipeTiles) {
    if (!k_ok || M % t.bm || N % t.bn) continue;
    for (int s : kSplits) {
      if (s > 1 && (!allow_split || K % (64 * s) || K / s < 256)) continue;
      const double c = cost(M, N, K, t.bm, t.bn, t.lds_kib, t.eff, s);
      if (c < best_t) {
        best_t = c;
        best = SplitPlan{t.id, s, K / s};
      }
    }
  }
  if (best_t < 1e30) return best;
  // General kernel (ragged shapes): split K when the grid is small.
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (allow_split && tiles < kCUs) {
    const int64_t want = (kCUs + tiles - 1) / tiles;
    const int64_t max_split = K / 256;
    const int64_t s = want < max_split ? want : max_split;
    if (s > 1) {
      int64_t chunk = (K + s - 1) / s;
      chunk = (chunk + 63) / 64 * 64;
      const int64_t n = (K + chunk - 1) / chunk;
      if (n > 1) best = SplitPlan{kGeneral128x128, static_cast<int>(n), chunk};
    }
  }
  return best;
}

hipError_t launch_gemm_bf16(const GemmParams& p, const SplitPlan& plan, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(p.a) & 15) == 0 && (p.lda & 7) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.b) & 15) == 0 && (p.ldb & 7) == 0;
  if (plan.tile >= kPipe256x256 && aligned) {
    const int ek = pipe_epilogue_kind(p);
    if (ek != kEpiNone) return launch_gemm_bf16_pipe(p, plan, ek, s);
  }
  return launch_gemm_bf16_general(p, plan, s);
}

}  // namespace tpmlp
