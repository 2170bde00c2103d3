// Host-side choice of GEMM tile and split-K, and the launch dispatch.
//
// The cost model counts rounds of tiles over the device's CUs (256 on MI355X); a round costs a
// fixed overhead (prologue, epilogue, launch) plus the tile's matrix work at a
// per-CU rate measured for each tile configuration on MI355X (the clock runs
// at 1.8-2.2 GHz under matrix load, below the 2.4 GHz peak). A split K adds the
// HBM time of the fp32 partials (written, then read by the fix-up) and one
// fix-up launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <functional>
#include <queue>
#include <vector>

#include "internal.h"

namespace tpmlp {

DeviceShape device_shape() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cached[kMaxDevices];  // cus << 8 | xcds, 0 = not queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return DeviceShape{256, 8};
  }
  int v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1)
      cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess ||
        xcds < 1 || xcds > 255)
      xcds = cus % 8 == 0 ? 8 : 1;
    (void)hipGetLastError();
    v = cus << 8 | xcds;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return DeviceShape{v >> 8, v & 255};
}

namespace {

int cus() { return device_shape().cus; }
constexpr double kRoundOverheadSec = 3.0e-6;
constexpr double kHbmBytesPerSec = 5.0e12;  // sustained, for partial traffic
constexpr double kLaunchSec = 2.0e-6;       // one extra kernel
// time of a paired launch over its simulated time (measured on the
// 175B-class shard's 256x192 pairs: 1.09 and 1.14)
constexpr double kPairSlowdown = 1.12;

struct PipeTile {
  TileId id;
  int bm, bn;
  double flop_per_sec_per_cu;
  bool split_ok;  // measured competitive with split K
};
constexpr PipeTile kPipeTiles[] = {
    {kPipe256x256, 256, 256, 5.0e12, true},
    {kPipe256x128, 256, 128, 4.4e12, true},
    {kPipe128x256, 128, 256, 4.6e12, true},
    {kPipe128x128, 128, 128, 4.0e12, true},
    {kPipe256x192, 256, 192, 4.6e12, true},
    // one wave per SIMD on a 64x96 wave tile: ahead of 128x256 on unsplit
    // GPT-2-small products (19.3 vs 20.6 us), behind 128x128 once K is split
    {kPipe128x192, 128, 192, 4.2e12, false},
};

double cost(int64_t M, int64_t N, int64_t K, const PipeTile& t, int split) {
  const int64_t tiles = (M / t.bm) * (N / t.bn) * split;
  const int64_t rounds = (tiles + cus() - 1) / cus();
  const double flops = 2.0 * t.bm * t.bn * static_cast<double>(K / split);
  double c = static_cast<double>(rounds) * (kRoundOverheadSec + flops / t.flop_per_sec_per_cu);
  // the slices write their partials and the fix-up reads them back
  if (split > 1) c += (2.0 * split + 1.0) * M * N * 4.0 / kHbmBytesPerSec + kLaunchSec;
  return c;
}

thread_local int g_force_tile = 0;
thread_local int g_force_split = 1;

const PipeTile* find_tile(int id) {
  for (const PipeTile& t : kPipeTiles)
    if (t.id == id) return &t;
  return nullptr;
}

SplitPlan plan_model(int64_t M, int64_t N, int64_t K, bool allow_split);

}  // namespace

int forced_tile() { return g_force_tile; }

bool set_gemm_override(int tile, int splitk) {
  if ((tile != 0 && !find_tile(tile)) || splitk < 1 || splitk > 16) return false;
  g_force_tile = tile;
  g_force_split = splitk;
  return true;
}

SplitPlan plan_gemm_bf16(int64_t M, int64_t N, int64_t K, bool allow_split) {
  SplitPlan plan = plan_model(M, N, K, allow_split);
  const PipeTile* t = find_tile(g_force_tile);
  if (t && K % 64 == 0 && M % t->bm == 0 && N % t->bn == 0) {
    plan = SplitPlan{t->id, 1, K};
    const int s = g_force_split;
    if (allow_split && s > 1 && K % (64 * s) == 0) plan = SplitPlan{t->id, s, K / s};
  }
  return plan;
}

namespace {

SplitPlan plan_model(int64_t M, int64_t N, int64_t K, bool allow_split) {
  SplitPlan best{kGeneral128x128, 1, K};
  double best_t = 1e30;
  static const int kSplits[] = {1, 2, 3, 4, 6, 8};
  const bool k_ok = K % 64 == 0;
  for (const PipeTile& t : kPipeTiles) {
    if (!k_ok || M % t.bm || N % t.bn) continue;
    for (int s : kSplits) {
      if (s > 1 && (!allow_split || !t.split_ok || K % (64 * s) || K / s < 256)) continue;
      const double c = cost(M, N, K, t, s);
      if (c < best_t) {
        best_t = c;
        best = SplitPlan{t.id, s, K / s};
      }
    }
  }
  if (best_t < 1e30) return best;
  // General kernel (ragged shapes): split K when the grid is small.
  const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
  if (allow_split && tiles < cus()) {
    const int64_t want = (cus() + tiles - 1) / tiles;
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

}  // namespace

namespace {

// Simulated time of one paired launch: the weight gradient on tile w in `sp`
// K slices, the data gradient on tile d; one block per CU (the pair's stages
// fill most of the LDS), blocks go to the CU that frees first, the weight
// gradient's slices first. A split adds its fix-up.
double pair_cost(const PipeTile* w, const PipeTile* d, int64_t T, int64_t k, int64_t n, int sp) {
  const double kw = 2.0 * w->bm * w->bn * 64.0 / w->flop_per_sec_per_cu;
  const double kd = 2.0 * d->bm * d->bn * 64.0 / d->flop_per_sec_per_cu;
  const int64_t tiles_w = (k / w->bm) * (n / w->bn), tiles_d = (T / d->bm) * (k / d->bn);
  std::priority_queue<double, std::vector<double>, std::greater<double>> cu;
  for (int c = 0, n = cus(); c < n; ++c) cu.push(0.0);
  auto run = [&](int64_t blocks, double sec) {
    for (int64_t b = 0; b < blocks; ++b) {
      const double f = cu.top();
      cu.pop();
      cu.push(f + kRoundOverheadSec + sec);
    }
  };
  run(tiles_w * sp, static_cast<double>(T / sp / 64) * kw);
  run(tiles_d, static_cast<double>(n / 64) * kd);
  double c = 0.0;
  while (!cu.empty()) {
    c = cu.top();
    cu.pop();
  }
  if (sp > 1) c += (2.0 * sp + 1.0) * k * n * 4.0 / kHbmBytesPerSec + kLaunchSec;
  return c;
}

}  // namespace

// A data gradient whose own tile has no paired kernel (128x256, 256x128,
// 256x256): pair both products on 128x128 where they tile exactly and the
// model puts the pair below the two calls (data gradient on its own tile,
// weight gradient with its own plan, one more launch).
SplitPlan plan_pair_other_tile(int64_t T, int64_t k, int64_t n, const SplitPlan& pd) {
  const SplitPlan none{kPairNone, 1, T};
  const PipeTile* t = find_tile(kPipe128x128);
  if (g_force_tile != 0 || pd.tile == 0 || T % t->bm || k % t->bn || n % t->bn) return none;
  const SplitPlan pw = plan_gemm_bf16(k, n, T, true);
  const PipeTile* td = find_tile(pd.tile);
  const PipeTile* tw = find_tile(pw.tile);
  if (!td || !tw) return none;
  const double two_calls = cost(T, k, n, *td, 1) + cost(k, n, T, *tw, pw.splitk) + kLaunchSec;
  int best = 0;
  double best_c = 1e30;
  for (int sp : {1, 2, 4, 8}) {
    if (sp > 1 && (T % (64 * sp) || T / sp < 256)) continue;
    const double c = pair_cost(t, t, T, k, n, sp);
    if (c < best_c) {
      best_c = c;
      best = sp;
    }
  }
  if (best == 0 || best_c >= two_calls) return none;
  return SplitPlan{kPairSame128x128, best, T / best};
}

SplitPlan plan_pair(int64_t T, int64_t k, int64_t n) {
  const SplitPlan none{kPairNone, 1, T};
  // the data gradient keeps its own tile; the weight gradient takes 128x128
  // beside a 128-row data-gradient tile (faster than 128x192 in TN) and
  // 256x192 beside 256x192
  const SplitPlan pd = plan_gemm_bf16(T, k, n, false);
  int kind = kPairNone;
  TileId tw = kPipe128x128;
  if (pd.tile == kPipe128x192) kind = kPairW128x128D128x192;
  else if (pd.tile == kPipe128x128) kind = kPairSame128x128;
  else if (pd.tile == kPipe256x192) kind = kPairSame256x192, tw = kPipe256x192;
  if (kind == kPairNone) return plan_pair_other_tile(T, k, n, pd);
  const PipeTile* w = find_tile(tw);
  const PipeTile* d = find_tile(pd.tile);
  if (T % 64 || k % w->bm || n % w->bn) return none;
  if (g_force_tile != 0 && g_force_split > 1 && T % (64 * g_force_split) == 0)
    return SplitPlan{kind, g_force_split, T / g_force_split};
  auto split_ok = [&](int sp) { return sp == 1 || (T % (64 * sp) == 0 && T / sp >= 256); };
  int best = 0;
  double best_c = 1e30;
  int64_t best_blocks = 0;
  // a candidate wins on lower simulated time, or on equal time with fewer
  // blocks (the model's ties come from a long weight gradient hiding the data
  // gradient's rounds, which fewer blocks still shorten)
  auto consider = [&](const PipeTile* tw_, const PipeTile* td_, int kind_) {
    for (int sp : {1, 2, 4, 8}) {
      if (!split_ok(sp)) continue;
      const double c = pair_cost(tw_, td_, T, k, n, sp);
      const int64_t blocks = (k / tw_->bm) * (n / tw_->bn) * sp + (T / td_->bm) * (k / td_->bn);
      if (c < best_c - 1e-9 || (c < best_c + 1e-9 && blocks < best_blocks)) {
        best_c = c;
        best = sp;
        best_blocks = blocks;
        kind = kind_;
      }
    }
  };
  consider(w, d, kind);
  if (g_force_tile == 0) {
    // Both products on 256x192 as well, where both tile exactly: fewer,
    // larger blocks can fit the launch into one round of the CUs where the
    // 128-row tiles need two (GPT-2 small's fc2 backward: 224 blocks
    // against 328).
    const PipeTile* big = find_tile(kPipe256x192);
    if (kind != kPairSame256x192 && T % big->bm == 0 && k % big->bn == 0 && k % big->bm == 0 &&
        n % big->bn == 0)
      consider(big, big, kPairSame256x192);
    // A 128x128 data gradient also as 128x192 where k allows (GPT-2 small's
    // fc1 backward: 200 blocks against 264).
    const PipeTile* wide = find_tile(kPipe128x192);
    if (pd.tile == kPipe128x128 && k % wide->bn == 0)
      consider(w, wide, kPairW128x128D128x192);
  }
  if (g_force_tile == 0) {
    // Pair only where the model puts the pair clearly below the two calls
    // (the data gradient on its own tile, the weight gradient with its own
    // plan, one more launch). A paired block runs slower than the same tile
    // in a launch of its own (one kernel holds both bodies, and the LDS pool
    // and register budget are the larger product's): on the 175B-class shard
    // the 256x192 pairs took 652 and 668 us against 572 and 613 us for the
    // two calls, where the model has both at the same number of rounds.
    const SplitPlan pw1 = plan_gemm_bf16(k, n, T, true);
    const PipeTile* tw1 = find_tile(pw1.tile);
    const PipeTile* td1 = find_tile(pd.tile);
    if (tw1 && td1) {
      const double two_calls =
          cost(T, k, n, *td1, 1) + cost(k, n, T, *tw1, pw1.splitk) + kLaunchSec;
      if (best_c * kPairSlowdown >= two_calls) return none;
    }
  }
  return SplitPlan{kind, best, T / best};
}

int pair_free_cus(const SplitPlan& pl, int64_t T, int64_t k, int64_t n) {
  TileId tw = kPipe128x128, td = kPipe128x128;
  if (pl.tile == kPairW128x128D128x192) td = kPipe128x192;
  else if (pl.tile == kPairSame256x192) tw = td = kPipe256x192;
  else if (pl.tile != kPairSame128x128) return 0;
  const PipeTile* w = find_tile(tw);
  const PipeTile* d = find_tile(td);
  const int64_t blocks = (k / w->bm) * (n / w->bn) * pl.splitk + (T / d->bm) * (k / d->bn);
  return blocks < cus() ? static_cast<int>(cus() - blocks) : 0;
}

namespace {
const TileId kF8Tiles[] = {kPipe256x192, kPipe128x256, kPipe128x192, kPipe128x128};
}  // namespace

SplitPlan plan_gemm_fp8(int64_t M, int64_t N, int64_t K, bool allow_split) {
  // the bf16 cost model at twice the per-CU matrix rate, over the FP8 tiles
  static const int kSplits[] = {1, 2, 3, 4, 6, 8};
  SplitPlan best{0, 1, K};
  double best_t = 1e30;
  if (K % 128) return best;
  for (TileId id : kF8Tiles) {  // a forced tile, where it fits
    const PipeTile* t = find_tile(id);
    if (id != g_force_tile || M % t->bm || N % t->bn) continue;
    const int sp = g_force_split;
    if (allow_split && sp > 1 && K % (128 * sp) == 0) return SplitPlan{id, sp, K / sp};
    return SplitPlan{id, 1, K};
  }
  for (TileId id : kF8Tiles) {
    PipeTile t = *find_tile(id);
    if (M % t.bm || N % t.bn) continue;
    t.flop_per_sec_per_cu *= 2.0;
    for (int sp : kSplits) {
      if (sp > 1 && (!allow_split || !t.split_ok || K % (128 * sp) || K / sp < 512)) continue;
      const double c = cost(M, N, K, t, sp);
      if (c < best_t) {
        best_t = c;
        best = SplitPlan{t.id, sp, K / sp};
      }
    }
  }
  return best;
}

int gemm_pipe_epilogue(const GemmParams& p, const SplitPlan& plan) {
  const bool aligned = (reinterpret_cast<uintptr_t>(p.a) & 15) == 0 && (p.lda & 7) == 0 &&
                       (reinterpret_cast<uintptr_t>(p.b) & 15) == 0 && (p.ldb & 7) == 0;
  if (plan.tile < kPipe256x256 || !aligned) return kEpiNone;
  return pipe_epilogue_kind(p);
}

hipError_t launch_gemm_bf16(const GemmParams& p0, const SplitPlan& plan, hipStream_t s) {
  GemmParams p = p0;
  p.xcds = device_shape().xcds;
  const int ek = gemm_pipe_epilogue(p, plan);
  if (ek != kEpiNone) return launch_gemm_bf16_pipe(p, plan, ek, s);
  return launch_gemm_bf16_general(p, plan, s);
}

}  // namespace tpmlp
