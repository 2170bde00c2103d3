// The row work of the MLP step of p tensor-parallel shards on one device
// ("Megatron" page, "Tensor Parallelism / mathematical principles":
// U_i = X A_i + a_i, Y_i = GeLU(U_i), Z = sum_i Y_i B_i + b; the backward is
// the derivative of the same definitions) in one persistent launch.
//
// Each XCD owns a slab of T / XCDs token rows and drains its own ticket queue
// of units over those rows, in this order:
//   for each shard i: fc1 forward tiles (bias + GeLU, U_i and Y_i saved),
//                     fc2 forward partial tiles (Zp_i, fp32);
//   the sum over shards Z = sum_i Zp_i + b, in units of 16 rows;
//   for each shard i: fc2 data-gradient tiles (dU_i = dZ B_i^T * GeLU'(U_i)),
//                     fc1 data-gradient partial tiles (dXp_i, fp32);
//   the sum dX = sum_i dXp_i.
// A launch runs the whole queue, or only its forward units (F1, F2, S1) or
// only its backward units (D2, D1, S2), in the same order, for callers that
// run the two halves as separate calls. In a backward-only launch fc2's data
// gradient does not wait for fc1's forward tiles (an earlier launch wrote
// U_i), and with recompute its epilogue also rebuilds Y_i = GeLU(U_i) from the
// saved U_i for the weight gradient that follows. A launch can also leave
// the dX sum out of its queue (no_dx_sum), for the weight-gradient launch
// that follows it to run beside its tiles: the sum's units would otherwise
// come last and run alone after the final fc1 data-gradient tiles.
// A unit waits only for units of the same row block that come earlier in the
// same queue (fc2 forward for fc1's row block, the sums for every shard's row
// block, fc2's data gradient for fc1's forward tile, fc1's data gradient for
// fc2's). Producer and consumer therefore run on the same XCD and meet in its
// L2: the producer's stores are complete (vmcnt 0) before it counts itself
// done with an agent-scope atomic, and the consumer's loads come after it sees
// the count. A consumer never touches those rows before their count is
// complete, and the launch's start invalidated every CU's L1, so it cannot
// hold a stale copy. Tickets are taken in queue order and a unit only waits
// for earlier tickets, which running blocks hold: the queue drains however
// many blocks are resident.
//
// The weight gradients dB_i = Y_i^T dZ and dA_i = X^T dU_i read every token
// row, which every XCD writes here; they run after this launch as products of
// their own.
//
// The launch's last block to finish (agent-scope done count) sets the counters
// back to zero, so consecutive calls on one stream need no reset. A dependency
// wait polls a bounded number of times; if it gives up it sets the
// workspace's error word and carries on, so every block still exits.
#include <hip/hip_runtime.h>

#include "step_queue.h"

namespace tpmlp {
namespace {

// Counter layout (unsigned words from s.ctr): the tickets (xcds), the done
// count, the per-row-block counts cF1 [p][nrb], cF2 [nrb], cD2 [p][nrb],
// cD1 [nrb].
struct Layout {
  int64_t nrb;
  int64_t ta, da, f1, f2, d2, d1, end;
  __host__ __device__ explicit Layout(const StepParams& s) {
    nrb = s.T / s.rb;
    ta = 0;
    da = ta + s.xcds;
    f1 = da + 1;
    f2 = f1 + s.p * nrb;
    d2 = f2 + nrb;
    d1 = d2 + s.p * nrb;
    end = d1 + nrb;
  }
};

// Phases of a queue, in order. A unit only waits for units of earlier
// phases: fc1 forward (F1), fc2 forward (F2, after F1 of its row block and
// shard), fc2's data gradient (D2, after F1), the forward sum (S1, after every
// shard's F2), fc1's data gradient (D1, after D2) and the dX sum (S2, after
// every shard's D1). Within a product the shards come in order.
enum RowsKind : int { kF1 = 0, kF2 = 1, kS1 = 2, kD2 = 3, kD1 = 4, kS2 = 5 };
constexpr int kPhases = 6;

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void mlp_rows_kernel(StepParams s) {
  constexpr int RB = C::RB, TN = C::TN;
  constexpr int SS = RB / kSumRows;  // sum units per row block
  uint8_t* pool = pool_buf<C::POOL>();
  const Layout L(s);
  const int x = xcc_id() % s.xcds;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.clk[0] = clock64();
    s.clk[1] = wall_clock64();
  }
  const int64_t T = s.T, h = s.h, F = s.F;
  const int R = s.rbx;
  const int n1 = static_cast<int>(F / TN), n2 = static_cast<int>(h / TN);
  // the queue's phases and their sizes, in queue order: all six, the forward
  // three or the backward three
  const int nf1 = s.p * R * n1, nf2 = s.p * R * n2, nsum = R * SS;
  int counts[kPhases], kinds[kPhases], nph = 0;
  auto add = [&](int kind, int n) {
    kinds[nph] = kind;
    counts[nph++] = n;
  };
  // (with no_dx_sum the dX sum is a phase of no units, which keeps the
  // phase tables' layout fixed: the compiler holds them in registers)
  const int ns2 = s.no_dx_sum ? 0 : nsum;
  if (s.phases == 3) {
    add(kF1, nf1), add(kF2, nf2), add(kD2, nf1), add(kS1, nsum), add(kD1, nf2), add(kS2, ns2);
  } else if (s.phases == 1) {
    add(kF1, nf1), add(kF2, nf2), add(kS1, nsum);
  } else {
    add(kD2, nf1), add(kD1, nf2), add(kS2, ns2);
  }
  // fc2's data gradient waits for fc1's forward tiles only in the same launch
  const bool d2_waits = (s.phases & 1) != 0;
  unsigned* ctr = s.ctr;
  for (;;) {
    const unsigned tk = next_ticket(ctr + L.ta + x, pool);
    if (tk >= static_cast<unsigned>(s.units_a)) break;
    int t = static_cast<int>(tk), ph = 0;
    while (ph < nph - 1 && t >= counts[ph]) t -= counts[ph++];
    const int kind = kinds[ph];
    // t within the phase: (shard i,) row block j, column tile (or sum slice) n
    int i = 0, j = 0, n = 0;
    if (kind == kF1 || kind == kD2) {
      i = t / (R * n1);
      j = (t % (R * n1)) / n1;
      n = t % n1;
    } else if (kind == kF2 || kind == kD1) {
      i = t / (R * n2);
      j = (t % (R * n2)) / n2;
      n = t % n2;
    } else {  // the sums
      j = t / SS;
      n = t % SS;
    }
    const int64_t rg = static_cast<int64_t>(x) * R + j;  // global row block
    const int64_t m0 = rg * RB;
    GemmParams g{};
    g.splitk = 1;
    g.xcds = s.xcds;
    switch (kind) {
      case kF1: {  // fc1 forward: U_i = X A_i + a_i, Y_i = GeLU(U_i)
        g.a = s.x;
        g.lda = s.ld_x;
        g.b = bf(s.a) + i * F;
        g.ldb = s.ld_a;
        g.c = bfw(s.y) + i * F;
        g.c2 = bfw(s.u) + i * F;
        g.ldc = g.ldc2 = s.ld_u;
        g.bias = s.bias_a ? bf(s.bias_a) + i * F : nullptr;
        g.M = T, g.N = F, g.K = h, g.k_chunk = h;
        unit_tile<RB, TN, C::WM, C::WN, C::BKN, C::SN, true, false, kEpiBiasGelu, C::POOL>(
            g, m0, static_cast<int64_t>(n) * TN, static_cast<int>(h / C::BKN));
        signal_count(ctr + L.f1 + i * L.nrb + rg);
        break;
      }
      case kF2: {  // fc2 forward partial: Zp_i = Y_i B_i
        wait_count(ctr + L.f1 + i * L.nrb + rg, n1, s.spin, s.err);
        g.a = bf(s.y) + i * F;
        g.lda = s.ld_u;
        g.b = bf(s.b) + i * F * s.ld_b;
        g.ldb = s.ld_b;
        g.c = s.zp + i * T * h;
        g.ldc = h;
        g.M = T, g.N = h, g.K = F, g.k_chunk = F;
        unit_tile<RB, TN, C::WM, C::WN, C::BKN, C::SN, true, false, kEpiF32, C::POOL>(
            g, m0, static_cast<int64_t>(n) * TN, static_cast<int>(F / C::BKN));
        signal_count(ctr + L.f2 + rg);
        break;
      }
      case kS1:  // Z = sum_i Zp_i + b
        wait_count(ctr + L.f2 + rg, static_cast<unsigned>(s.p * n2), s.spin, s.err);
        rows_sum_unit(s.zp, T * h, s.p, h, s.bias_b, s.z, s.ld_z, m0 + n * kSumRows, h);
        break;
      case kD2: {  // fc2 data gradient: dU_i = (dZ B_i^T) * GeLU'(U_i)
        if (d2_waits) wait_count(ctr + L.f1 + i * L.nrb + rg, n1, s.spin, s.err);
        g.a = s.dz;
        g.lda = s.ld_dz;
        g.b = bf(s.b) + i * F * s.ld_b;
        g.ldb = s.ld_b;
        g.c = bfw(s.du) + i * F;
        g.ldc = s.ld_u;
        g.u = bf(s.u) + i * F;
        g.ldu = s.ld_u;
        if (s.recompute) {  // Y_i = GeLU(U_i) from the saved U_i
          g.c2 = bfw(s.y) + i * F;
          g.ldc2 = s.ld_u;
        }
        g.M = T, g.N = F, g.K = h, g.k_chunk = h;
        unit_tile<RB, TN, C::WM, C::WN, C::BKT, C::ST, true, true, kEpiDGelu, C::POOL>(
            g, m0, static_cast<int64_t>(n) * TN, static_cast<int>(h / C::BKT));
        signal_count(ctr + L.d2 + i * L.nrb + rg);
        break;
      }
      case kD1: {  // fc1 data-gradient partial: dXp_i = dU_i A_i^T
        wait_count(ctr + L.d2 + i * L.nrb + rg, n1, s.spin, s.err);
        g.a = bf(s.du) + i * F;
        g.lda = s.ld_u;
        g.b = bf(s.a) + i * F;
        g.ldb = s.ld_a;
        g.c = s.dxp + i * T * h;
        g.ldc = h;
        g.M = T, g.N = h, g.K = F, g.k_chunk = F;
        unit_tile<RB, TN, C::WM, C::WN, C::BKT, C::ST, true, true, kEpiF32, C::POOL>(
            g, m0, static_cast<int64_t>(n) * TN, static_cast<int>(F / C::BKT));
        signal_count(ctr + L.d1 + rg);
        break;
      }
      default:  // kS2: dX = sum_i dXp_i
        wait_count(ctr + L.d1 + rg, static_cast<unsigned>(s.p * n2), s.spin, s.err);
        rows_sum_unit(s.dxp, T * h, s.p, h, nullptr, s.dx, s.ld_dx, m0 + n * kSumRows, h);
        break;
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.clk[2] = clock64();
    s.clk[3] = wall_clock64();
  }
  finish_launch(ctr, L.da, L.ta, L.end);
}

// Queue length and workspace layout of a step (shapes and device only).
struct Plan {
  bool large;  // 256 x 128 tiles (RowsLarge), else 128 x 128 (RowsSmall)
  int xcds, rb, rbx, units_a;  // units_a: of one half (forward or backward)
  size_t off_ctr, bytes;
};

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Units of the forward (or of the backward) half of a queue.
template <class C>
int rows_units_half(int64_t T, int64_t h, int64_t F, int p, int X) {
  const int R = static_cast<int>(T / C::RB / X);
  const int n1 = static_cast<int>(F / C::TN), n2 = static_cast<int>(h / C::TN);
  const int ss = C::RB / kSumRows;
  return p * R * n1 + p * R * n2 + R * ss;
}

bool plan_step(int64_t T, int64_t h, int64_t F, int p, Plan* pl) {
  const DeviceShape d = device_shape();
  const int X = d.xcds;
  if (p < 1 || p > kMaxPartials || T < 1 || h < 1 || F < 1) return false;
  if (T % (static_cast<int64_t>(kRows) * X) || h % 128 || F % 128) return false;
  // the fused launch is for products too small to fill the device on their
  // own; above ~20 GFLOP a product keeps the one-product-per-launch path
  if (2.0 * T * h * F > 2.0e10) return false;
  Plan q{};
  q.xcds = X;
  // 256 x 128 tiles where the rows divide, else 128 x 128; 128 x 128 when
  // tp_set_gemm_override forces that tile
  q.large = T % (static_cast<int64_t>(RowsLarge::RB) * X) == 0 && forced_tile() != kPipe128x128;
  q.rb = q.large ? RowsLarge::RB : RowsSmall::RB;
  q.rbx = static_cast<int>(T / q.rb / X);
  q.units_a = q.large ? rows_units_half<RowsLarge>(T, h, F, p, X)
                      : rows_units_half<RowsSmall>(T, h, F, p, X);
  StepParams tmp{};
  tmp.T = T;
  tmp.p = p;
  tmp.xcds = X;
  tmp.rb = q.rb;
  const Layout lay(tmp);
  q.off_ctr = 128;
  q.bytes = align256(q.off_ctr + lay.end * sizeof(unsigned));
  *pl = q;
  return true;
}

thread_local long long g_wait_limit = 0;  // 0: the default

}  // namespace

bool mlp_step_supported(int64_t T, int64_t h, int64_t F, int p) {
  Plan q;
  return plan_step(T, h, F, p, &q);
}

size_t mlp_step_workspace_bytes(int64_t T, int64_t h, int64_t F, int p) {
  Plan q;
  return plan_step(T, h, F, p, &q) ? q.bytes : 0;
}

void set_step_wait_limit(long long polls) { g_wait_limit = polls; }

long long step_wait_polls() {
  // about 0.25 s of polling at the default
  return g_wait_limit > 0 ? g_wait_limit : (g_wait_limit < 0 ? 0 : (1ll << 22));
}

hipError_t launch_mlp_rows(StepParams s, void* workspace, hipStream_t stream) {
  Plan q;
  if (!plan_step(s.T, s.h, s.F, s.p, &q)) return hipErrorInvalidValue;
  char* w = static_cast<char*>(workspace);
  s.err = reinterpret_cast<unsigned*>(w);
  s.clk = reinterpret_cast<unsigned long long*>(w + 64);
  s.ctr = reinterpret_cast<unsigned*>(w + q.off_ctr);
  s.xcds = q.xcds;
  s.rb = q.rb;
  s.rbx = q.rbx;
  if (s.phases < 1 || s.phases > 3) return hipErrorInvalidValue;
  s.units_a = s.phases == 3 ? 2 * q.units_a : q.units_a;
  if (s.phases & 2) {
    if (s.no_dx_sum) s.units_a -= q.rbx * (q.rb / kSumRows);  // the dX sum units
  } else {
    s.no_dx_sum = 0;
  }
  s.spin = step_wait_polls();
  const int cus = device_shape().cus;
  if (q.large)
    hipLaunchKernelGGL(mlp_rows_kernel<RowsLarge>, dim3(cus * RowsLarge::MINB),
                       dim3(RowsLarge::THREADS), 0, stream, s);
  else
    hipLaunchKernelGGL(mlp_rows_kernel<RowsSmall>, dim3(cus * RowsSmall::MINB),
                       dim3(RowsSmall::THREADS), 0, stream, s);
  return hipGetLastError();
}

}  // namespace tpmlp
