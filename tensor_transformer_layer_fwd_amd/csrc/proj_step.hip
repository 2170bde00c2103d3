// The attention projections of p tensor-parallel shards on one device in one
// persistent launch ("Megatron" page, "Transformer-layer tensor parallelism":
// the QKV projection is column-parallel, QKV_i = X W_i; the output projection
// is row-parallel, Zpa_i = C_i O_i, and the sum over shards Za = sum_i Zpa_i
// stands in for the All-Reduce; the backward is the derivative of the same
// definitions: dC_i = dZa O_i^T, dXqp_i = dQKV_i W_i^T, dXq = sum_i dXqp_i).
//
// Every output here has token rows, so the launch is organised like the MLP
// step's row launch (mlp_step.hip): each XCD owns a slab of T / XCDs token rows
// and drains its own ticket queue of units over those rows, in this order:
//   for each shard i: QKV tiles (bf16), output-projection partial tiles (fp32);
//   for each shard i: dC tiles (bf16);
//   the sum Za = sum_i Zpa_i, in units of 16 rows;
//   for each shard i: dXq partial tiles (fp32);
//   the sum dXq = sum_i dXqp_i.
// The products read only the launch's inputs (C_i and dQKV_i come from the
// attention core or the caller), so only the sums wait: for every shard's
// partial tiles of their row block, counted with the same protocol as the MLP
// step (stores complete, then an agent-scope count; the consumer polls, then
// reads through the XCD's L2). A launch runs any subset of the four stages, in
// the same order: with the attention core between them, a caller runs the QKV
// stage, the core, the output projection, then dC, the core's backward and
// dXq. The weight gradients dO_i = C_i^T dZa and dW_i = X^T dQKV_i read every
// token row; they run after this launch as two products over the stacked
// shards. When they follow in the same call and their launch has room, it
// also runs the dXq sum, and this launch leaves that sum out (no_dx_sum).
#include "step_queue.h"

namespace tpmlp {
namespace {

// Counter layout (unsigned words from s.ctr): the tickets (xcds), the done
// count, the per-row-block counts of output-projection partials [nrb] and of
// dXq partials [nrb].
struct ProjLayout {
  int64_t nrb;
  int64_t ta, da, po, px, end;
  __host__ __device__ ProjLayout(int64_t T, int rb, int xcds) {
    nrb = T / rb;
    ta = 0;
    da = ta + xcds;
    po = da + 1;
    px = po + nrb;
    end = px + nrb;
  }
};

enum ProjKind : int { kPQ = 0, kPO = 1, kPC = 2, kPS1 = 3, kPX = 4, kPS2 = 5 };

template <class C>
__global__ __launch_bounds__(C::THREADS, C::MINB) void proj_rows_kernel(ProjParams s) {
  constexpr int RB = C::RB, TN = C::TN;
  constexpr int SS = RB / kSumRows;  // sum units per row block
  uint8_t* pool = pool_buf<C::POOL>();
  const ProjLayout L(s.T, s.rb, s.xcds);
  const int x = xcc_id() % s.xcds;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    s.clk[0] = clock64();
    s.clk[1] = wall_clock64();
  }
  const int64_t T = s.T, h = s.h, Q = s.Q, O = s.O;
  const int R = s.rbx;
  const int nq = static_cast<int>(Q / TN), nh = static_cast<int>(h / TN),
            no = static_cast<int>(O / TN);
  // sizes of the queue's phases, in queue order (0 for a stage not run)
  const int cq = (s.phases & kProjQkv) ? s.p * R * nq : 0;
  const int co = (s.phases & kProjOut) ? s.p * R * nh : 0;
  const int cc = (s.phases & kProjDc) ? s.p * R * no : 0;
  const int c1 = (s.phases & kProjOut) ? R * SS : 0;
  const int cx = (s.phases & kProjDx) ? s.p * R * nh : 0;
  unsigned* ctr = s.ctr;
  for (;;) {
    const unsigned tk = next_ticket(ctr + L.ta + x, pool);
    if (tk >= static_cast<unsigned>(s.units_a)) break;
    int t = static_cast<int>(tk), kind;
    if (t < cq) {
      kind = kPQ;
    } else if ((t -= cq) < co) {
      kind = kPO;
    } else if ((t -= co) < cc) {
      kind = kPC;
    } else if ((t -= cc) < c1) {
      kind = kPS1;
    } else if ((t -= c1) < cx) {
      kind = kPX;
    } else {
      t -= cx;
      kind = kPS2;
    }
    // t within the phase: (shard i,) row block j, column tile (or sum slice) n
    int i = 0, j = 0, n = 0;
    if (kind == kPS1 || kind == kPS2) {
      j = t / SS;
      n = t % SS;
    } else {
      const int nc = kind == kPQ ? nq : (kind == kPC ? no : nh);
      i = t / (R * nc);
      j = (t % (R * nc)) / nc;
      n = t % nc;
    }
    const int64_t rg = static_cast<int64_t>(x) * R + j;  // global row block
    const int64_t m0 = rg * RB;
    const int64_t n0 = static_cast<int64_t>(n) * TN;
    GemmParams g{};
    g.splitk = 1;
    g.xcds = s.xcds;
    g.M = T;
    switch (kind) {
      case kPQ:  // QKV_i = X W_i
        g.a = s.x;
        g.lda = s.ld_x;
        g.b = bf(s.w) + i * Q;
        g.ldb = s.ld_w;
        g.c = bfw(s.qkv) + i * Q;
        g.ldc = s.ld_qkv;
        g.N = Q, g.K = h, g.k_chunk = h;
        unit_tile<RB, TN, C::WM, C::WN, C::BKN, C::SN, true, false, kEpiBF16, C::POOL>(
            g, m0, n0, static_cast<int>(h / C::BKN));
        break;
      case kPO:  // Zpa_i = C_i O_i
        g.a = bf(s.c) + i * O;
        g.lda = s.ld_c;
        g.b = bf(s.ow) + i * O * s.ld_ow;
        g.ldb = s.ld_ow;
        g.c = s.zp + i * T * h;
        g.ldc = h;
        g.N = h, g.K = O, g.k_chunk = O;
        unit_tile<RB, TN, C::WM, C::WN, C::BKN, C::SN, true, false, kEpiF32, C::POOL>(
            g, m0, n0, static_cast<int>(O / C::BKN));
        signal_count(ctr + L.po + rg);
        break;
      case kPC:  // dC_i = dZa O_i^T
        g.a = s.dz;
        g.lda = s.ld_dz;
        g.b = bf(s.ow) + i * O * s.ld_ow;
        g.ldb = s.ld_ow;
        g.c = bfw(s.dc) + i * O;
        g.ldc = s.ld_dc;
        g.N = O, g.K = h, g.k_chunk = h;
        unit_tile<RB, TN, C::WM, C::WN, C::BKT, C::ST, true, true, kEpiBF16, C::POOL>(
            g, m0, n0, static_cast<int>(h / C::BKT));
        break;
      case kPS1:  // Za = sum_i Zpa_i
        wait_count(ctr + L.po + rg, static_cast<unsigned>(s.p * nh), s.spin, s.err);
        rows_sum_unit(s.zp, T * h, s.p, h, nullptr, s.z, s.ld_z, m0 + n * kSumRows, h);
        break;
      case kPX:  // dXqp_i = dQKV_i W_i^T
        g.a = bf(s.dqkv) + i * Q;
        g.lda = s.ld_dqkv;
        g.b = bf(s.w) + i * Q;
        g.ldb = s.ld_w;
        g.c = s.dxp + i * T * h;
        g.ldc = h;
        g.N = h, g.K = Q, g.k_chunk = Q;
        unit_tile<RB, TN, C::WM, C::WN, C::BKT, C::ST, true, true, kEpiF32, C::POOL>(
            g, m0, n0, static_cast<int>(Q / C::BKT));
        signal_count(ctr + L.px + rg);
        break;
      default:  // kPS2: dXq = sum_i dXqp_i
        wait_count(ctr + L.px + rg, static_cast<unsigned>(s.p * nh), s.spin, s.err);
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

// Queue length per phase set and workspace layout (shapes and device only).
struct ProjPlan {
  bool large;  // 256 x 128 tiles (RowsLarge), else 128 x 128 (RowsSmall)
  int xcds, rb, rbx;
  size_t off_ctr, bytes;
};

bool plan_proj(int64_t T, int64_t h, int64_t Q, int64_t O, int p, ProjPlan* pl) {
  const DeviceShape d = device_shape();
  const int X = d.xcds;
  if (p < 1 || p > kMaxPartials || T < 1 || h < 1 || Q < 1 || O < 1) return false;
  if (T % (static_cast<int64_t>(kRows) * X) || h % 128 || Q % 128 || O % 128) return false;
  // like the MLP step: products of at most about 20 GFLOP
  if (2.0 * T * h * (Q > O ? Q : O) > 2.0e10) return false;
  ProjPlan q{};
  q.xcds = X;
  q.large = T % (static_cast<int64_t>(RowsLarge::RB) * X) == 0 && forced_tile() != kPipe128x128;
  q.rb = q.large ? RowsLarge::RB : RowsSmall::RB;
  q.rbx = static_cast<int>(T / q.rb / X);
  const ProjLayout lay(T, q.rb, X);
  q.off_ctr = 128;
  q.bytes = (q.off_ctr + lay.end * sizeof(unsigned) + 255) / 256 * 256;
  *pl = q;
  return true;
}

template <class C>
int proj_units(const ProjParams& s, int R) {
  const int nq = static_cast<int>(s.Q / C::TN), nh = static_cast<int>(s.h / C::TN),
            no = static_cast<int>(s.O / C::TN), ss = C::RB / kSumRows;
  int u = 0;
  if (s.phases & kProjQkv) u += s.p * R * nq;
  if (s.phases & kProjOut) u += s.p * R * nh + R * ss;
  if (s.phases & kProjDc) u += s.p * R * no;
  if (s.phases & kProjDx) u += s.p * R * nh + (s.no_dx_sum ? 0 : R * ss);
  return u;
}

}  // namespace

bool proj_step_supported(int64_t T, int64_t h, int64_t Q, int64_t O, int p) {
  ProjPlan q;
  return plan_proj(T, h, Q, O, p, &q);
}

size_t proj_step_workspace_bytes(int64_t T, int64_t h, int64_t Q, int64_t O, int p) {
  ProjPlan q;
  return plan_proj(T, h, Q, O, p, &q) ? q.bytes : 0;
}

hipError_t launch_proj_rows(ProjParams s, void* workspace, hipStream_t stream) {
  ProjPlan q;
  if (!plan_proj(s.T, s.h, s.Q, s.O, s.p, &q)) return hipErrorInvalidValue;
  if (s.phases < 1 || s.phases > 15) return hipErrorInvalidValue;
  char* w = static_cast<char*>(workspace);
  s.err = reinterpret_cast<unsigned*>(w);
  s.clk = reinterpret_cast<unsigned long long*>(w + 64);
  s.ctr = reinterpret_cast<unsigned*>(w + q.off_ctr);
  s.xcds = q.xcds;
  s.rb = q.rb;
  s.rbx = q.rbx;
  s.units_a = q.large ? proj_units<RowsLarge>(s, q.rbx) : proj_units<RowsSmall>(s, q.rbx);
  s.spin = step_wait_polls();
  const int cus = device_shape().cus;
  if (q.large)
    hipLaunchKernelGGL(proj_rows_kernel<RowsLarge>, dim3(cus * RowsLarge::MINB),
                       dim3(RowsLarge::THREADS), 0, stream, s);
  else
    hipLaunchKernelGGL(proj_rows_kernel<RowsSmall>, dim3(cus * RowsSmall::MINB),
                       dim3(RowsSmall::THREADS), 0, stream, s);
  return hipGetLastError();
}

}  // namespace tpmlp
