"""Benchmark of the tensor-parallel shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2s]

One step is the whole hot path of a workload: for every shard the column-
parallel forward (fc1 with fused bias + GeLU; the QKV projection), the
row-parallel partial (fc2; the output projection), the sum over shards, the
data gradients (fc2's with the fused GeLU derivative), the weight and bias
gradients and the sum of the dX partials. The step is captured once into a
HIP graph and replayed; inputs are resident in HBM before timing starts.

Prints one JSON line for the GPT-2-small TP=2 MLP shard (the headline): TFLOP/s
of the GEMM work (2*M*N*K per product, all shards) over the wall time of
whole steps, the fraction of the MI355X bf16 dense matrix-core peak, a
roofline record for the step's dominant kernel (its own duration measured
with HIP events on its stream) and the float64 CPU oracle timed on a bounded
sample of the same workload. `configs` holds the same record for every other
bf16 workload (attention projections, ~350M layer, 175B-class shard); the
attention workloads also report the whole attention block, with the shard's
attention core between the projections.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % bf16 MFMA peak, TP-MLP shard fwd+bwd, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # dense FP8 matrix-core peak, twice bf16
SPEC_SCLK_MHZ = 2400.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-s", type=float, default=0.25,
                    help="seconds of untimed steps before the warm-up steps (engine clock)")
    ap.add_argument("--workload", default="gpt2s")
    ap.add_argument("--configs", default="attn,gpt350m,gpt175b",
                    help="comma-separated workloads also measured and reported under 'configs'")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="seconds of float64 oracle work for the headline's cpu_baseline "
                         "(the other workloads take a third of it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the recompute and FP8 variants of the MLP steps")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--only-call", default=None,
                    help="profiling aid: comma-separated calls of shard 0 of --workload, each "
                         "launched --steps times")
    ap.add_argument("--per-product", action="store_true",
                    help="profiling aid (with --only-call): the MLP as one call per product "
                         "instead of tp_mlp_step")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="profiling aid (with --only-call): also copy MIB MiB device-to-device "
                         "three times, to scale HBM byte counters")
    return ap.parse_args()


# --------------------------------------------------------------------------- #
# workloads and their calls                                                    #
# --------------------------------------------------------------------------- #
def workload_label(cfg, attn_core=False) -> str:
    parts = []
    if cfg.mlp:
        parts.append(f"MLP (fc1 {cfg.h}x{cfg.F} + GeLU, fc2 {cfg.F}x{cfg.h})")
    if cfg.attn:
        proj = f"QKV {cfg.h}x{cfg.Q}, out-proj {cfg.O}x{cfg.h}"
        parts.append(f"attention block ({proj}, causal core of {cfg.heads // cfg.p} heads x 64)"
                     if attn_core else f"attention projections ({proj})")
    shards = (f"p={cfg.p} shards run serially" if len(cfg.shards) == cfg.p
              else f"shard {cfg.shards[0]} of p={cfg.p} at its real shape")
    return (f"{cfg.name}: TP shard step of {' + '.join(parts)}, fwd+bwd, tokens={cfg.T} "
            f"(micro-batch {cfg.micro_batch} x seq {cfg.seq}), h={cfg.h}, {shards}, "
            f"{cfg.dtype} (fp32 accumulation)")


def attention_core_flops(cfg):
    """Flops of the attention core of one shard, fwd and bwd: the unmasked
    half of the score matrix, 4*L^2*d/2 per sequence and head forward (Q K^T
    and P V), 2.5 times that backward (five products)."""
    H = cfg.heads // cfg.p
    f = 4.0 * cfg.micro_batch * H * cfg.seq * cfg.seq * 64 / 2
    return f, 2.5 * f


class Call:
    def __init__(self, name, fn, flops, nbytes, single, geom=None, post=None):
        self.name, self.fn, self.flops, self.bytes = name, fn, flops, nbytes
        self.single = single  # one kernel launch: its duration is that kernel's
        self.geom = geom or {}
        # the rest of the step, run after the call when it is timed where the
        # step runs it (time_in_step)
        self.post = post


def shard_calls(step, i=0):
    """The calls of shard i's step, each with its GEMM flops and algorithmic
    bytes (every operand read once, every output written once; bf16
    activations, fp32 partials and weight gradients). `single`: the call is
    one kernel launch, so its duration times that kernel alone. Layer
    gradients are timed as the step runs them: one tp_linear_bwd call where
    the layer pairs (without the bias gradient, which the step adds as column
    partials), else the dgrad and wgrad calls."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    cfg, o, inp = step.cfg, step.out, step.inp
    T, h = cfg.T, cfg.h
    e = 2 if cfg.dtype == "bf16" else 4
    calls = []

    def layer(tag, dOut, W, U, In, dIn, dW, k, n, act, din_bytes):
        pr, sk = L.tp_linear_bwd_plan(T, k, n) if cfg.dtype == "bf16" else (0, 1)
        u_bytes = T * k * e if U is not None else 0
        if pr and step.fused_bwd:
            calls.append(Call(
                f"{tag}_bwd_pair",
                lambda: L.tp_linear_bwd(dOut, W, U, In, dIn, dW, None, act=act,
                                        workspace=step.workspace),
                4 * T * k * n, T * n * e + k * n * e + u_bytes + T * k * e + T * k * din_bytes +
                k * n * 4, sk == 1, {"T": T, "k": k, "n": n, "pairing": pr, "splitk": sk}))
        else:
            calls.append(Call(f"{tag}_dgrad",
                              lambda: L.tp_linear_bwd_dgrad(dOut, W, U, dIn, act=act),
                              2 * T * k * n, T * n * e + k * n * e + u_bytes + T * k * din_bytes,
                              True, {"M": T, "N": k, "K": n}))
            wt = L.tp_gemm_plan(k, n, T, allow_split=True) if cfg.dtype == "bf16" else (0, 1, T)
            calls.append(Call(f"{tag}_wgrad",
                              lambda: L.tp_linear_bwd_wgrad(In, dOut, dW, None,
                                                            workspace=step.workspace),
                              2 * T * k * n, T * k * e + T * n * e + k * n * 4, wt[1] == 1,
                              {"M": k, "N": n, "K": T, "tile": wt[0], "splitk": wt[1]}))

    if cfg.mlp and step.step_call:
        # the MLP of every shard in two launches: forward, sums and data
        # gradients (four products per shard); weight gradients (two)
        F, p = cfg.F, cfg.p
        fused = L.tp_mlp_step_plan(T, h, F, p, step.tp_dt)
        fr = p * 4 * 2 * T * h * F
        br = (T * h * e + h * p * F * e + p * F * h * e + T * h * e  # X, A, B, dZ
              + 3 * T * p * F * e + 2 * p * T * h * 4 + 2 * T * h * e  # U, Y, dU; Zp, dXp; Z, dX
              + 3 * T * p * F * e + 2 * p * T * h * 4)  # re-read: Y, U, dU; Zp, dXp
        fw = p * 2 * 2 * T * h * F
        bw = 2 * T * p * F * e + 2 * T * h * e + 2 * p * F * h * 4  # Y, dU; dZ, X; dB, dA
        geom = {"T": T, "h": h, "F": F, "p": p, "fused": fused}
        calls.append(Call("mlp_step_rows", lambda: step.mlp_step("rows"), fr, br, fused, geom,
                          post=lambda: step.mlp_step("wgrad")))
        calls.append(Call("mlp_step_wgrad", lambda: step.mlp_step("wgrad"), fw, bw, fused, geom))
        calls.append(Call("mlp_step", lambda: step.mlp_step(), fr + fw, br + bw, False, geom))
    elif cfg.mlp:
        F = cfg.F
        A_i, B_i = step._col("A", i, F), step._row("B", i, F)
        a_i = step._col("a", i, F) if cfg.has_bias else None
        Y_i = step._y(i)
        calls.append(Call("fc1_fwd",
                          lambda: L.tp_column_linear_fwd(inp["X"], A_i, a_i, Y_i, o[f"U_{i}"],
                                                         act="gelu"),
                          2 * T * h * F, T * h * e + h * F * e + (F * e if a_i is not None else 0)
                          + 2 * T * F * e, True, {"M": T, "N": F, "K": h}))
        calls.append(Call("fc2_fwd", lambda: L.tp_row_linear_fwd_partial(Y_i, B_i, o[f"Zp_{i}"]),
                          2 * T * h * F, T * F * e + F * h * e + T * h * 4, True,
                          {"M": T, "N": h, "K": F}))
        layer("fc2", inp["dZ"], B_i, o[f"U_{i}"], Y_i, o[f"dU_{i}"], o[f"dB_{i}"], F, h, "gelu", e)
        layer("fc1", o[f"dU_{i}"], A_i, None, inp["X"], o[f"dXp_{i}"], o[f"dA_{i}"], h, F, "none",
              4)
    if cfg.attn and step.proj_call:
        # every shard's attention projections: one persistent launch (QKV,
        # the output projection and its sum, dC, the dXq partials and their
        # sum), then the weight gradients (two products). With the core the
        # QKV forward runs per product, the core in between, and the
        # persistent launch twice (output projection with dC; dXq)
        Q, O, p = cfg.Q, cfg.O, cfg.p
        fused = L.tp_attn_proj_step_plan(T, h, Q, O, p, step.tp_dt)
        geom = {"T": T, "h": h, "Q": Q, "O": O, "p": p, "fused": fused}
        f_q, f_o, f_c, f_x = (p * 2 * T * h * Q, p * 2 * T * O * h, p * 2 * T * h * O,
                              p * 2 * T * Q * h)
        fw = p * 2 * T * O * h + p * 2 * T * h * Q
        bw = (T * p * O * e + T * h * e + T * h * e + T * p * Q * e  # C, dZa, X, dQKV
              + p * O * h * 4 + h * p * Q * 4)  # dO, dW
        if not step.attn_core:
            fr = f_q + f_o + f_c + f_x
            br = (T * h * e + h * p * Q * e + p * O * h * e + T * p * O * e + T * h * e
                  + T * p * Q * e  # X, W, Ow, C, dZa, dQKV
                  + T * p * Q * e + T * p * O * e  # QKV, dC
                  + 2 * 2 * p * T * h * 4 + 2 * T * h * e)  # Zpa, dXqp written and read; Za, dXq
            calls.append(Call("attn_proj_rows", lambda: step.proj_step(15), fr, br, fused, geom,
                              post=lambda: step.proj_step(16)))
            calls.append(Call("attn_proj_wgrad", lambda: step.proj_step(16), fw, bw, fused, geom))
            calls.append(Call("attn_proj_step", lambda: step.proj_step(31), fr + fw, br + bw,
                              False, geom))
        else:
            b, Ls, H = cfg.micro_batch, cfg.seq, cfg.heads // cfg.p
            W_i = step._col("W", i, Q)
            calls.append(Call("qkv_fwd",
                              lambda: L.tp_column_linear_fwd(inp["X"], W_i, None, o[f"QKV_{i}"],
                                                             None, act="none"),
                              2 * T * h * Q, T * h * e + h * Q * e + T * Q * e, True,
                              {"M": T, "N": Q, "K": h}))
            br6 = (T * p * O * e + p * O * h * e + T * h * e  # C, Ow, dZa
                   + T * p * O * e + 2 * p * T * h * 4 + T * h * e)  # dC; Zpa written, read; Za
            calls.append(Call("attn_proj_out_dc", lambda: step.proj_step(6), f_o + f_c, br6, fused,
                              geom))
            br8 = T * p * Q * e + h * p * Q * e + 2 * p * T * h * 4 + T * h * e
            calls.append(Call("attn_proj_dx_wgrad", lambda: step.proj_step(24), f_x + fw, br8 + bw,
                              False, geom))
            # the core of every shard's heads in one launch per direction
            ff, fb = attention_core_flops(cfg)
            hd, a = p * H * 64, step.attn
            calls.append(Call("attn_fwd_shards",
                              lambda: L.tp_attention_fwd(a["QKV"], a["C"], a["lse"], b, Ls, H,
                                                         shards=p),
                              p * ff, T * 3 * hd * 2 + T * hd * 2 + b * p * H * Ls * 4, True))
            calls.append(Call("attn_bwd_shards",
                              lambda: L.tp_attention_bwd(a["QKV"], a["C"], a["dC"], a["lse"],
                                                         step.delta, a["dQKV"], b, Ls, H,
                                                         shards=p),
                              p * fb, T * 3 * hd * 2 * 2 + 2 * T * hd * 2 + b * p * H * Ls * 4 * 3,
                              False))
    elif cfg.attn:
        Q, O = cfg.Q, cfg.O
        W_i, Ow_i = step._col("W", i, Q), step._row("Ow", i, O)
        C_i = step._c(i)
        dQKV_i = o[f"dQKV_{i}"] if step.attn_core else step._col("dQKV", i, Q)
        calls.append(Call("qkv_fwd",
                          lambda: L.tp_column_linear_fwd(inp["X"], W_i, None, o[f"QKV_{i}"], None,
                                                         act="none"),
                          2 * T * h * Q, T * h * e + h * Q * e + T * Q * e, True,
                          {"M": T, "N": Q, "K": h}))
        calls.append(Call("out_fwd", lambda: L.tp_row_linear_fwd_partial(C_i, Ow_i, o[f"Zpa_{i}"]),
                          2 * T * O * h, T * O * e + O * h * e + T * h * 4, True,
                          {"M": T, "N": h, "K": O}))
        layer("out", inp["dZa"], Ow_i, None, C_i, o[f"dC_{i}"], o[f"dOw_{i}"], O, h, "none", e)
        layer("qkv", dQKV_i, W_i, None, inp["X"], o[f"dXqp_{i}"], o[f"dW_{i}"], h, Q, "none", 4)
        if step.attn_core:
            b, Ls, H = cfg.micro_batch, cfg.seq, cfg.heads // cfg.p
            ff, fb = attention_core_flops(cfg)
            hd = H * 64
            calls.append(Call("attn_fwd",
                              lambda: L.tp_attention_fwd(o[f"QKV_{i}"], o[f"C_{i}"], o[f"lse_{i}"],
                                                         b, Ls, H),
                              ff, T * 3 * hd * 2 + T * hd * 2 + b * H * Ls * 4, True))
            calls.append(Call("attn_bwd",
                              lambda: L.tp_attention_bwd(o[f"QKV_{i}"], o[f"C_{i}"], o[f"dC_{i}"],
                                                         o[f"lse_{i}"], step.delta,
                                                         o[f"dQKV_{i}"], b, Ls, H),
                              fb, T * 3 * hd * 2 * 2 + 2 * T * hd * 2 + b * H * Ls * 4 * 3,
                              False))
    return calls


# --------------------------------------------------------------------------- #
# timing                                                                       #
# --------------------------------------------------------------------------- #
def time_call(fn, reps):
    """Average device duration (ms) of one call: `reps` back-to-back calls are
    captured into a HIP graph (so host launch cost is off the timed path) and
    the replay is timed with HIP events on the stream it runs on."""
    import torch
    for _ in range(2):
        fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    g.replay()
    e1.record(s)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


def time_in_step(fn, post, reps):
    """Average device duration (ms) of fn where the step runs it: HIP events
    on its stream just before and after it, the rest of the step (post)
    between repetitions. Both parts replay as captured graphs, so the host
    enqueues the next call while the device still runs the previous post."""
    import torch
    graphs = []
    for part in (fn, post):
        for _ in range(2):
            part()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            part()
        graphs.append(g)
    g_fn, g_post = graphs
    for _ in range(3):
        g_fn.replay()
        g_post.replay()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for e0, e1 in ev:
        e0.record(s)
        g_fn.replay()
        e1.record(s)
        g_post.replay()
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / reps


SETTLE_S = 0.25  # untimed steps before the warm-up, set from --settle-s


def time_steps(step, steps, warmup):
    """Wall and event ms per step over `steps` timed steps. Before the
    `warmup` untimed steps, untimed steps run for SETTLE_S seconds: a fresh
    process starts with the engine clock at idle, and its first window of 20
    steps ran 10% slower than every later one (218.5 against 196-198 us on
    the GPT-2-small shard)."""
    import torch
    t_end = time.perf_counter() + SETTLE_S
    while time.perf_counter() < t_end:
        for _ in range(8):
            step.run()
        torch.cuda.synchronize()
    for _ in range(warmup):
        step.run()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(s)
    for _ in range(steps):
        step.run()
    e1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall / steps * 1e3, e0.elapsed_time(e1) / steps


def step_flops(cfg, attn_core=False):
    f = cfg.gemm_flops()
    if attn_core and cfg.attn:
        f += sum(attention_core_flops(cfg)) * len(cfg.shards)
    return f


# --------------------------------------------------------------------------- #
# traffic records (profiles/traffic.json)                                      #
# --------------------------------------------------------------------------- #
def traffic_record(workload, call):
    """HBM bytes per launch of `call` (FETCH_SIZE + WRITE_SIZE from two
    rocprofv3 --pmc runs, scaled by a plain copy) from profiles/traffic.json,
    or None when there is no record or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        recs = json.load(open(path))["records"]
        from tensor_transformer_layer_fwd_amd.prof_summary import source_hash
        rec = recs.get(f"{workload}:{call}")
        if rec and rec.get("source_sha256") == source_hash():
            return rec
    except (OSError, ValueError, KeyError):
        pass
    return None


# --------------------------------------------------------------------------- #
# host facts: clock and CPU                                                    #
# --------------------------------------------------------------------------- #
def sample_sclk(busy_fn, seconds=0.6):
    """Engine clock (MHz) sampled with amdsmi every 20 ms while busy_fn keeps
    the GPU at work; median and range of the samples, or None if amdsmi is
    unavailable."""
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        if not handles:
            return None
        h = handles[0]
    except Exception as exc:  # noqa: BLE001
        log(f"[bench] amdsmi unavailable: {exc}")
        return None
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                samples.append(float(amdsmi.amdsmi_get_clock_info(
                    h, amdsmi.AmdSmiClkType.GFX)["clk"]))
            except Exception:  # noqa: BLE001
                pass
            time.sleep(0.02)

    import torch
    # keep the queue deep (a few ms of replays ahead of the host) so that the
    # GPU never idles between samples
    batch = 64
    th = threading.Thread(target=sampler, daemon=True)
    t0 = time.perf_counter()
    th.start()
    ev = None
    while time.perf_counter() - t0 < seconds:
        for _ in range(batch):
            busy_fn()
        e = torch.cuda.Event()
        e.record()
        if ev is not None:
            ev.synchronize()
        ev = e
    torch.cuda.synchronize()
    stop.set()
    th.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    if not samples:
        return None
    samples.sort()
    return {"median_mhz": samples[len(samples) // 2], "min_mhz": samples[0],
            "max_mhz": samples[-1], "samples": len(samples), "spec_mhz": SPEC_SCLK_MHZ,
            "how": "amdsmi GFX clock every 20 ms while headline step replays run back to back"}


def step_sclk(step):
    """Engine clock of the step's first persistent launch: block 0's shader
    clock (s_memtime) over the 100 MHz real-time clock (s_memrealtime), both
    read at its start and end and left in the workspace; None without it."""
    if not getattr(step, "step_call", False):
        return None
    import torch
    torch.cuda.synchronize()
    c = step.step_ws[64:96].view(torch.int64).cpu().tolist()
    cyc, wall = c[2] - c[0], (c[3] - c[1]) / 100e6
    if cyc <= 0 or wall <= 0:
        return None
    return {"mhz": round(cyc / wall / 1e6, 1), "spec_mhz": SPEC_SCLK_MHZ,
            "window_us": round(wall * 1e6, 2),
            "how": "s_memtime over s_memrealtime across block 0 of the last step's first launch"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or None


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((d.get("num_threads", 1) for d in threadpool_info()
                    if d.get("user_api") == "blas"), default=1)
    except Exception:  # noqa: BLE001
        return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, inputs, seconds, attn_core=False, max_gflop=120.0):
    """The float64 oracle, as it stands, on the host cores, on a bounded sample
    of the workload: whole sequences of it (the first micro-batch entries),
    as many as keep one run under about max_gflop; the 175B-class shard's
    single 2048-token sequence is cut to its first 256 tokens (the MLP acts
    per token). Repeated for about `seconds`; TFLOP/s of the sample's flops."""
    import dataclasses

    import oracle
    from tp_inputs.generate import HostTensor
    per_seq = step_flops(dataclasses.replace(cfg, micro_batch=1), attn_core)
    mb = max(1, min(cfg.micro_batch, int(max_gflop * 1e9 // per_seq)))
    if attn_core and cfg.attn:
        mb = 1  # the oracle's attention core (einsum over all score entries) is the slow part
    seq = cfg.seq
    if mb == 1 and per_seq > max_gflop * 1e9 and not (attn_core and cfg.attn):
        seq = 256
    run_cfg = dataclasses.replace(cfg, micro_batch=mb, seq=seq)
    rows = run_cfg.T
    run_inputs = {k: (HostTensor(v.raw[:rows], v.dtype) if v.raw.shape[0] == cfg.T else v)
                  for k, v in inputs.items()}
    if run_cfg.T == cfg.T:
        sample = "the whole fwd+bwd step"
    elif seq < cfg.seq:
        sample = f"the fwd+bwd step on the first {rows} of {cfg.T} tokens"
    else:
        sample = f"the fwd+bwd step on the first {mb} of {cfg.micro_batch} sequences"
    flops = step_flops(run_cfg, attn_core)
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run_config(run_cfg, run_inputs, attn_core=attn_core)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {
        "value": round(flops * reps / el / 1e12, 5),
        "unit": "TFLOP/s",
        "cores": int(blas_threads()),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{cfg.name}: {sample} (T={run_cfg.T}, h={cfg.h}, shards {list(cfg.shards)}"
                   f"{', attention core included' if attn_core and cfg.attn else ''}) in "
                   f"float64 numpy on the BLAS threads, {reps} run(s) in {el:.1f} s"),
    }


# --------------------------------------------------------------------------- #
# one workload                                                                 #
# --------------------------------------------------------------------------- #
def roofline(cfg, step, reps):
    """Per-call durations of shard 0 and the roofline record of the dominant
    kernel: the slowest call that is a single kernel launch. Its bound is the
    roof that takes longer at peak: GEMM flops at the bf16 peak, or its
    algorithmic bytes at 8 TB/s."""
    per_call, best = {}, None
    for c in shard_calls(step):
        ms = time_call(c.fn, reps)
        per_call[c.name] = {"us": round(ms * 1e3, 2),
                            "tflops": round(c.flops / (ms * 1e-3) / 1e12, 1),
                            "single_kernel": c.single, **c.geom}
        if c.single and (best is None or ms > best[1]):
            best = (c, ms)
    c, ms = best
    how = "back-to-back launches in one graph"
    if c.post is not None:
        ms = time_in_step(c.fn, c.post, reps)
        per_call[c.name]["us_in_step"] = round(ms * 1e3, 2)
        how = "HIP events around the launch inside the step, the rest of the step between"
    s = ms * 1e-3
    tf, gbs = c.flops / s / 1e12, c.bytes / s / 1e9
    hbm = c.bytes / (PEAK_HBM_GBS * 1e9) > c.flops / (PEAK_BF16_TFLOPS * 1e12)
    tr = traffic_record(cfg.name, c.name)
    rec = {"bound": "hbm" if hbm else "mfma", "kernel": c.name,
           "achieved": round(gbs if hbm else tf, 1),
           "peak": PEAK_HBM_GBS if hbm else PEAK_BF16_TFLOPS,
           "unit": "GB/s" if hbm else "TFLOP/s",
           "frac": round(gbs / PEAK_HBM_GBS if hbm else tf / PEAK_BF16_TFLOPS, 4),
           "traffic": round(tr["traffic_bytes_per_launch"]) if tr else None,
           "algorithmic_bytes": c.bytes, "gemm_flops": c.flops, "tflops": round(tf, 1),
           "GB/s": round(gbs, 1), "mfma_frac": round(tf / PEAK_BF16_TFLOPS, 4),
           "us_per_launch": round(ms * 1e3, 2), "timing": how, **c.geom}
    return rec, per_call


def attention_core_record(step, reps):
    """The attention core's launches in the step (the forward, and the
    backward's delta pass with its dK/dV + dQ launch), each against its own
    roofline: the larger of its flops at the bf16 peak (the causal half of the
    scores) and its algorithmic bytes at HBM peak."""
    out = {}
    for c in shard_calls(step):
        if not c.name.startswith(("attn_fwd", "attn_bwd")):
            continue
        ms = time_call(c.fn, reps)
        t_mfma = c.flops / (PEAK_BF16_TFLOPS * 1e12)
        t_hbm = c.bytes / (PEAK_HBM_GBS * 1e9)
        out[c.name] = {"us": round(ms * 1e3, 2), "tflops": round(c.flops / (ms * 1e-3) / 1e12, 1),
                       "algorithmic_bytes": c.bytes, "flops": c.flops,
                       "bound": "hbm" if t_hbm > t_mfma else "mfma",
                       "roofline_us": round(max(t_mfma, t_hbm) * 1e6, 2),
                       "frac": round(max(t_mfma, t_hbm) / (ms * 1e-3), 4)}
    return out


def measure(name, args, inputs=None, attn_core=False, with_roofline=True, cpu_seconds=None):
    import torch
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    cfg = get_config(name)
    if inputs is None:
        log(f"[bench] {name}: drawing inputs (T={cfg.T} h={cfg.h} p={cfg.p})")
        inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, "cuda:0", attn_core=attn_core)
    step.capture()
    wall_ms, ev_ms = time_steps(step, args.steps, args.warmup)
    flops = step_flops(cfg, attn_core)
    tflops = flops / (wall_ms * 1e-3) / 1e12
    log(f"[bench] {workload_label(cfg, attn_core)}: {wall_ms * 1e3:.1f} us/step "
        f"(events {ev_ms * 1e3:.1f}), {tflops:.1f} TFLOP/s = "
        f"{100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")
    rec = {"workload": workload_label(cfg, attn_core), "tflops": round(tflops, 2),
           "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
           "ms_per_step": round(wall_ms, 5), "event_ms_per_step": round(ev_ms, 5),
           "steps": args.steps, "warmup": args.warmup, "settle_s": SETTLE_S,
           "flops_per_step": flops, "gemm_gflop_per_step": round(cfg.gemm_flops() / 1e9, 2)}
    if attn_core:
        rec["attention_core_gflop_per_step"] = round(
            sum(attention_core_flops(cfg)) * len(cfg.shards) / 1e9, 3)
    if with_roofline:
        rec["roofline"], rec["per_call_shard0"] = roofline(cfg, step, args.kernel_reps)
        log(f"[bench] {name} roofline: {json.dumps(rec['roofline'])}")
    if attn_core and cfg.attn:
        rec["attention_core"] = attention_core_record(step, args.kernel_reps)
        log(f"[bench] {name} attention core: {json.dumps(rec['attention_core'])}")
    secs = args.cpu_seconds if cpu_seconds is None else cpu_seconds
    if not args.no_cpu_baseline and secs > 0:
        log(f"[bench] {name}: timing the float64 oracle on the host for ~{secs:.0f} s")
        rec["cpu_baseline"] = cpu_baseline(cfg, inputs, secs, attn_core)
    return cfg, inputs, step, rec


def hbm_passes(cfg, inputs, step, reps):
    """The HBM-bound passes of the headline: the sum over shards (fp32
    partials -> bf16 + bias), the standalone bias + GeLU pass (fp32 U -> bf16 Y,
    an ablation of the epilogue fused into fc1) and, from the counter record,
    the fused fc1 epilogue's written bytes over fc1's duration."""
    import torch
    from tensor_transformer_layer_fwd_amd import _lib as L
    o = step.out
    parts = [o[f"Zp_{i}"] for i in cfg.shards]
    z_out = o["Z"]
    esz = z_out.element_size()
    red_bytes = len(parts) * cfg.T * cfg.h * 4 + cfg.T * cfg.h * esz + \
        (cfg.h * esz if cfg.has_bias else 0)
    red_ms = time_call(lambda: L.tp_reduce_partials(parts, step.inp.get("b"), z_out), reps)
    u32 = torch.randn(cfg.T, cfg.F, device="cuda:0")
    a32 = torch.randn(cfg.F, device="cuda:0")
    ybf = torch.empty(cfg.T, cfg.F, dtype=torch.bfloat16, device="cuda:0")
    gelu_bytes = cfg.T * cfg.F * (4 + 2) + cfg.F * 4
    gelu_ms = time_call(lambda: L.tp_bias_act(u32, a32, ybf, act="gelu"), reps)
    del u32, ybf
    out = {"reduce_partials": {"GB/s": round(red_bytes / (red_ms * 1e-3) / 1e9, 1),
                               "bytes": red_bytes, "us": round(red_ms * 1e3, 2)},
           "bias_gelu_standalone": {"GB/s": round(gelu_bytes / (gelu_ms * 1e-3) / 1e9, 1),
                                    "bytes": gelu_bytes, "us": round(gelu_ms * 1e3, 2)},
           "peak_GB/s": PEAK_HBM_GBS}
    # fc1 as its own product (tp_column_linear_fwd), as the counter record has it
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    own = ShardStep(cfg, inputs, "cuda:0", step_call=False)
    fc1 = next(c for c in shard_calls(own) if c.name == "fc1_fwd")
    fc1_ms = time_call(fc1.fn, reps)
    del own
    tr = traffic_record(cfg.name, "fc1_fwd")
    algo_w = 2 * cfg.T * cfg.F * 2
    out["fc1_fused_epilogue"] = {
        "us": round(fc1_ms * 1e3, 2), "algorithmic_write_bytes": algo_w,
        "algorithmic_write_GB/s": round(algo_w / (fc1_ms * 1e-3) / 1e9, 1),
        "counter_write_bytes": round(tr["write_bytes_per_launch"]) if tr else None,
        "counter_write_GB/s": (round(tr["write_bytes_per_launch"] / (fc1_ms * 1e-3) / 1e9, 1)
                               if tr else None),
        "note": "U_i and Y_i (bf16) written by fc1's epilogue over the whole fc1 kernel's time"}
    return out


def variants(cfg, inputs, args, wall_ms):
    """The headline step with activation recompute, and the MLP steps in FP8."""
    import torch
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    flops = cfg.gemm_flops()
    rs = ShardStep(cfg, inputs, "cuda:0", recompute=True)
    rs.capture()
    r_ms, _ = time_steps(rs, args.steps, args.warmup)
    recompute = {"ms_per_step": round(r_ms, 5), "tflops": round(flops / (r_ms * 1e-3) / 1e12, 1),
                 "vs_stored": round(wall_ms / r_ms, 4),
                 "activation_bytes_saved_per_shard": cfg.T * cfg.F * 2,
                 "split": rs.split_step}
    del rs
    if recompute["split"]:
        # recompute runs the step as its forward and backward calls: the
        # stored step split the same way is the like-for-like reference
        ss = ShardStep(cfg, inputs, "cuda:0", split_step=True)
        ss.capture()
        s_ms, _ = time_steps(ss, args.steps, args.warmup)
        recompute["split_stored_ms_per_step"] = round(s_ms, 5)
        recompute["vs_split_stored"] = round(s_ms / r_ms, 4)
        del ss
    log(f"[bench] {cfg.name} with recompute: {json.dumps(recompute)}")
    fp8 = {}
    for name in (cfg.name, "gpt175b"):
        c8 = get_config(name)
        s8 = ShardStep(c8, inputs if name == cfg.name else make_inputs(c8), "cuda:0", fp8=True)
        s8.capture()
        f_ms, _ = time_steps(s8, args.steps, args.warmup)
        tf8 = c8.gemm_flops() / (f_ms * 1e-3) / 1e12
        fp8[name] = {"ms_per_step": round(f_ms, 5), "tflops": round(tf8, 1),
                     "frac_of_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4)}
        log(f"[bench] {name} FP8 step: {json.dumps(fp8[name])}")
        del s8
        torch.cuda.empty_cache()
    return recompute, fp8


def only_calls(args):
    import torch
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    cfg = get_config(args.workload)
    inputs = make_inputs(cfg)
    steps = {}

    def find(name):
        # the step as the headline runs it, else (attention workloads) the
        # attention block with the core
        for core in (False, True) if cfg.attn else (False,):
            if core not in steps:
                st = ShardStep(cfg, inputs, "cuda:0", attn_core=core,
                               step_call=not args.per_product)
                st.run_eager()
                steps[core] = (st, {c.name: c for c in shard_calls(st)})
            if name in steps[core][1]:
                return steps[core][1][name]
        raise KeyError(f"{args.workload} has no call {name}")

    for name in args.only_call.split(","):
        c = find(name)
        ms = time_call(c.fn, args.steps)
        log(f"[bench] {args.workload} {name}: {ms * 1e3:.2f} us/launch, "
            f"{c.flops / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        print(json.dumps({"workload": args.workload, "call": name, "us_per_launch": ms * 1e3,
                          "tflops": c.flops / (ms * 1e-3) / 1e12, "single_kernel": c.single}))
    if args.calibrate_copy:
        n = args.calibrate_copy * 1024 * 1024 // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.calibrate_copy} MiB three times for counter calibration")


def main():
    global SETTLE_S
    args = parse()
    SETTLE_S = max(0.0, args.settle_s)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the shards of a workload run serially on "
              f"cuda:0 and are summed locally; --gpus {args.gpus} is not supported.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(2)
    if args.only_call:
        only_calls(args)
        return

    cfg, inputs, step, head = measure(args.workload, args, cpu_seconds=0)
    wall_ms = head["ms_per_step"]
    step.run()
    sclk = {"in_kernel": step_sclk(step), "amdsmi": sample_sclk(step.run)}
    log(f"[bench] engine clock under the step: {json.dumps(sclk)}")
    hbm = hbm_passes(cfg, inputs, step, args.kernel_reps) if cfg.mlp and "Z" in step.out else None
    log(f"[bench] HBM passes: {json.dumps(hbm)}")
    recompute = fp8 = None
    if not args.no_variants and cfg.mlp:
        recompute, fp8 = variants(cfg, inputs, args, wall_ms)
    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] {cfg.name}: timing the float64 oracle on the host for "
            f"~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(cfg, inputs, args.cpu_seconds)
    del step
    torch.cuda.empty_cache()

    configs = {}
    for name in [w for w in args.configs.split(",") if w and w != args.workload]:
        c2, in2, s2, rec = measure(name, args, cpu_seconds=args.cpu_seconds / 3)
        del s2
        torch.cuda.empty_cache()
        if c2.attn:
            # the whole attention block: the core between the projections
            _, _, s3, blk = measure(name, args, inputs=in2, attn_core=True,
                                    cpu_seconds=args.cpu_seconds / 3)
            rec["attention_block"] = blk
            del s3
            torch.cuda.empty_cache()
        configs[name] = rec

    rec = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": SETTLE_S,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "frac_of_peak": head["frac_of_peak"],
        "config": {"workload": head["workload"], "tokens": cfg.T, "h": cfg.h, "p": cfg.p,
                   "ffn_shard": cfg.F, "gemm_gflop_per_step": head["gemm_gflop_per_step"]},
        "roofline": head["roofline"],
        "per_call_shard0": head["per_call_shard0"],
        "cpu_baseline": cpu,
        "sclk": sclk,
        "hbm_passes": hbm,
        "recompute": recompute,
        "fp8": fp8,
        "configs": configs,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
