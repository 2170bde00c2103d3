"""Benchmark of the tensor-parallel MLP shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gpt2s]

One step is the whole hot path of a workload: for every shard the column-
parallel fc1 forward with fused bias + GeLU, the row-parallel fc2 partial, the
sum over shards, the fc2 dgrad with the fused GeLU derivative, both wgrads with
bias gradients, the fc1 dgrad and the sum of the dX partials. The step is
captured once into a HIP graph and replayed; inputs are resident in HBM before
timing starts.

Prints one JSON line: TFLOP/s of the GEMM work (2*M*N*K per product, all
shards) over the wall time of whole steps, the fraction of the MI355X bf16
dense matrix-core peak, a roofline record for the dominant kernel (its own
duration measured with HIP events on its stream) and the float64 CPU oracle
timed on a bounded sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s + % bf16 MFMA peak, TP-MLP shard fwd+bwd, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0
PEAK_FP8_TFLOPS = 5033.2  # dense FP8 matrix-core peak, twice bf16


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gpt2s")
    ap.add_argument("--extra", default="gpt175b",
                    help="comma-separated workloads also timed and reported under 'extra'")
    ap.add_argument("--attention", default="attn,gpt350m",
                    help="comma-separated workloads whose shard attention core (forward and "
                         "backward) is timed and reported under 'attention'; empty: none")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=20)
    ap.add_argument("--only-call", default=None,
                    help="profiling aid: comma-separated calls of shard 0, each launched "
                         "--steps times")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="profiling aid (with --only-call): also copy MIB MiB device-to-device "
                         "three times, to scale HBM byte counters")
    return ap.parse_args()


def shard_calls(step, i=0):
    """The per-shard calls of the MLP step as (name, thunk, gemm flops, kernels)."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    cfg, o, inp = step.cfg, step.out, step.inp
    T, h, F = cfg.T, cfg.h, cfg.F
    A_i, B_i = step._col("A", i, F), step._row("B", i, F)
    a_i = step._col("a", i, F) if cfg.has_bias else None
    f = 2 * T * h * F
    return [
        ("fc1_fwd", lambda: L.tp_column_linear_fwd(inp["X"], A_i, a_i, o[f"Y_{i}"], o[f"U_{i}"],
                                                   act="gelu"), f),
        ("fc2_fwd", lambda: L.tp_row_linear_fwd_partial(o[f"Y_{i}"], B_i, o[f"Zp_{i}"]), f),
        ("fc2_dgrad", lambda: L.tp_linear_bwd_dgrad(inp["dZ"], B_i, o[f"U_{i}"], o[f"dU_{i}"],
                                                    act="gelu"), f),
        ("fc2_wgrad", lambda: L.tp_linear_bwd_wgrad(o[f"Y_{i}"], inp["dZ"], o[f"dB_{i}"],
                                                    o.get("db"), workspace=step.workspace), f),
        ("fc1_dgrad", lambda: L.tp_linear_bwd_dgrad(o[f"dU_{i}"], A_i, None, o[f"dXp_{i}"],
                                                    act="none"), f),
        ("fc1_wgrad", lambda: L.tp_linear_bwd_wgrad(inp["X"], o[f"dU_{i}"], o[f"dA_{i}"],
                                                    o.get(f"da_{i}"), workspace=step.workspace),
         f),
    ]


def layer_bwd_calls(step, i=0):
    """Both gradients of each MLP layer of shard i in one tp_linear_bwd call, as
    the step runs them: (name, thunk, gemm flops)."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    cfg, o, inp = step.cfg, step.out, step.inp
    F = cfg.F
    A_i, B_i = step._col("A", i, F), step._row("B", i, F)
    f = 4 * cfg.T * cfg.h * F
    return [
        ("fc2_bwd", lambda: L.tp_linear_bwd(inp["dZ"], B_i, o[f"U_{i}"], o[f"Y_{i}"], o[f"dU_{i}"],
                                            o[f"dB_{i}"], o.get("db"), act="gelu",
                                            workspace=step.workspace), f),
        ("fc1_bwd", lambda: L.tp_linear_bwd(o[f"dU_{i}"], A_i, None, inp["X"], o[f"dXp_{i}"],
                                            o[f"dA_{i}"], o.get(f"da_{i}"), act="none",
                                            workspace=step.workspace), f),
    ]


def pair_calls(step, i=0):
    """The layers of shard i whose fused backward is a paired kernel launch,
    each called without its bias gradient, which the step adds as column
    partials and a short second pass: (name, thunk, gemm flops, (T, k, n,
    pairing, splitk)). With splitk > 1 the call adds a fix-up launch (in the
    step it rides in the next paired launch), so only splitk == 1 calls time
    the paired kernel alone."""
    from tensor_transformer_layer_fwd_amd import _lib as L
    cfg, o, inp = step.cfg, step.out, step.inp
    if not (cfg.mlp and step.fused_bwd and cfg.dtype == "bf16"):
        return []
    T, h, F = cfg.T, cfg.h, cfg.F
    A_i, B_i = step._col("A", i, F), step._row("B", i, F)
    f = 4 * T * h * F
    out = []
    for name, k, n, fn in (
            ("fc2_bwd_pair", F, h,
             lambda: L.tp_linear_bwd(inp["dZ"], B_i, o[f"U_{i}"], o[f"Y_{i}"], o[f"dU_{i}"],
                                     o[f"dB_{i}"], None, act="gelu", workspace=step.workspace)),
            ("fc1_bwd_pair", h, F,
             lambda: L.tp_linear_bwd(o[f"dU_{i}"], A_i, None, inp["X"], o[f"dXp_{i}"],
                                     o[f"dA_{i}"], None, act="none", workspace=step.workspace))):
        pr, sk = L.tp_linear_bwd_plan(T, k, n)
        if pr:
            out.append((name, fn, f, (T, k, n, pr, sk)))
    return out


def gemm_call_bytes(cfg, name):
    """Algorithmic HBM bytes of one single-kernel call of the bf16 MLP step:
    every operand read once, every output written once (bf16 activations, fp32
    partials and weight gradients)."""
    T, h, F, e = cfg.T, cfg.h, cfg.F, 2
    return {
        "fc1_fwd": T * h * e + h * F * e + (F * e if cfg.has_bias else 0) + 2 * T * F * e,
        "fc2_fwd": T * F * e + F * h * e + T * h * 4,
        "fc2_dgrad": T * h * e + F * h * e + 2 * T * F * e,
        "fc1_dgrad": T * F * e + h * F * e + T * h * 4,
        # both products of a layer: the shared dOut read once, dW in fp32
        "fc2_bwd_pair": T * h * e + F * h * e + 3 * T * F * e + F * h * 4,
        "fc1_bwd_pair": T * F * e + h * F * e + T * h * e + T * h * 4 + h * F * 4,
    }[name]


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


def time_steps(step, steps, warmup):
    import torch
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


def run_workload(name, steps, warmup):
    from tensor_transformer_layer_fwd_amd.shard import ShardStep
    from tp_inputs import get_config, make_inputs
    cfg = get_config(name)
    log(f"[bench] {name}: drawing inputs (T={cfg.T} h={cfg.h} p={cfg.p})")
    inputs = make_inputs(cfg)
    step = ShardStep(cfg, inputs, "cuda:0")
    step.capture()
    log(f"[bench] {name}: graph captured; timing {steps} steps after {warmup} warm-up")
    wall_ms, ev_ms = time_steps(step, steps, warmup)
    flops = cfg.gemm_flops()
    tflops = flops / (wall_ms * 1e-3) / 1e12
    return cfg, inputs, step, wall_ms, ev_ms, flops, tflops


def measured_traffic(call):
    """HBM bytes per launch of `call` from profiles/traffic.json (two rocprofv3
    --pmc runs, FETCH_SIZE and WRITE_SIZE, scaled by a plain copy), or None when
    the record is for another call or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))
        from tensor_transformer_layer_fwd_amd.prof_summary import source_hash
        if rec.get("call") == call and rec.get("source_sha256") == source_hash():
            return round(float(rec["traffic_bytes_per_launch"]))
    except (OSError, ValueError, KeyError):
        pass
    return None


def time_attention(name, reps, with_oracle):
    """The attention core of one shard of `name` (its micro-batch x seq tokens
    and the shard's heads of 64), causal, forward and backward, on N(0,1)
    bf16 inputs. Flops count the unmasked half of the score matrix: 4*L^2*d/2
    per sequence and head forward (Q K^T and P V), 2.5x that backward (five
    products). Algorithmic bytes: every tensor read once and written once."""
    import numpy as np
    import torch
    import tensor_transformer_layer_fwd_amd as tp
    from tp_inputs import get_config
    cfg = get_config(name)
    b, L, H = cfg.micro_batch, cfg.seq, cfg.Q // 192
    T, hd = b * L, H * 64
    g = torch.Generator(device="cuda:0").manual_seed(1234)
    x = torch.randn(T, 3 * hd, device="cuda:0", generator=g).to(torch.bfloat16)
    dC = torch.randn(T, hd, device="cuda:0", generator=g).to(torch.bfloat16)
    C = torch.empty(T, hd, dtype=torch.bfloat16, device="cuda:0")
    dx = torch.empty_like(x)
    lse = torch.empty(b * H * L, device="cuda:0")
    delta = torch.empty_like(lse)
    fwd_ms = time_call(lambda: tp.tp_attention_fwd(x, C, lse, b, L, H), reps)
    bwd_ms = time_call(lambda: tp.tp_attention_bwd(x, C, dC, lse, delta, dx, b, L, H), reps)
    f_fwd = 4.0 * b * H * L * L * 64 / 2
    f_bwd = 2.5 * f_fwd
    by_fwd = T * 3 * hd * 2 + T * hd * 2 + b * H * L * 4
    by_bwd = T * 3 * hd * 2 + 2 * T * hd * 2 + b * H * L * 4 * 3 + T * 3 * hd * 2
    rec = {"batch": b, "seq": L, "heads": H, "head_dim": 64, "causal": True}
    for tag, ms, f, by in (("fwd", fwd_ms, f_fwd, by_fwd), ("bwd", bwd_ms, f_bwd, by_bwd)):
        t_roof = max(f / (PEAK_BF16_TFLOPS * 1e12), by / (PEAK_HBM_GBS * 1e9))
        rec[tag] = {"us": round(ms * 1e3, 2), "tflops": round(f / (ms * 1e-3) / 1e12, 1),
                    "gflop": round(f / 1e9, 3), "bytes": by,
                    "roofline_us": round(t_roof * 1e6, 2),
                    "frac_of_roofline": round(t_roof / (ms * 1e-3), 4)}
    if with_oracle:
        from oracle.attention import attention_core_bwd, attention_core_fwd
        xs = x.float().cpu().numpy().astype(np.float64)
        dcs = dC.float().cpu().numpy().astype(np.float64)
        t0 = time.perf_counter()
        attention_core_fwd(xs, b, L, H, 64, True)
        attention_core_bwd(xs, dcs, b, L, H, 64, True)
        rec["cpu_oracle_fwd_bwd_ms"] = round((time.perf_counter() - t0) * 1e3, 1)
    del x, dC, C, dx, lse, delta
    torch.cuda.empty_cache()
    return rec


def cpu_baseline(cfg, inputs, seconds):
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max((d.get("num_threads", 1) for d in threadpool_info()
                       if d.get("user_api") == "blas"), default=1)
    except Exception:  # threadpoolctl missing: report the affinity mask size
        threads = len(os.sched_getaffinity(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.run_config(cfg, inputs)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 50:
            break
    return {
        "value": cfg.gemm_flops() * reps / el / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"{cfg.name}: the whole fwd+bwd step (T={cfg.T}, h={cfg.h}, all {cfg.p} "
                   f"shards) in float64 numpy, {reps} run(s) in {el:.1f} s"),
    }


def main():
    args = parse()
    from tp_inputs import get_config, make_inputs
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
        from tensor_transformer_layer_fwd_amd.shard import ShardStep
        from tp_inputs import get_config, make_inputs
        cfg = get_config(args.workload)
        step = ShardStep(cfg, make_inputs(cfg), "cuda:0")
        step.run_eager()
        calls = {n: (fn, f) for n, fn, f in shard_calls(step)}
        calls.update({n: (fn, f) for n, fn, f, _ in pair_calls(step)})
        for name in args.only_call.split(","):
            fn, f = calls[name]
            ms = time_call(fn, args.steps)
            log(f"[bench] {args.workload} {name}: {ms * 1e3:.2f} us/launch, "
                f"{f / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
            print(json.dumps({"workload": args.workload, "call": name,
                              "us_per_launch": ms * 1e3, "tflops": f / (ms * 1e-3) / 1e12}))
        if args.calibrate_copy:
            n = args.calibrate_copy * 1024 * 1024 // 4
            src = torch.ones(n, device="cuda:0")
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
            log(f"[bench] copied {args.calibrate_copy} MiB three times for counter calibration")
        return

    cfg, inputs, step, wall_ms, ev_ms, flops, tflops = run_workload(
        args.workload, args.steps, args.warmup)
    log(f"[bench] {cfg.name}: {wall_ms * 1e3:.1f} us/step (events {ev_ms * 1e3:.1f}), "
        f"{tflops:.1f} TFLOP/s = {100 * tflops / PEAK_BF16_TFLOPS:.1f}% of bf16 peak")

    # per-call durations of shard 0 (HIP events on the launch stream)
    kernels = {}
    for name, fn, f in shard_calls(step):
        ms = time_call(fn, args.kernel_reps)
        kernels[name] = {"us": round(ms * 1e3, 2), "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
    gemm_sum_us = sum(v["us"] for v in kernels.values()) * len(cfg.shards)
    # each layer's two gradients as the step runs them: one tp_linear_bwd call
    layer_bwd = {}
    for name, fn, f in layer_bwd_calls(step):
        ms = time_call(fn, args.kernel_reps)
        layer_bwd[name] = {"us": round(ms * 1e3, 2), "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
    # dominant kernel: the slowest single-kernel launch the step makes that a
    # call can time alone. A layer whose fused backward is a paired launch
    # contributes that kernel when its weight gradient is not split (a split
    # adds a fix-up launch to the call; in the step the fix-up rides in the
    # next paired launch). A layer that does not pair runs its data gradient
    # as a kernel of its own (its weight gradient call also launches a
    # split-K fix-up and the bias column sums)
    flops_of = {name: f for name, _, f in shard_calls(step)}
    pair_geom = {}
    for name, fn, f, geom in pair_calls(step):
        ms = time_call(fn, args.kernel_reps)
        kernels[name] = {"us": round(ms * 1e3, 2), "tflops": round(f / (ms * 1e-3) / 1e12, 1),
                         "pairing": geom[3], "splitk": geom[4]}
        flops_of[name], pair_geom[name] = f, geom
    single = ["fc1_fwd", "fc2_fwd"]
    for layer in ("fc2", "fc1"):
        geom = pair_geom.get(f"{layer}_bwd_pair")
        if geom is None:
            single.append(f"{layer}_dgrad")
        elif geom[4] == 1:
            single.append(f"{layer}_bwd_pair")
    dom = max(single, key=lambda k: kernels[k]["us"])
    dom_flops = flops_of[dom]
    dom_bytes = gemm_call_bytes(cfg, dom)
    dom_s = kernels[dom]["us"] * 1e-6
    dom_tf = dom_flops / dom_s / 1e12
    dom_gbs = dom_bytes / dom_s / 1e9
    # the roof that takes longer at peak bounds the kernel
    hbm_bound = dom_bytes / (PEAK_HBM_GBS * 1e9) > dom_flops / (PEAK_BF16_TFLOPS * 1e12)
    from tensor_transformer_layer_fwd_amd import _lib as L
    if dom in pair_geom:
        T_, k_, n_, pr_, sk_ = pair_geom[dom]
        dom_gemm = {"T": T_, "k": k_, "n": n_, "pairing": pr_, "splitk": sk_,
                    "us_per_launch": kernels[dom]["us"]}
    else:
        M_, N_, K_ = {"fc1_fwd": (cfg.T, cfg.F, cfg.h), "fc2_fwd": (cfg.T, cfg.h, cfg.F),
                      "fc2_dgrad": (cfg.T, cfg.F, cfg.h), "fc1_dgrad": (cfg.T, cfg.h, cfg.F)}[dom]
        dom_gemm = {"M": M_, "N": N_, "K": K_, "tile": L.tp_gemm_plan(M_, N_, K_)[0],
                    "us_per_launch": kernels[dom]["us"]}
    log(f"[bench] per-call: {json.dumps(kernels)}")

    # HBM-bound passes: the sum over shards (fp32 partials -> bf16 + bias) and
    # the standalone bias + GeLU pass (fp32 U -> bf16 Y) over one shard's [T, F]
    from tensor_transformer_layer_fwd_amd import _lib as L
    o = step.out
    parts = [o[f"Zp_{i}"] for i in cfg.shards]
    z_out = o.get("Z")
    if len(parts) < cfg.p or z_out is None:
        # a workload that runs a subset of its shards: time the sum over all p
        # partials with stand-in buffers of the same shape (zero-filled)
        parts += [torch.zeros_like(parts[0]) for _ in range(cfg.p - len(parts))]
        z_out = torch.empty(cfg.T, cfg.h, dtype=step.dt, device="cuda:0")
    esz = z_out.element_size()
    red_bytes = len(parts) * cfg.T * cfg.h * 4 + cfg.T * cfg.h * esz + (cfg.h * esz if cfg.has_bias else 0)
    red_ms = time_call(lambda: L.tp_reduce_partials(parts, step.inp.get("b"), z_out),
                       args.kernel_reps)
    del parts, z_out
    u32 = torch.randn(cfg.T, cfg.F, device="cuda:0")
    a32 = torch.randn(cfg.F, device="cuda:0")
    ybf = torch.empty(cfg.T, cfg.F, dtype=torch.bfloat16, device="cuda:0")
    gelu_bytes = cfg.T * cfg.F * (4 + 2) + cfg.F * 4
    gelu_ms = time_call(lambda: L.tp_bias_act(u32, a32, ybf, act="gelu"), args.kernel_reps)
    hbm = {"reduce_partials": {"GB/s": round(red_bytes / (red_ms * 1e-3) / 1e9, 1),
                               "bytes": red_bytes, "us": round(red_ms * 1e3, 2)},
           "bias_gelu": {"GB/s": round(gelu_bytes / (gelu_ms * 1e-3) / 1e9, 1),
                         "bytes": gelu_bytes, "us": round(gelu_ms * 1e3, 2)},
           "peak_GB/s": PEAK_HBM_GBS}
    log(f"[bench] HBM passes: {json.dumps(hbm)}")
    del u32, ybf

    # the same step with activation recompute: Y_i is not kept across the
    # step but recomputed from U_i in the fc2 dgrad epilogue
    recompute = None
    if cfg.mlp:
        from tensor_transformer_layer_fwd_amd.shard import ShardStep
        rs = ShardStep(cfg, inputs, "cuda:0", recompute=True)
        rs.capture()
        r_ms, _ = time_steps(rs, args.steps, args.warmup)
        esz = 2 if cfg.dtype == "bf16" else 4
        recompute = {"ms_per_step": round(r_ms, 5), "tflops": round(flops / (r_ms * 1e-3) / 1e12, 1),
                     "vs_stored": round(wall_ms / r_ms, 4),
                     "activation_bytes_saved_per_shard": cfg.T * cfg.F * esz}
        log(f"[bench] {cfg.name} with recompute: {json.dumps(recompute)}")
        del rs
        torch.cuda.empty_cache()

    # the same MLP step with every product in FP8 (E4M3 / E5M2, per-tensor
    # current scaling, quantisation passes inside the timed step)
    fp8 = {}
    for name in [args.workload] + [w for w in args.extra.split(",") if w and w != args.workload]:
        c8 = get_config(name)
        if not (c8.mlp and not c8.attn and c8.dtype == "bf16"):
            continue
        from tensor_transformer_layer_fwd_amd.shard import ShardStep
        s8 = ShardStep(c8, inputs if name == args.workload else make_inputs(c8), "cuda:0",
                       fp8=True)
        s8.capture()
        f_ms, _ = time_steps(s8, max(5, args.steps // 5), 3)
        tf8 = c8.gemm_flops() / (f_ms * 1e-3) / 1e12
        fp8[name] = {"ms_per_step": round(f_ms, 5), "tflops": round(tf8, 1),
                     "frac_of_fp8_peak": round(tf8 / PEAK_FP8_TFLOPS, 4)}
        log(f"[bench] {name} FP8 step: {json.dumps(fp8[name])}")
        del s8
        torch.cuda.empty_cache()

    extra = {}
    for name in [w for w in args.extra.split(",") if w and w != args.workload]:
        c2, _, s2, w2, e2, f2, t2 = run_workload(name, max(5, args.steps // 5), 3)
        k2 = {}
        for n, fn, f in shard_calls(s2):
            ms = time_call(fn, 5)
            k2[n] = {"us": round(ms * 1e3, 1), "tflops": round(f / (ms * 1e-3) / 1e12, 1)}
        extra[name] = {"tflops": round(t2, 1), "frac_of_peak": round(t2 / PEAK_BF16_TFLOPS, 4),
                       "ms_per_step": round(w2, 4), "gemm_gflop": round(f2 / 1e9, 2),
                       "per_call": k2}
        log(f"[bench] {name}: {w2 * 1e3:.1f} us/step, {t2:.1f} TFLOP/s; per-call {k2}")
        del s2
        torch.cuda.empty_cache()

    attention = {}
    for name in [w for w in args.attention.split(",") if w]:
        attention[name] = time_attention(name, args.kernel_reps, not args.no_cpu_baseline)
        log(f"[bench] attention core {name}: {json.dumps(attention[name])}")

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] timing the float64 oracle on the host for ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(cfg, inputs, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "config": {"workload": f"{cfg.name}: GPT-2-small TP=2 MLP shard step, fwd+bwd, "
                               f"tokens={cfg.T} (micro-batch {cfg.micro_batch} x seq {cfg.seq}), "
                               f"h={cfg.h}, p={cfg.p} shards run serially",
                   "tokens": cfg.T, "h": cfg.h, "p": cfg.p, "ffn_shard": cfg.F,
                   "gemm_gflop_per_step": round(flops / 1e9, 2)},
        "roofline": {"bound": "hbm" if hbm_bound else "mfma", "kernel": dom,
                     "achieved": round(dom_gbs if hbm_bound else dom_tf, 1),
                     "peak": PEAK_HBM_GBS if hbm_bound else PEAK_BF16_TFLOPS,
                     "unit": "GB/s" if hbm_bound else "TFLOP/s",
                     "frac": round(dom_gbs / PEAK_HBM_GBS if hbm_bound
                                   else dom_tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(dom),
                     "algorithmic_bytes": dom_bytes, "gemm_flops": dom_flops,
                     "tflops": round(dom_tf, 1),
                     "mfma_frac": round(dom_tf / PEAK_BF16_TFLOPS, 4),
                     "gemm": dom_gemm},
        "per_call_shard0": kernels,
        "gemm_calls_sum_us": round(gemm_sum_us, 1),
        "layer_bwd_shard0": layer_bwd,
        "hbm_passes": hbm,
        "cpu_baseline": cpu,
        "extra": extra,
        "attention": attention,
        "recompute": recompute,
        "fp8": fp8,
    }
    print(json.dumps(rec))


if __name__ == "__main__":
    main()
