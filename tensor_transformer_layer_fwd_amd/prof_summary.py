"""Summaries of rocprofv3 output for the committed profiles.

    python -m tensor_transformer_layer_fwd_amd.prof_summary stats KERNEL_STATS_CSV \
        --cmd "the profiled command" [--out profiles/NAME.txt]
    python -m tensor_transformer_layer_fwd_amd.prof_summary traffic \
        --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --kernel SUBSTRING \
        --workload NAME --call NAME [--grid GRID_SIZE] --copy-mib MIB \
        --cmd-fetch "..." --cmd-write "..." [--out profiles/traffic.json]
    python -m tensor_transformer_layer_fwd_amd.prof_summary mfma COUNTER_CSV --cmd "..." \
        [--sclk-mhz MHZ] [--out profiles/NAME.txt]
    python -m tensor_transformer_layer_fwd_amd.prof_summary stalls COUNTER_CSV ... \
        --cmd "..." ... [--kernel SUBSTRING] [--sclk-mhz MHZ] [--out profiles/NAME.txt]

`traffic` converts FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of one kernel into
HBM bytes per launch, scaled by what the same counters read for a plain device
copy of known size run in the same process (bench.py --calibrate-copy), and
records it under "workload:call" in profiles/traffic.json with a hash of the
pipelined GEMM sources, so that bench.py reports the figure only while the
kernels are unchanged.

`mfma` turns SQ_VALU_MFMA_BUSY_CYCLES into the fraction of the matrix cores'
cycles a dispatch kept busy. The counter adds, over every SIMD, the cycles each
MFMA instruction occupies its unit (32 per v_mfma_f32_32x32x16_bf16: 32768
flops at 1024 flops per clock per SIMD). The cycles the units had are SIMDs x
the dispatch's duration (its own start and end timestamps in the counter run)
x the engine clock: at the 2.4 GHz spec clock the fraction equals achieved
flops over the spec peak; at the measured engine clock (--sclk-mhz) it is the
utilisation of the clock the part held, never below the former.
GRBM_GUI_ACTIVE is not used: summed over the XCDs and divided by their number
it gave 2.69 GHz over a 35.7 us dispatch, above the part's highest clock, so its
window is wider than the dispatch.

`stalls` merges counter passes of one command (each pass a run of its own) per
kernel and grid and reports medians over dispatches: MFMA busy as above; the
wave-cycle fractions spent waiting for anything (SQ_WAIT_ANY), for an
instruction's operands or issue (SQ_WAIT_INST_ANY) and for LDS issue
(SQ_WAIT_INST_LDS), all over SQ_WAVE_CYCLES (same quad-cycle units); LDS bank
conflict cycles over LDS-active cycles; the derived VmemLatency and LdsLatency
(cycles from issue to completion, averaged over instructions); the L2 hit rate
TCC_HIT / (TCC_HIT + TCC_MISS); and the average latency of L2 misses
(TCC_EA0_RDREQ_LEVEL / TCC_EA0_RDREQ, cycles).
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import os
import statistics

PKG = os.path.dirname(os.path.abspath(__file__))


# Sources of the pipelined bf16 GEMM kernels, of the fused step's persistent
# launch and of their tile choice: the kernels whose HBM traffic
# profiles/traffic.json records.
GEMM_SOURCES = ("gemm_bf16_pipe.hip", "gemm_tile.h", "mlp_step.hip", "proj_step.hip",
                "step_queue.h", "device_common.h", "internal.h", "colsum_device.h", "plan.hip")


def source_hash() -> str:
    """sha256 over the pipelined GEMM sources (the public header declares the
    entry points only; the kernels do not include it)."""
    h = hashlib.sha256()
    csrc = os.path.join(PKG, "csrc")
    files = [os.path.join(csrc, f) for f in GEMM_SOURCES]
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _short(name: str) -> str:
    name = name.replace("tpmlp::(anonymous namespace)::", "").replace("(tpmlp::GemmParams)", "")
    return name if len(name) <= 120 else name[:117] + "..."


def cmd_stats(a):
    rows = list(csv.DictReader(open(a.csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows)
    lines = [f"# rocprofv3 kernel statistics", f"# command: {a.cmd}", "",
             f"{'calls':>6} {'avg_us':>9} {'min_us':>9} {'max_us':>9} {'share':>7}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:9.2f} "
                     f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f} "
                     f"{100 * float(r['TotalDurationNs']) / total:6.2f}%  {_short(r['Kernel_Name'] if 'Kernel_Name' in r else r['Name'])}")
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    print(text)


def _per_dispatch(path):
    d = collections.OrderedDict()
    for r in csv.DictReader(open(path)):
        key = (int(r["Dispatch_Id"]), r["Kernel_Name"], int(r["Grid_Size"]))
        d.setdefault(key, collections.Counter())[r["Counter_Name"]] += float(r["Counter_Value"])
    return d


def _kernel_value(d, counter, substr, grid):
    vals = [c[counter] for (did, name, g), c in d.items()
            if substr in name and (grid is None or g == grid)]
    if not vals:
        raise SystemExit(f"no dispatch of {substr!r} (grid {grid}) in the counter file")
    return statistics.median(vals), len(vals)


def _copy_value(d, counter):
    vals = [c[counter] for (did, name, g), c in d.items() if "copy" in name.lower() or
            "elementwise" in name.lower()]
    return max(vals) if vals else None


def cmd_traffic(a):
    f = _per_dispatch(a.fetch)
    w = _per_dispatch(a.write)
    fk, nf = _kernel_value(f, "FETCH_SIZE", a.kernel, a.grid)
    wk, nw = _kernel_value(w, "WRITE_SIZE", a.kernel, a.grid)
    copy_bytes = a.copy_mib * 1024 * 1024
    fc, wc = _copy_value(f, "FETCH_SIZE"), _copy_value(w, "WRITE_SIZE")
    f_scale = copy_bytes / (fc * 1024) if fc else 1.0
    w_scale = copy_bytes / (wc * 1024) if wc else 1.0
    rec = {
        "workload": a.workload, "call": a.call, "kernel": a.kernel, "grid": a.grid,
        "fetch_kib_per_dispatch": fk, "write_kib_per_dispatch": wk, "dispatches": [nf, nw],
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": fc, "write_kib": wc,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "fetch_bytes_per_launch": fk * 1024 * f_scale,
        "write_bytes_per_launch": wk * 1024 * w_scale,
        "traffic_bytes_per_launch": fk * 1024 * f_scale + wk * 1024 * w_scale,
        "source_sha256": source_hash(),
        "commands": {"fetch": a.cmd_fetch, "write": a.cmd_write},
    }
    out = {"records": {}}
    if a.out and os.path.exists(a.out):
        try:
            out = json.load(open(a.out))
            out.setdefault("records", {})
        except ValueError:
            out = {"records": {}}
    out["records"][f"{a.workload}:{a.call}"] = rec
    text = json.dumps(out, indent=1)
    if a.out:
        open(a.out, "w").write(text + "\n")
    print(json.dumps(rec, indent=1))


SIMDS = 1024  # 256 CUs x 4 SIMDs on MI355X
SPEC_MHZ = 2400.0


def mfma_rows(path, sclk_mhz=None):
    """(kernel, grid, dispatches, median duration us, median busy cycles,
    busy at the spec clock, busy at sclk_mhz or None) per kernel and grid."""
    dur = collections.defaultdict(list)
    cyc = collections.defaultdict(list)
    seen = set()
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] != "SQ_VALU_MFMA_BUSY_CYCLES":
            continue
        key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
        did = int(r["Dispatch_Id"])
        if (did, key) in seen:
            continue
        seen.add((did, key))
        dur[key].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
        cyc[key].append(float(r["Counter_Value"]))
    rows = []
    for key in dur:
        d, c = statistics.median(dur[key]), statistics.median(cyc[key])
        if d <= 0:
            continue
        spec = c / (SIMDS * d * 1e-6 * SPEC_MHZ * 1e6)
        at = c / (SIMDS * d * 1e-6 * sclk_mhz * 1e6) if sclk_mhz else None
        rows.append((key[0], key[1], len(dur[key]), d, c, spec, at))
    rows.sort(key=lambda r: -r[4] * 1.0)
    return rows


def cmd_mfma(a):
    rows = mfma_rows(a.csv, a.sclk_mhz)
    lines = ["# rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES",
             f"# command: {a.cmd}",
             "# busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x dispatch duration x clock);",
             f"# busy_spec at the {SPEC_MHZ:.0f} MHz spec clock (= achieved flops / spec peak)",
             (f"# busy_sclk at the measured engine clock ({a.sclk_mhz:.0f} MHz)" if a.sclk_mhz
              else "# busy_sclk: no measured clock given"),
             "",
             f"{'dispatches':>10} {'dur_us':>9} {'busy_cycles':>13} {'busy_spec':>9} "
             f"{'busy_sclk':>9}  kernel (grid)"]
    for name, g, n, d, c, spec, at in rows:
        if c == 0:
            continue
        ats = f"{100 * at:8.1f}%" if at is not None else f"{'-':>9}"
        lines.append(f"{n:10d} {d:9.2f} {c:13.0f} {100 * spec:8.1f}% {ats}  {name} ({g})")
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    print(text)


def _dispatches(path):
    """{(kernel, grid, dispatch): {counter: value, "dur_us": duration}}."""
    d = collections.defaultdict(dict)
    for r in csv.DictReader(open(path)):
        name = r["Kernel_Name"].replace("tpmlp::(anonymous namespace)::", "")
        name = name.replace("(tpmlp::GemmParams)", "")
        key = (name, int(r["Grid_Size"]), int(r["Dispatch_Id"]))
        d[key][r["Counter_Name"]] = float(r["Counter_Value"])
        d[key]["dur_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
    return d


def cmd_stalls(a):
    per = collections.defaultdict(lambda: collections.defaultdict(list))
    for path in a.csv:
        for (name, grid, _), vals in _dispatches(path).items():
            if a.kernel and a.kernel not in name:
                continue
            for c, v in vals.items():
                per[(name, grid)][c].append(v)

    def med(vals, c):
        return statistics.median(vals[c]) if vals.get(c) else None

    def ratio(vals, num, den):
        n, d = med(vals, num), med(vals, den)
        return n / d if n is not None and d else None

    lines = ["# rocprofv3 --pmc passes of one command (one pass per run), medians over dispatches",
             *[f"# command: {c}" for c in a.cmd],
             f"# mfma: SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x dispatch duration x "
             f"{a.sclk_mhz or SPEC_MHZ:.0f} MHz)",
             "# wait_any, wait_inst, wait_lds: SQ_WAIT_ANY, SQ_WAIT_INST_ANY, SQ_WAIT_INST_LDS "
             "over SQ_WAVE_CYCLES",
             "# bank: SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS; vmem_lat, lds_lat: VmemLatency, "
             "LdsLatency (cycles)",
             "# l2_hit: TCC_HIT / (TCC_HIT + TCC_MISS); miss_lat: TCC_EA0_RDREQ_LEVEL / "
             "TCC_EA0_RDREQ (cycles)",
             ""]
    hdr = ["dur_us", "mfma", "wait_any", "wait_inst", "wait_lds", "bank", "vmem_lat", "lds_lat",
           "l2_hit", "miss_lat"]
    lines.append(" ".join(f"{h:>9}" for h in hdr) + "  kernel (grid)")
    clk = (a.sclk_mhz or SPEC_MHZ) * 1e6
    rows = []
    for (name, grid), vals in per.items():
        dur = med(vals, "dur_us")
        busy = None
        if vals.get("SQ_VALU_MFMA_BUSY_CYCLES"):
            busy = statistics.median(
                c / (SIMDS * t * 1e-6 * clk)
                for c, t in zip(vals["SQ_VALU_MFMA_BUSY_CYCLES"], vals["dur_us"]) if t > 0)
        hit, miss = med(vals, "TCC_HIT_sum"), med(vals, "TCC_MISS_sum")
        cols = [dur, busy, ratio(vals, "SQ_WAIT_ANY", "SQ_WAVE_CYCLES"),
                ratio(vals, "SQ_WAIT_INST_ANY", "SQ_WAVE_CYCLES"),
                ratio(vals, "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES"),
                ratio(vals, "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS"),
                med(vals, "VmemLatency"), med(vals, "LdsLatency"),
                hit / (hit + miss) if hit is not None and miss is not None and hit + miss else None,
                ratio(vals, "TCC_EA0_RDREQ_LEVEL_sum", "TCC_EA0_RDREQ_sum")]
        rows.append((dur or 0.0, name, grid, cols))
    rows.sort(key=lambda r: -r[0])
    fmt = ["{:9.1f}", "{:9.3f}", "{:9.3f}", "{:9.3f}", "{:9.3f}", "{:9.3f}", "{:9.0f}",
           "{:9.0f}", "{:9.3f}", "{:9.0f}"]
    for _, name, grid, cols in rows[:a.top]:
        cells = [f"{'-':>9}" if v is None else f.format(v) for f, v in zip(fmt, cols)]
        short = name if len(name) <= 110 else name[:107] + "..."
        lines.append(" ".join(cells) + f"  {short} ({grid})")
    text = "\n".join(lines) + "\n"
    if a.out:
        open(a.out, "w").write(text)
    print(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    s.add_argument("--out")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--call", required=True, help="the bench.py call the kernel belongs to")
    t.add_argument("--workload", required=True, help="the bench.py workload of the call")
    t.add_argument("--grid", type=int, default=None)
    t.add_argument("--copy-mib", type=int, required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    t.add_argument("--out")
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--cmd", required=True)
    m.add_argument("--sclk-mhz", type=float, default=None)
    m.add_argument("--out")
    st = sub.add_parser("stalls")
    st.add_argument("csv", nargs="+")
    st.add_argument("--cmd", action="append", required=True, help="one per pass, in order")
    st.add_argument("--kernel", default=None)
    st.add_argument("--sclk-mhz", type=float, default=None)
    st.add_argument("--top", type=int, default=12)
    st.add_argument("--out")
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma, "stalls": cmd_stalls}[a.what](a)


if __name__ == "__main__":
    main()
