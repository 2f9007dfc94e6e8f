#!/usr/bin/env python3
"""Turn two rocprofv3 counter runs of bench.py into the HBM traffic per launch of
the quantizer kernel, calibrated against a plain copy of known size.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch -- \\
        python3 bench.py --steps 8 --warmup 2 --no-cpu --eager --no-gemm --no-ceiling --no-mlp --no-sweep --no-shard --no-quality --calib-copy-mib 256
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write -- \\
        python3 bench.py --steps 8 --warmup 2 --no-cpu --eager --no-gemm --no-ceiling --no-mlp --no-sweep --no-shard --no-quality --calib-copy-mib 256
    python3 bench_pmc.py DIR 256

FETCH_SIZE / WRITE_SIZE are read in KiB per dispatch.  The copy kernel reads and
writes exactly 256 MiB; the ratio of that to what the counter reports for it
scales the quantizer's counts to bytes.  Writes profiles/*_traffic.json (read by
bench.py, together with a hash of the kernel sources it was measured on) and a
short markdown summary.
"""
import csv
import glob
import json
import os
import statistics
import sys

import bench

ROOT = os.path.dirname(os.path.abspath(__file__))


# kernels whose traffic is summarized: (key, name prefix in the trace, algorithmic
# read bytes, algorithmic write bytes, what it is)
FLUX_E = 4608 * 3072
WEIGHT_E = 12288 * 3072
KERNELS = [
    ("kq", "void kq::(anonymous namespace)::butterfly_kernel<0, false, 0>", FLUX_E * 2 + 96 * 60,
     FLUX_E // 2 + FLUX_E // 32, "kq_quantize (butterfly), 4608x3072 bf16"),
    ("hq", "void kq::(anonymous namespace)::butterfly_kernel<0, false, 2>", FLUX_E * 2,
     FLUX_E // 2 + FLUX_E // 32, "hq_quantize (block Hadamard), 4608x3072 bf16"),
    ("sq", "void kq::(anonymous namespace)::sq_kernel<0, false>", FLUX_E * 2 + 3072 * 4,
     FLUX_E // 2 + FLUX_E // 32, "sq_quantize (SmoothQuant), 4608x3072 bf16"),
    ("norm", "void kq::(anonymous namespace)::norm_hw_kernel<true, false, 3>", FLUX_E * 2 + 2 * 3072 * 4 + 96 * 60,
     FLUX_E // 2 + FLUX_E // 32, "kq_norm_quantize (LayerNorm + modulation fused), 4608x3072 bf16"),
    ("weights", "void kq::(anonymous namespace)::butterfly_kernel<0, false, 1>", WEIGHT_E * 2 + 96 * 60,
     WEIGHT_E // 2 + WEIGHT_E // 32, "kq_quantize_weights, 12288x3072 bf16"),
]


def per_kernel(csv_path, counter):
    out = {k[0]: [] for k in KERNELS}
    out["copy"] = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        for key, prefix, *_ in KERNELS:
            if name.startswith(prefix):
                out[key].append(v)
                break
        else:
            # the calibration copy (a device-to-device tensor copy) runs on the runtime's
            # buffer-copy kernel; torch's elementwise copy kernels are not it
            if name.startswith("__amd_rocclr_copyBuffer"):
                out["copy"].append(v)
    return out


# (the 4608 x 12288, shard, quality and sweep legs: left out)
CMD = ("python3 bench.py --steps 8 --warmup 2 --no-cpu --eager --no-gemm --no-ceiling --no-mlp "
       "--no-sweep --no-shard --no-quality --calib-copy-mib %d")


def main():
    d, mib = sys.argv[1], int(sys.argv[2])
    fetch = per_kernel(glob.glob(os.path.join(d, "fetch", "*counter_collection.csv"))[0], "FETCH_SIZE")
    write = per_kernel(glob.glob(os.path.join(d, "write", "*counter_collection.csv"))[0], "WRITE_SIZE")
    copy_bytes = mib << 20
    # the copy's largest dispatches are the calibration copies
    f_copy = max(fetch["copy"]) * 1024.0
    w_copy = max(write["copy"]) * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    rows = {}
    for key, _, algo_rd, algo_wr, what in KERNELS:
        if not fetch[key] or not write[key]:
            continue
        rd = statistics.median(fetch[key]) * 1024.0 * f_scale
        wr = statistics.median(write[key]) * 1024.0 * w_scale
        rows[key] = dict(what=what, fetch_kib=statistics.median(fetch[key]),
                         write_kib=statistics.median(write[key]), rd=rd, wr=wr, algo_rd=algo_rd,
                         algo_wr=algo_wr)
    kq = rows["kq"]
    res = {
        "kernel": "butterfly_kernel<bf16> (kq_quantize, KQ_T_PARAMS), 4608x3072 bf16, 96 factor sets",
        "kernel_source_sha256": bench.kernel_source_hash(),
        "fetch_size_kib_per_launch": kq["fetch_kib"],
        "write_size_kib_per_launch": kq["write_kib"],
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": f_copy / 1024, "write_kib": w_copy / 1024,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "read_bytes_per_launch": kq["rd"],
        "write_bytes_per_launch": kq["wr"],
        "traffic_bytes_per_launch": kq["rd"] + kq["wr"],
        "algorithmic_read_bytes": kq["algo_rd"],
        "algorithmic_write_bytes": kq["algo_wr"],
        "other_kernels": {k: {kk: v for kk, v in r.items()} for k, r in rows.items() if k != "kq"},
    }
    json.dump(res, open(bench.TRAFFIC_FILE, "w"), indent=1)
    md = ["# HBM traffic of the quantizer kernels (FETCH_SIZE / WRITE_SIZE), one MI355X", "",
          "Commands (repository root):", "", "```",
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc/fetch -o fetch -- " + CMD % mib,
          "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc/write -o write -- " + CMD % mib,
          "python3 bench_pmc.py gpurun_out/pmc %d" % mib, "```", "",
          "Counters are medians per dispatch, scaled by what the same counter reads for a plain "
          "%d MiB device copy (read scale %.4f, write scale %.4f)." % (mib, f_scale, w_scale), "",
          "| kernel | read bytes / launch | algorithmic read | write bytes / launch | algorithmic write | total / algorithmic |",
          "|---|---|---|---|---|---|"]
    for key, r in rows.items():
        md.append(f"| {r['what']} | {r['rd']:,.0f} | {r['algo_rd']:,} | {r['wr']:,.0f} | {r['algo_wr']:,} | "
                  f"{(r['rd'] + r['wr']) / (r['algo_rd'] + r['algo_wr']):.3f}x |")
    md += ["", f"kq_quantize: {kq['rd'] + kq['wr']:,.0f} B per launch against "
               f"{kq['algo_rd'] + kq['algo_wr']:,} algorithmic; this figure is bench.py's roofline traffic "
               "while the kernel sources hash to the value stored in the JSON beside this file.", ""]
    open(os.path.join(ROOT, "profiles", "kq_butterfly_flux_4608x3072_traffic.md"), "w").write("\n".join(md))
    print("\n".join(md))


TRACE_KERNELS = [
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 0>",
     "`butterfly_kernel<bf16, -, forward>` (kq_quantize; also the quantize step of the unfused sequence)"),
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 2>", "`butterfly_kernel<bf16, -, hadamard>` (hq_quantize)"),
    ("void kq::(anonymous namespace)::sq_kernel<0, false>", "`sq_kernel<bf16>` (sq_quantize)"),
    ("(anonymous namespace)::stream_kernel", "`stream_kernel` (same-bytes ceiling, 5 grid sizes; when traced)"),
    ("void kq::(anonymous namespace)::norm_hw_kernel<true, false, 3>",
     "`norm_hw_kernel<modulated, -, 3 blocks per lane>` (kq_norm_quantize)"),
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 1>",
     "`butterfly_kernel<bf16, -, weights>` (kq_quantize_weights, 12288x3072)"),
    ("gemm unsplit 216", "`mx_gemm_kernel<256x256 tiles, bf16 out, staged>` (kq_mx_gemm, 4608x12288x3072, 216 workgroups)"),
    ("gemm unsplit 48", "`mx_gemm_kernel<256x256 tiles, bf16 out, staged>` (kq_mx_gemm, 1024x3072x12288, 48 workgroups)"),
    ("gemm split 48", "`mx_gemm_kernel<..., split>` (kq_mx_gemm_ws, 4608x256x3072 in 2 K parts, 48 workgroups)"),
    ("fused gemm 256", "`fused_gemm_kernel` (kq_mx_gemm_fused, 4608x12288x3072, 256 workgroups)"),
    ("fused gemm 36", "`fused_gemm_kernel` (kq_mx_gemm_fused, 4608x256x3072 whole tiles, 36 workgroups)"),
    ("fused gemm 160", "`fused_gemm_kernel<..., split>` (kq_mx_gemm_fused_ws, 4608x256x3072 in 4 K parts, 160 workgroups)"),
    ("gemm split 192", "`mx_gemm_kernel<..., split>` (kq_mx_gemm_ws, 1024x3072x12288 in 4 K parts, 192 workgroups)"),
    ("gemm split 96",
     "`mx_gemm_kernel<..., split>` (kq_mx_gemm_static, 1024x3072x12288 in 2 K parts, 96 workgroups)"),
    ("mlp-shape void kq::(anonymous namespace)::butterfly_kernel<0, false, 0>",
     "`butterfly_kernel<bf16, -, forward>` on 4608x12288 (the last leg)"),
    ("void at::native::(anonymous namespace)::vectorized_layer_norm_kernel", "torch layer_norm (unfused sequence)"),
    ("void at::native::elementwise_kernel_manual_unroll<128, 8, at::native::gpu_kernel_impl_nocast<at::native::addcm",
     "torch addcmul (unfused sequence)"),
]


def trace(trace_dir, bench_json):
    """Kernel-trace summary (durations per kernel: average, median, p10, p90) of
    `rocprofv3 --kernel-trace --stats ... -- python3 bench.py --no-cpu --no-sweep --no-shard --no-quality --no-overlap --no-ceiling`, with the
    unprofiled bench line of the same build for the cross-check."""
    rows = list(csv.DictReader(open(glob.glob(os.path.join(trace_dir, "*kernel_trace.csv"))[0])))
    # bench.py's legs run in order and (without the sweep) the 4608 x 12288 leg comes
    # last, after the W4A4 product: forward-quantizer dispatches after the last product
    # dispatch are that shape
    gemm_end = max((int(r["End_Timestamp"]) for r in rows if "mx_gemm_kernel" in r["Kernel_Name"]), default=None)
    fwd = TRACE_KERNELS[0][0]
    dur = {}
    for r in rows:
        name = r["Kernel_Name"]
        if name.startswith(fwd) and gemm_end is not None and int(r["Start_Timestamp"]) > gemm_end:
            name = "mlp-shape " + name
        if "mx_gemm_kernel<" in name:
            # one row per product: the split variant's last template argument is true;
            # the grid (workgroups of 512 lanes) tells the two unsplit shapes apart
            grid = int(r.get("Grid_Size_X") or r.get("Grid_Size") or 0) // 512
            name = f"gemm {'split' if name.split('>(')[0].endswith('true') else 'unsplit'} {grid}"
        elif "fused_gemm_kernel<" in name:
            name = f"fused gemm {int(r.get('Grid_Size_X') or r.get('Grid_Size') or 0) // 512}"
        dur.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    b = json.load(open(bench_json))

    def q(v, f):
        v = sorted(v)
        return v[min(len(v) - 1, int(f * len(v)))]

    md = ["# Kernel trace of bench.py, FLUX.1-schnell-like 4608x3072 bf16 workload (one MI355X)", "",
          "Commands (repository root):", "", "```",
          "rocprofv3 --kernel-trace --stats --output-format csv -d gpurun_out/trace -o bench -- python3 bench.py --no-cpu --no-sweep --no-shard --no-quality --no-overlap --no-ceiling",
          "python3 bench.py --no-cpu --no-sweep --no-shard --no-quality --no-overlap > gpurun_out/bench.json",
          "python3 bench_pmc.py trace gpurun_out/trace gpurun_out/bench.json", "```", "",
          "bench.py replays each timed leg from one captured HIP graph (%d rotating buffer sets for the "
          "4608x3072 legs).  Durations from the trace (end - start per dispatch), microseconds:"
          % b.get("config", {}).get("pool_sets", 0), "",
          "| kernel | dispatches | average | median | p10 | p90 |", "|---|---|---|---|---|---|"]
    kq_avg = None
    for prefix, label in TRACE_KERNELS:
        v = [x for n, vals in dur.items() if n.startswith(prefix) for x in vals]
        if not v:
            continue
        avg = statistics.mean(v)
        if kq_avg is None:
            kq_avg = avg
        md.append(f"| {label} | {len(v)} | {avg:.2f} | {statistics.median(v):.2f} | {q(v, 0.1):.2f} | "
                  f"{q(v, 0.9):.2f} |")
    md += ["", f"The quantizer kernel's average duration here ({kq_avg:.2f} us) against the unprofiled bench line of "
               f"the same build: {b['ms_per_step'] * 1e3:.2f} us per step by HIP events on the launch stream "
               f"({b['roofline']['achieved']:.0f} GB/s algorithmic, {100 * b['roofline']['frac']:.1f} % of 8 TB/s); "
               f"they agree within {100 * abs(b['ms_per_step'] * 1e3 - kq_avg) / kq_avg:.1f} % (the event time per step "
               "also holds the dependency gap between consecutive kernels of the graph, so it is the larger).", ""]
    open(os.path.join(ROOT, "profiles", "kq_kernels_flux_4608x3072_kernel_trace.md"), "w").write("\n".join(md))
    print("\n".join(md))


CLOCK_KERNELS = [
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 0>", "kq_quantize (butterfly)"),
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 2>", "hq_quantize (block Hadamard)"),
    ("void kq::(anonymous namespace)::sq_kernel<0, false>", "sq_quantize (SmoothQuant)"),
    ("(anonymous namespace)::stream_kernel", "same bytes, one unit per lane"),
    ("(anonymous namespace)::stream_pair_kernel", "same bytes, two units per lane"),
    ("(anonymous namespace)::stream_ring_kernel", "same bytes, two units in flight"),
    ("(anonymous namespace)::stream_read_kernel", "read half alone"),
    ("(anonymous namespace)::stream_write_kernel", "write half alone"),
    ("void kq::(anonymous namespace)::norm_hw_kernel<true, false, 3>", "kq_norm_quantize (fused norm)"),
]
CLOCK_CMD = ("python3 bench.py --steps 20 --warmup 5 --no-cpu --eager --no-weights --no-gemm --no-mlp "
             "--no-shard --no-quality --no-sweep --no-overlap")
CLOCK_COUNTERS = "GRBM_GUI_ACTIVE SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_ACTIVE_INST_VALU SQ_WAIT_INST_ANY"


def clock(run_dir):
    """Per-kernel medians of a `rocprofv3 --kernel-trace --pmc CLOCK_COUNTERS` run of
    CLOCK_CMD: duration, the counters, and the clock they imply (GRBM_GUI_ACTIVE
    cycles of the busy GPU over the dispatch's duration)."""
    ctr = list(csv.DictReader(open(glob.glob(os.path.join(run_dir, "*counter_collection.csv"))[0])))
    kt = glob.glob(os.path.join(run_dir, "*kernel_trace.csv"))
    times = {}
    if kt:
        for r in csv.DictReader(open(kt[0])):
            times[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    per = {}
    for r in ctr:
        key = next((k for k, _ in CLOCK_KERNELS if r["Kernel_Name"].startswith(k)), None)
        if key is None:
            continue
        d = per.setdefault(key, {}).setdefault(r["Dispatch_Id"], {})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if "Start_Timestamp" in r and r.get("End_Timestamp"):
            d["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        elif r["Dispatch_Id"] in times:
            d["_us"] = times[r["Dispatch_Id"]]
    names = CLOCK_COUNTERS.split()
    rows = []
    for key, label in CLOCK_KERNELS:
        ds = [d for d in per.get(key, {}).values() if "_us" in d]
        if not ds:
            continue
        med = {n: statistics.median(d.get(n, 0.0) for d in ds) for n in names}
        rows.append((label, len(ds), statistics.median(d["_us"] for d in ds), med))
    # GRBM_GUI_ACTIVE holds a fixed count of the profiler's window around each dispatch
    # plus the busy cycles of the 8 XCDs: fit count = c0 + 8 f t over the kernels (one
    # clock f for all), then each kernel's own clock is (count - c0) / (8 t)
    ts = [r[2] for r in rows]
    gs = [r[3]["GRBM_GUI_ACTIVE"] for r in rows]
    n = len(ts)
    tm, gm = sum(ts) / n, sum(gs) / n
    slope = sum((t - tm) * (g - gm) for t, g in zip(ts, gs)) / sum((t - tm) ** 2 for t in ts)
    c0 = gm - slope * tm
    md = ["# Clock and instruction counters per kernel, 4608x3072 bf16 (one MI355X)", "",
          "Commands (repository root):", "", "```",
          "rocprofv3 --kernel-trace --pmc " + CLOCK_COUNTERS + " --output-format csv -d gpurun_out/clock -o clock -- "
          + CLOCK_CMD, "python3 bench_pmc.py clock gpurun_out/clock", "```", "",
          "Medians per dispatch (counters summed over the device).  GRBM_GUI_ACTIVE counts a fixed window of the "
          "profiler around each dispatch plus 8 XCDs x the busy cycles; a least-squares fit over these kernels gives "
          f"the window as {c0:,.0f} counts and one clock of {slope / 8 / 1e3:.3f} GHz; `GHz` is each kernel's own "
          "(count - window) / (8 x duration).  `VALU/wave` = SQ_INSTS_VALU / SQ_WAVES.", "",
          "| kernel | dispatches | us | " + " | ".join(names) + " | GHz | VALU/wave |",
          "|---|---|---|" + "---|" * len(names) + "---|---|"]
    for label, nd, us, med in rows:
        ghz = (med["GRBM_GUI_ACTIVE"] - c0) / (8 * us) / 1e3 if us else 0.0
        vpw = med["SQ_INSTS_VALU"] / med["SQ_WAVES"] if med["SQ_WAVES"] else 0.0
        md.append(f"| {label} | {nd} | {us:.2f} | " + " | ".join(f"{med[n]:,.0f}" for n in names)
                  + f" | {ghz:.2f} | {vpw:.0f} |")
    md.append("")
    open(os.path.join(ROOT, "profiles", "kq_kernels_flux_4608x3072_clock.md"), "w").write("\n".join(md))
    print("\n".join(md))


def counters(out_md, title, commands, dirs):
    """Medians per dispatch of every counter in the rocprofv3 counter runs under
    `dirs`, one row per (kernel, grid size), for the kernels named in CLOCK_KERNELS,
    TRACE_KERNELS and the matrix-core and norm kernels; written as a markdown table
    under profiles/ with the commands that produced the runs."""
    known = [(k, v) for k, v in CLOCK_KERNELS] + [
        ("void kq::(anonymous namespace)::mfma_kernel<false>", "matrix-core kq_quantize (design A)"),
        ("void kq::(anonymous namespace)::norm_hw_kernel<true, false, 3>", "kq_norm_quantize (fused norm)"),
        ("void kq::(anonymous namespace)::mx_gemm_kernel<", "kq_mx_gemm (W4A4 product)")]
    per = {}
    for dd in dirs:
        for path in glob.glob(os.path.join(dd, "*counter_collection.csv")):
            for r in csv.DictReader(open(path)):
                label = next((v for k, v in known if r["Kernel_Name"].startswith(k)), None)
                if label is None:
                    continue
                key = (label, int(r["Grid_Size"]))
                d = per.setdefault(key, {}).setdefault((dd, int(r["Dispatch_Id"])), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                if r.get("End_Timestamp"):
                    d["_us"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
    # a kernel timed in two legs of one run (the same grid on two shapes) shows as two
    # runs of dispatch ids with other work between them: split at gaps of > 20 ids
    split = {}
    for (label, g), v in per.items():
        ids = sorted(v)
        legs, cur = [], [ids[0]]
        for a, b in zip(ids, ids[1:]):
            if b[0] != a[0] or b[1] - a[1] > 20:
                legs.append(cur)
                cur = []
            cur.append(b)
        legs.append(cur)
        # the same leg in several runs (dirs) lines up by order within each run
        by_dir = {}
        for leg in legs:
            by_dir.setdefault(leg[0][0], []).append(leg)
        nlegs = max(len(x) for x in by_dir.values())
        for i in range(nlegs):
            name = label if nlegs == 1 else f"{label}, leg {i + 1}"
            split[(name, g)] = {k: v[k] for x in by_dir.values() if i < len(x) for k in x[i]}
    per = split
    names = sorted({n for v in per.values() for d in v.values() for n in d if not n.startswith("_")})
    md = [f"# {title}", "", "Commands (repository root):", "", "```"] + commands + ["```", "",
          "Medians per dispatch, counters summed over the device (FETCH_SIZE / WRITE_SIZE in KiB as "
          "the counter reports them).  Grid = work-items launched.", ""]
    md.append("| counter | " + " | ".join(f"{lab} (grid {g:,})" for lab, g in per) + " |")
    md.append("|---|" + "---|" * len(per))
    def med(v, n, fmt):
        xs = [d[n] for d in v.values() if n in d]
        return format(statistics.median(xs), fmt) if xs else "-"
    rows = [("dispatches (per run)", lambda v: f"{len(v) // max(1, len({k[0] for k in v}))}"),
            ("duration us", lambda v: med(v, "_us", ".2f"))]
    rows += [(n, (lambda n: lambda v: med(v, n, ",.0f"))(n)) for n in names]
    for name, fn in rows:
        md.append(f"| {name} | " + " | ".join(fn(v) for v in per.values()) + " |")
    md.append("")
    open(os.path.join(ROOT, "profiles", out_md), "w").write("\n".join(md))
    print("\n".join(md))


if __name__ == "__main__":
    if sys.argv[1] == "counters":
        # bench_pmc.py counters OUT.md "title" "cmd1;cmd2;..." DIR [DIR ...]
        counters(sys.argv[2], sys.argv[3], sys.argv[4].split(";"), sys.argv[5:])
    elif sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3])
    elif sys.argv[1] == "clock":
        clock(sys.argv[2])
    else:
        main()
