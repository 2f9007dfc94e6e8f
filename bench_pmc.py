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
    ("norm", "void kq::(anonymous namespace)::norm_kernel<0, true, false>", FLUX_E * 2 + 2 * 3072 * 4 + 96 * 60,
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
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d out/pmc/fetch -o fetch -- " + CMD % mib,
          "rocprofv3 --pmc WRITE_SIZE --output-format csv -d out/pmc/write -o write -- " + CMD % mib,
          "python3 bench_pmc.py out/pmc %d" % mib, "```", "",
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
    ("void kq::(anonymous namespace)::norm_kernel<0, true, false>", "`norm_kernel<bf16, modulated>` (kq_norm_quantize)"),
    ("void kq::(anonymous namespace)::butterfly_kernel<0, false, 1>",
     "`butterfly_kernel<bf16, -, weights>` (kq_quantize_weights, 12288x3072)"),
    ("void kq::(anonymous namespace)::mx_gemm_kernel<", "`mx_gemm_kernel<256x256 tiles, bf16 out, staged>` (kq_mx_gemm, 4608x12288x3072)"),
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
        dur.setdefault(name, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0)
    b = json.load(open(bench_json))

    def q(v, f):
        v = sorted(v)
        return v[min(len(v) - 1, int(f * len(v)))]

    md = ["# Kernel trace of bench.py, FLUX.1-schnell-like 4608x3072 bf16 workload (one MI355X)", "",
          "Commands (repository root):", "", "```",
          "rocprofv3 --kernel-trace --stats --output-format csv -d out/trace -o bench -- python3 bench.py --no-cpu --no-sweep --no-shard --no-quality --no-overlap --no-ceiling",
          "python3 bench.py --no-cpu --no-sweep --no-shard --no-quality --no-overlap > out/bench.json",
          "python3 bench_pmc.py trace out/trace out/bench.json", "```", "",
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


if __name__ == "__main__":
    if sys.argv[1] == "trace":
        trace(sys.argv[2], sys.argv[3])
    else:
        main()
