#!/usr/bin/env python3
"""Turn two rocprofv3 counter runs of bench.py into the HBM traffic per launch of
the quantizer kernel, calibrated against a plain copy of known size.

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR/fetch -o fetch -- \\
        python3 bench.py --steps 8 --warmup 2 --no-cpu --no-sq --eager --calib-copy-mib 256
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR/write -o write -- \\
        python3 bench.py --steps 8 --warmup 2 --no-cpu --no-sq --eager --calib-copy-mib 256
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


def per_kernel(csv_path, counter):
    out = {"kq": [], "copy": []}
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] != counter:
            continue
        name = r["Kernel_Name"]
        v = float(r["Counter_Value"])
        if "butterfly_kernel<0, false>" in name:
            out["kq"].append(v)
        elif "copy" in name.lower() and "bfloat16" not in name:
            out["copy"].append(v)
    return out


def main():
    d, mib = sys.argv[1], int(sys.argv[2])
    fetch = per_kernel(glob.glob(os.path.join(d, "fetch", "*counter_collection.csv"))[0], "FETCH_SIZE")
    write = per_kernel(glob.glob(os.path.join(d, "write", "*counter_collection.csv"))[0], "WRITE_SIZE")
    copy_bytes = mib << 20
    # the copy's largest dispatches are the calibration copies
    f_copy = max(fetch["copy"]) * 1024.0
    w_copy = max(write["copy"]) * 1024.0
    f_scale, w_scale = copy_bytes / f_copy, copy_bytes / w_copy
    rd = statistics.median(fetch["kq"]) * 1024.0 * f_scale
    wr = statistics.median(write["kq"]) * 1024.0 * w_scale
    elems = 4608 * 3072
    algo_rd, algo_wr = elems * 2 + 96 * 60, elems // 2 + elems // 32
    res = {
        "kernel": "butterfly_kernel<bf16> (kq_quantize, KQ_T_PARAMS), 4608x3072 bf16, 96 factor sets",
        "kernel_source_sha256": bench.kernel_source_hash(),
        "fetch_size_kib_per_launch": statistics.median(fetch["kq"]),
        "write_size_kib_per_launch": statistics.median(write["kq"]),
        "copy_calibration": {"bytes_each_way": copy_bytes, "fetch_kib": f_copy / 1024, "write_kib": w_copy / 1024,
                             "fetch_scale": f_scale, "write_scale": w_scale},
        "read_bytes_per_launch": rd,
        "write_bytes_per_launch": wr,
        "traffic_bytes_per_launch": rd + wr,
        "algorithmic_read_bytes": algo_rd,
        "algorithmic_write_bytes": algo_wr,
    }
    json.dump(res, open(bench.TRAFFIC_FILE, "w"), indent=1)
    md = ["# HBM traffic of kq_quantize (butterfly), 4608x3072 bf16", "",
          "Commands (repository root, one MI355X):", "", "```",
          "rocprofv3 --pmc FETCH_SIZE --output-format csv -d gpurun_out/pmc/fetch -o fetch -- python3 bench.py --steps 8 --warmup 2 --no-cpu --no-sq --eager --calib-copy-mib %d" % mib,
          "rocprofv3 --pmc WRITE_SIZE --output-format csv -d gpurun_out/pmc/write -o write -- python3 bench.py --steps 8 --warmup 2 --no-cpu --no-sq --eager --calib-copy-mib %d" % mib,
          "python3 bench_pmc.py gpurun_out/pmc %d" % mib, "```", "",
          "| | counter (KiB/dispatch) | scale from the %d MiB copy | bytes per launch | algorithmic bytes |" % mib,
          "|---|---|---|---|---|",
          f"| read (FETCH_SIZE) | {res['fetch_size_kib_per_launch']:.1f} | {f_scale:.4f} | {rd:,.0f} | {algo_rd:,} |",
          f"| write (WRITE_SIZE) | {res['write_size_kib_per_launch']:.1f} | {w_scale:.4f} | {wr:,.0f} | {algo_wr:,} |",
          "", f"Total {rd + wr:,.0f} B per launch against {algo_rd + algo_wr:,} algorithmic "
              f"({(rd + wr) / (algo_rd + algo_wr):.3f}x).", ""]
    open(os.path.join(ROOT, "profiles", "kq_butterfly_flux_4608x3072_traffic.md"), "w").write("\n".join(md))
    print("\n".join(md))


if __name__ == "__main__":
    main()
