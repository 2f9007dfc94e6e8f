#!/usr/bin/env python3
"""Benchmark of the KroQuant online activation quantizer on one MI355X.

One step = one kq_quantize call (factor expansion, block transform, amax, E8M0
scale, E2M1 encode and packed stores, all in one kernel) over the FLUX.1-schnell
joint-stream activation X[4608, 3072] bf16 with its 96 factor sets.  Inputs are
resident in HBM before the timed region; the steps rotate through a pool of
distinct input/output buffer sets larger than the 256 MB last-level cache, so
every step reads its activations from HBM rather than from cache.

Prints one JSON line.  Extra keys beside the contract: the SmoothQuant and
Hadamard baselines timed the same way, the other kernels' legs, one GPU's share
at 8-way sharding, and (in the CPU leg, the only part that runs the oracle) a
parity summary of one step against it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "quantized activations Gelem/s and % of peak HBM GB/s, 4608x3072 bf16 on 1 MI355X"
PEAK_HBM_GBS = 8000.0
BYTES_PER_ELEM = 2 + 0.5 + 1 / 32  # bf16 in, E2M1 codes out, one E8M0 byte per 32


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--pool", type=int, default=32, help="distinct buffer sets rotated over (1.15 GB at 32)")
    ap.add_argument("--variant", choices=["butterfly", "mfma"], default="butterfly")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--no-sq", action="store_true",
                    help="skip the SmoothQuant and block-Hadamard comparison timings")
    ap.add_argument("--no-weights", action="store_true", help="skip the weight-side timing")
    ap.add_argument("--no-gemm", action="store_true", help="skip the W4A4 product timing")
    ap.add_argument("--no-mlp", action="store_true", help="skip the 4608x12288 quantizer timing")
    ap.add_argument("--no-shard", action="store_true", help="skip the 8-way shard timing")
    ap.add_argument("--no-quality", action="store_true",
                    help="skip the quantization-error comparison of the transforms")
    ap.add_argument("--warm-ms", type=float, default=100.0,
                    help="untimed graph replays before each timed one, at least this many ms")
    ap.add_argument("--no-overlap", action="store_true",
                    help="skip the timing of independent steps alternating over two streams")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the 28-call batched sweep (14 x 18432x3072 + 14 x 18432x12288)")
    ap.add_argument("--no-norm", action="store_true",
                    help="skip the normalization-fused quantizer timing")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the same-bytes streaming kernel (practical HBM ceiling)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a captured graph")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (4 times) as the "
                         "known-size reference for hardware byte counters")
    return ap.parse_args()


REPLAYS = 7  # timed repetitions of each leg; the line reports their median (p10 and p90 beside it)


class Timing(float):
    """Milliseconds per step: the median over the timed repetitions of a leg, with
    the 10th and 90th percentiles and the repetition count as attributes."""

    def __new__(cls, samples):
        a = np.asarray(samples, np.float64)
        t = super().__new__(cls, float(np.median(a)))
        t.p10, t.p90, t.n = float(np.percentile(a, 10)), float(np.percentile(a, 90)), len(a)
        return t

    def summary(self, steps):
        return {"replays": self.n, "steps_per_replay": steps, "median_ms": round(float(self), 6),
                "p10_ms": round(self.p10, 6), "p90_ms": round(self.p90, 6)}


def timed(fn, steps, warmup, stream):
    """Milliseconds per call of fn(i): REPLAYS repetitions of `steps` calls launched
    from Python, each timed with HIP events on `stream`."""
    import torch
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    samples = []
    for _ in range(REPLAYS):
        start.record(stream)
        for i in range(steps):
            fn(i)
        end.record(stream)
        end.synchronize()
        samples.append(start.elapsed_time(end) / steps)
    torch.cuda.synchronize()
    return Timing(samples)


WARM_MS = 100.0  # untimed replays before each timed one: at least this much GPU time


def warm_replays(g, stream):
    """Replays g untimed until WARM_MS of GPU time has passed (at least once), so the
    timed replay starts from the clocks of sustained work, not from an idle GPU."""
    t0 = time.perf_counter()
    while True:
        g.replay()
        stream.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= WARM_MS:
            break


def _replay_timed(g, stream):
    """REPLAYS timed replays of graph g on `stream` (after the untimed warm-up
    replays); milliseconds per replay."""
    import torch
    warm_replays(g, stream)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = []
    for _ in range(REPLAYS):
        start.record(stream)
        g.replay()
        end.record(stream)
        end.synchronize()
        out.append(start.elapsed_time(end))
    return out


def timed_graph(fn, steps, warmup):
    """Milliseconds per step when exactly `steps` steps (fn(0) .. fn(steps-1)) are
    replayed from one captured HIP graph: the median over REPLAYS timed replays.
    The graph holds the same kernel launches on the same buffers as the eager loop;
    it only removes the per-launch host work.  Untimed replays for at least WARM_MS
    (after `warmup` eager steps) precede the timed ones."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(1, warmup)):
            fn(i)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        samples = _replay_timed(g, side)
    torch.cuda.synchronize()
    return Timing([t / steps for t in samples])


KERNEL_SOURCES = ("kq_butterfly.hip", "kq_device.hpp", "kq_factors.hpp", "kq_launch.hpp")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kq_butterfly_flux_4608x3072_traffic.json")


def timed_graph_two_streams(fn, steps, warmup):
    """As timed_graph, but the captured steps alternate between two streams (even
    steps on the capture stream, odd ones on a second stream, each chain in order):
    consecutive steps are independent (distinct buffer sets), so one step's ramp-up
    may overlap the previous step's drain."""
    import torch
    side, other = torch.cuda.Stream(), torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(max(1, warmup)):
            fn(i)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            cap = torch.cuda.current_stream()
            other.wait_stream(cap)
            for i in range(steps):
                if i % 2:
                    with torch.cuda.stream(other):
                        fn(i)
                else:
                    fn(i)
            cap.wait_stream(other)
    torch.cuda.synchronize()
    with torch.cuda.stream(side):
        samples = _replay_timed(g, side)
    torch.cuda.synchronize()
    return Timing([t / steps for t in samples])


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "online_activation_quantizer_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed counter runs, or None when the kernel
    sources changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(x, p, seconds):
    import oracle
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.quantize(x, p, nthreads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": round(x.size * reps / el / 1e9, 4), "unit": "Gelem/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full {x.shape[0]}x{x.shape[1]} bf16 input, {reps} passes "
                      f"({el:.1f} s, fp64 dense 32x32 per block + MXFP4 encode)"}


CEILING_DESIGNS = (("lane", (768, 1024, 1536, 2048)), ("pair", (512, 768, 864)), ("ring", (256, 768)))


def stream_ceiling(args, xs, qs, ss, kq_ms):
    """The same bytes per call (64 B read, 17 B written per 32-element unit) moved
    with no arithmetic, timed like the quantizer step over the same buffer pool:
    three access designs at a few grid sizes each (the fastest is the practical
    ceiling of one call at this size), the read half and the write half alone, and
    the runtime's device-to-device copy of the same total bytes (half read, half
    written)."""
    import torch

    from online_activation_quantizer_amd import bench_stream as bs
    P = len(xs)
    elems = xs[0].numel()
    units = elems // 32
    run = (lambda f: timed(f, args.steps, args.warmup, torch.cuda.current_stream())) if args.eager else \
        (lambda f: timed_graph(f, args.steps, args.warmup))

    def leg(design, grid):
        def step(i):
            j = i % P
            bs.kq_bench_stream(xs[j], qs[j], ss[j], grid, design=design)
        return run(step)

    designs, best = {}, None
    codes = {"lane": bs.KQB_LANE, "pair": bs.KQB_PAIR, "ring": bs.KQB_RING}
    for name, grids in CEILING_DESIGNS:
        for grid in grids:
            ms = leg(codes[name], grid)
            if name not in designs or ms < designs[name][0]:
                designs[name] = (ms, grid)
            if best is None or ms < best[0]:
                best = (ms, grid, name)
    ms, grid, name = best
    gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    out = {"ms_per_step": round(ms, 6), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
           "design": name, "grid": grid, "timing": ms.summary(args.steps),
           "kq_time_over_ceiling_time": round(kq_ms / ms, 4),
           "designs": {k: {"us": round(v[0] * 1e3, 3), "grid": v[1]} for k, v in designs.items()}}
    for key, design, nbytes in (("read_only", bs.KQB_READ, units * 64), ("write_only", bs.KQB_WRITE, units * 17)):
        t = min(leg(design, g) for g in (1728, 2048))
        out[key] = {"us": round(t * 1e3, 3), "bytes": nbytes,
                    "hbm_frac": round(nbytes / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    half = (units * 81 // 2) // 256 * 256
    srcs = [x.view(torch.uint8).view(-1)[:half] for x in xs]
    dsts = [torch.empty(half, dtype=torch.uint8, device="cuda") for _ in range(P)]

    def copy_step(i):
        j = i % P
        dsts[j].copy_(srcs[j])
    t = run(copy_step)
    out["runtime_copy"] = {"us": round(t * 1e3, 3), "bytes_moved": 2 * half,
                           "hbm_frac": round(2 * half / (t * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "how": "torch copy_ of half the bytes between two device buffers"}
    del dsts
    return out


def norm_timing(args, cfg, xs, ps, qs, ss, kq_ms):
    """LayerNorm + adaptive-norm modulation fused ahead of the quantizer
    (kq_norm_quantize) on the same pool, against the unfused sequence it replaces
    as torch runs it: layer_norm, then the modulation (addcmul), both in bf16 with
    their outputs written to and re-read from HBM, then kq_quantize."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    P = len(xs)
    shift, scale = synth.make_modulation(1, cfg.d, np.random.default_rng(cfg.seed + 77))
    shd, scd = torch.from_numpy(shift).cuda(), torch.from_numpy(scale).cuda()
    xb = [x.view(torch.bfloat16) for x in xs]
    hbuf = torch.empty((cfg.rows, cfg.d), dtype=torch.bfloat16, device="cuda")
    sc_b, sh_b = (1 + scd).to(torch.bfloat16), shd.to(torch.bfloat16)

    def fused(i):
        j = i % P
        kq.kq_norm_quantize(xs[j], ps[j], shd, scd, cfg.rows, 1e-6, q=qs[j], s=ss[j])

    def unfused(i):
        j = i % P
        h = torch.nn.functional.layer_norm(xb[j], (cfg.d,), eps=1e-6)
        torch.addcmul(sh_b, h, sc_b, out=hbuf)
        kq.kq_quantize(hbuf.view(torch.int16), ps[j], q=qs[j], s=ss[j])

    run = (lambda f, n: timed(f, n, args.warmup, torch.cuda.current_stream())) if args.eager else \
        (lambda f, n: timed_graph(f, n, args.warmup))
    steps = max(8, args.steps // 4)
    f_ms = run(fused, steps)
    u_ms = run(unfused, steps)
    elems = cfg.rows * cfg.d
    gbs = elems * BYTES_PER_ELEM / (f_ms * 1e-3) / 1e9
    return {"workload": f"{cfg.rows}x{cfg.d} bf16 pre-norm activations, 1 modulation vector",
            "ms_per_call": round(f_ms, 6), "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "unfused_ms_per_call": round(u_ms, 6), "unfused_over_fused": round(u_ms / f_ms, 4),
            "fused_over_quantizer_alone": round(f_ms / kq_ms, 4)}


def mlp_timing(args):
    """The same quantizer on the FLUX MLP input width, X[4608, 12288] bf16 (384 factor
    sets), over 4 rotating sets (570 MB, beyond the last-level cache)."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    cfg = synth.get_config("flux_mlp")
    sets = 4
    xs = [synth.make_activations_device(cfg, cfg.seed + 1000 * i).view(torch.int16) for i in range(sets)]
    ps = [torch.from_numpy(synth.make_params(cfg.nb, np.random.default_rng(cfg.seed + i))).cuda()
          for i in range(sets)]
    qs = [torch.empty((cfg.rows, cfg.d // 2), dtype=torch.uint8, device="cuda") for _ in range(sets)]
    ss = [torch.empty((cfg.rows, cfg.d // 32), dtype=torch.uint8, device="cuda") for _ in range(sets)]
    if args.variant == "mfma":
        ts = [kq.kq_expand_factors(p, kq.KQ_T_DENSE_BF16X3) for p in ps]
        tfmt, var = kq.KQ_T_DENSE_BF16X3, kq.KQ_MFMA
    else:
        ts, tfmt, var = ps, kq.KQ_T_PARAMS, kq.KQ_BUTTERFLY

    def step(i):
        j = i % sets
        kq.kq_quantize(xs[j], ts[j], tfmt, var, q=qs[j], s=ss[j])

    steps = max(8, args.steps // 4)
    ms = (timed(step, steps, args.warmup, torch.cuda.current_stream()) if args.eager
          else timed_graph(step, steps, args.warmup))
    elems = cfg.rows * cfg.d
    gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    del xs, qs, ss
    return {"workload": f"{cfg.rows}x{cfg.d} bf16, {cfg.nb} factor sets, {args.variant}", "ms_per_call": round(ms, 6),
            "gelem_s": round(elems / (ms * 1e-3) / 1e9, 3), "gbs": round(gbs, 1),
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


E2M1_VALUES = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # OCP MX FP4 magnitudes, codes 0..7


def mxfp4_values(q, s):
    """float32 [rows, 32 nb] decoded from MXFP4 codes q [rows, 16 nb] (low nibble first,
    bit 3 the sign) and E8M0 scales s [rows, nb]; measurement only."""
    import torch
    mag = torch.tensor(E2M1_VALUES, dtype=torch.float32, device=q.device)
    table = torch.cat([mag, -mag])
    rows = q.shape[0]
    codes = torch.stack([q & 15, q >> 4], dim=-1).reshape(rows, -1).long()
    scale = torch.exp2(s.float() - 127.0)
    return (table[codes].view(rows, -1, 32) * scale.unsqueeze(-1)).view(rows, -1)


def quality_leg(x, p_lu, m_dev, times):
    """Quantization error of the transforms the pages compare, beside their kernel
    times: relative RMS error ||x_hat - x|| / ||x|| of the activation X (bf16 values)
    after MXFP4 and the transform's inverse.  For orthogonal transforms (identity,
    block Hadamard, KroQuant factors that are plane rotations) this is the error of
    y = T x itself; for the synthetic uncalibrated LU factors x_hat solves
    T_b x_hat = y_hat per block; for SmoothQuant x_hat = y_hat / mult."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    rows, d = x.shape
    nb = d // 32
    xf = x.view(torch.bfloat16).double()

    def err(a, b):
        return round(float(torch.linalg.norm(a.double() - b.double()) / torch.linalg.norm(b.double())), 6)

    out = {"workload": f"{rows}x{d} bf16 (the headline input), relative RMS error after MXFP4"}
    pid = torch.from_numpy(synth.make_identity_params(nb)).cuda()
    q, s = kq.kq_quantize(x, pid)
    out["plain_mxfp4"] = {"rel_err": err(mxfp4_values(q, s), xf), "us_per_call": times.get("kq")}
    q, s, y = kq.hq_transform_debug(x)
    out["block_hadamard"] = {"rel_err": err(mxfp4_values(q, s), y), "us_per_call": times.get("hq")}
    for name, pr in (("kroquant_rotations_45deg", synth.make_rotation_params(nb)),
                     ("kroquant_random_rotations", synth.make_rotation_params(nb, np.random.default_rng(11)))):
        q, s, y = kq.kq_transform_debug(x, torch.from_numpy(pr).cuda())
        out[name] = {"rel_err": err(mxfp4_values(q, s), y), "us_per_call": times.get("kq")}
    q, s = kq.kq_quantize(x, p_lu)
    T = kq.kq_expand_factors(p_lu, kq.KQ_T_DENSE_F32).view(nb, 32, 32).double()
    yh = mxfp4_values(q, s).double().view(rows, nb, 32).permute(1, 2, 0).contiguous()
    xh = torch.linalg.solve(T, yh).permute(2, 0, 1).reshape(rows, d)
    out["kroquant_random_lu_factors"] = {"rel_err": err(xh, xf), "us_per_call": times.get("kq"),
                                         "note": "uncalibrated synthetic factors (ill-conditioned)"}
    if m_dev is not None:
        q, s = kq.sq_quantize(x, m_dev)
        out["smoothquant_random_scales"] = {"rel_err": err(mxfp4_values(q, s).double() / m_dev.double(), xf),
                                            "us_per_call": times.get("sq")}
    torch.cuda.synchronize()
    return out


def shard_timing(args, xs, ps):
    """One GPU's share of the FLUX layer at 8-way sharding, each call on its own
    buffers from a pool larger than the last-level cache: token shards X[576, 3072]
    (all 96 factor sets; contiguous row ranges of the pool's inputs) and channel
    shards X[4608, 384] (12 factor sets; contiguous copies of column ranges)."""
    import torch

    import online_activation_quantizer_amd as kq
    rows, d = xs[0].shape
    nb = d // 32
    P = len(xs)
    out = {"workload": f"one GPU's share of {rows}x{d} bf16 at 8-way sharding"}
    legs = {
        "token_shard": [(x[r:r + rows // 8], p) for x, p in zip(xs, ps) for r in range(0, rows, rows // 8)],
        "channel_shard": [(xs[i % P][:, (i // P % 8) * (d // 8):(i // P % 8 + 1) * (d // 8)].contiguous(),
                           ps[i % P][(i // P % 8) * (nb // 8):(i // P % 8 + 1) * (nb // 8)].contiguous())
                          for i in range(min(8 * P, 96))],
    }
    for name, sets in legs.items():
        qs = [torch.empty((x.shape[0], x.shape[1] // 2), dtype=torch.uint8, device="cuda") for x, _ in sets]
        ss = [torch.empty((x.shape[0], x.shape[1] // 32), dtype=torch.uint8, device="cuda") for x, _ in sets]

        def step(i, sets=sets, qs=qs, ss=ss):
            j = i % len(sets)
            kq.kq_quantize(sets[j][0], sets[j][1], q=qs[j], s=ss[j])

        ms = (timed(step, args.steps, args.warmup, torch.cuda.current_stream()) if args.eager
              else timed_graph(step, args.steps, args.warmup))
        elems = sets[0][0].numel()
        gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
        out[name] = {"shape": list(sets[0][0].shape), "distinct_sets": len(sets), "us_per_call": round(ms * 1e3, 3),
                     "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
        del qs, ss
    return out


def sweep_timing(args):
    """The batched sweep: 28 layer-shaped calls alternating X[18432, 3072] and
    X[18432, 12288] bf16, each with its own inputs, factor set and outputs (10 GB moved,
    no reuse between calls), replayed as one graph a few times; time per sweep."""
    import torch

    import synth
    from synth.configs import SWEEP_CALLS, sweep_call
    import online_activation_quantizer_amd as kq
    calls = []
    elems = 0
    for i in range(SWEEP_CALLS):
        cfg = sweep_call(i)
        x = synth.make_activations_device(cfg, cfg.seed).view(torch.int16)
        p = torch.from_numpy(synth.make_params(cfg.nb, np.random.default_rng(cfg.seed))).cuda()
        q = torch.empty((cfg.rows, cfg.d // 2), dtype=torch.uint8, device="cuda")
        s = torch.empty((cfg.rows, cfg.d // 32), dtype=torch.uint8, device="cuda")
        calls.append((x, p, q, s))
        elems += cfg.rows * cfg.d

    def step(i):
        for x, p, q, s in calls:
            kq.kq_quantize(x, p, q=q, s=s)

    reps = 3
    ms = (timed(step, reps, 1, torch.cuda.current_stream()) if args.eager else timed_graph(step, reps, 1))
    gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    del calls
    torch.cuda.empty_cache()
    return {"workload": "14 x 18432x3072 + 14 x 18432x12288 bf16, own inputs and factors per call",
            "ms_per_sweep": round(ms, 4), "gelem_s": round(elems / (ms * 1e-3) / 1e9, 3),
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


PEAK_FP4_TFLOPS = 10100.0  # dense fp4 matrix-core peak of one MI355X


def gemm_timing(args, qs, ss):
    """The W4A4 product consuming the quantizer's output: FLUX.1-schnell MLP
    up-projection, Y[4608, 12288] = deq(Qx)[4608, 3072] deq(Qw)[12288, 3072]^T, with
    the activation codes of the pool's first set and quantized weights, bf16 out."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    wcfg = synth.get_weight_config("flux_w_mlp")
    w, p = synth.make_weights(wcfg)
    qw, sw = kq.kq_quantize_weights(torch.from_numpy(w.view(np.int16)).cuda(), torch.from_numpy(p).cuda())
    M, N, K = qs[0].shape[0], wcfg.rows, wcfg.d
    out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    P = len(qs)

    def step(i):
        j = i % P
        kq.kq_mx_gemm(qs[j], ss[j], qw, sw, out=out)

    steps = max(8, args.steps // 10)
    ms = (timed(step, steps, args.warmup, torch.cuda.current_stream()) if args.eager
          else timed_graph(step, steps, min(args.warmup, 10)))
    tflops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
    res = {"workload": f"FLUX.1-schnell MLP up-projection {M}x{N}x{K}, fp4 x fp4 (MXFP4), bf16 out",
           "ms_per_call": round(ms, 6), "tflops": round(tflops, 1),
           "mfma_frac_fp4": round(tflops / PEAK_FP4_TFLOPS, 4)}
    if hasattr(ms, "summary"):
        res["timing"] = ms.summary(steps)
    if not args.eager:
        res["library_baseline"] = library_gemm_timing(args, qs, ss, qw, sw, out)
    return res


def gemm_split_timing(args):
    """A product with few tiles and a long K, where splitting each tile in K parts
    (kq_mx_gemm_ws, through a workspace) pays: the FLUX MLP down-projection for
    1024 tokens, Y[1024, 3072] = deq(Qx)[1024, 12288] deq(Qw)[3072, 12288]^T (48
    tiles of 256 x 256 on 256 compute units), bf16 out; unsplit beside it, and
    kq_mx_gemm_static (the library's static array: fewer part slots, so fewer
    parts)."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    cfg, wcfg = synth.get_config("flux_mlp"), synth.get_weight_config("flux_w_down")
    M, N, K = 1024, wcfg.rows, cfg.d
    x, p, _ = synth.make_inputs(cfg, rows=M)
    w, _ = synth.make_weights(wcfg)
    pd = torch.from_numpy(p).cuda()
    qx, sx = kq.kq_quantize(torch.from_numpy(x.view(np.int16)).cuda(), pd)
    qw, sw = kq.kq_quantize_weights(torch.from_numpy(w.view(np.int16)).cuda(), pd)
    nbytes = kq.kq_mx_gemm_workspace_size(M, N, K)
    ws = torch.zeros(max(nbytes, 4096), dtype=torch.uint8, device="cuda")
    out, out_ws = (torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for _ in range(2))
    steps = max(8, args.steps // 10)
    out_st = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    legs = {}
    for name, fn in (("unsplit", lambda i: kq.kq_mx_gemm(qx, sx, qw, sw, out=out)),
                     ("split", lambda i: kq.kq_mx_gemm_ws(qx, sx, qw, sw, ws, out=out_ws)),
                     ("static", lambda i: kq.kq_mx_gemm_static(qx, sx, qw, sw, out=out_st))):
        ms = (timed(fn, steps, args.warmup, torch.cuda.current_stream()) if args.eager
              else timed_graph(fn, steps, min(args.warmup, 10)))
        leg = {"ms_per_call": round(ms, 6), "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        if hasattr(ms, "summary"):
            leg["timing"] = ms.summary(steps)
        legs[name] = leg
    torch.cuda.synchronize()
    rel = float((out_ws.float() - out.float()).norm() / out.float().norm())
    rel_st = float((out_st.float() - out.float()).norm() / out.float().norm())
    # K parts per tile: the workspace holds one 256 KiB slot per part of every tile;
    # the static array 128 slots
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    parts = (nbytes - 4096) // (tiles * 256 * 256 * 4) if nbytes else 1
    return {"workload": f"FLUX.1-schnell MLP down-projection, 1024 tokens: {M}x{N}x{K}, bf16 out",
            "entry": "kq_mx_gemm_ws", "workspace_bytes": nbytes,
            "parts": {"split": parts, "static": min(parts, 128 // tiles)}, **legs,
            "t_split_over_t_unsplit": round(legs["split"]["ms_per_call"] / legs["unsplit"]["ms_per_call"], 4),
            "t_static_over_t_unsplit": round(legs["static"]["ms_per_call"] / legs["unsplit"]["ms_per_call"], 4),
            "rel_diff_vs_unsplit": round(rel, 6), "static_rel_diff_vs_unsplit": round(rel_st, 6)}


def gemm_fused_timing(args):
    """The product with the quantizer in its prologue (kq_mx_gemm_fused: bf16 X and
    the factor parameters in, no MXFP4 activation operand in memory) beside the
    unfused pair (kq_quantize, then the product, in one graph) on the FLUX.1-schnell
    MLP up-projection, and on its first 256 weight rows (one tile column of Y, the
    case where the fused path quantizes each activation tile only once).  Both
    products run through their workspace entries (kq_mx_gemm_fused_ws and
    kq_mx_gemm_ws), which split few tiles in K parts; "fused_whole" is the fused
    product without a workspace."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    cfg, wcfg = synth.get_config("flux"), synth.get_weight_config("flux_w_mlp")
    x, p, _ = synth.make_inputs(cfg)
    w, pw = synth.make_weights(wcfg)
    xd, pd = torch.from_numpy(x.view(np.int16)).cuda(), torch.from_numpy(p).cuda()
    qw, sw = kq.kq_quantize_weights(torch.from_numpy(w.view(np.int16)).cuda(), torch.from_numpy(pw).cuda())
    M, K = xd.shape
    q = torch.empty((M, K // 2), dtype=torch.uint8, device="cuda")
    s = torch.empty((M, K // 32), dtype=torch.uint8, device="cuda")
    steps = max(8, args.steps // 10)
    res = {"workload": f"FLUX.1-schnell MLP up-projection from bf16 activations, {M}x{wcfg.rows}x{K} and "
                       f"{M}x256x{K}, bf16 out"}
    for N in (wcfg.rows, 256):
        qb, sb = qw[:N], sw[:N]
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        nf, nu = kq.kq_mx_gemm_fused_workspace_size(M, N, K), kq.kq_mx_gemm_workspace_size(M, N, K)
        wsf = torch.zeros(max(nf, 4096), dtype=torch.uint8, device="cuda")
        wsu = torch.zeros(max(nu, 4096), dtype=torch.uint8, device="cuda")
        legs = {}
        for name, fn in (("fused", lambda i: kq.kq_mx_gemm_fused_ws(xd, pd, qb, sb, wsf, out=out)),
                         ("fused_whole", lambda i: kq.kq_mx_gemm_fused(xd, pd, qb, sb, out=out)),
                         ("quantize_then_product", lambda i: (kq.kq_quantize(xd, pd, q=q, s=s),
                                                              kq.kq_mx_gemm_ws(q, s, qb, sb, wsu, out=out)))):
            ms = (timed(fn, steps, args.warmup, torch.cuda.current_stream()) if args.eager
                  else timed_graph(fn, steps, min(args.warmup, 10)))
            legs[name] = {"ms_per_call": round(ms, 6),
                          "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1)}
        legs["workspace_bytes"] = {"fused": nf, "product": nu}
        legs["t_fused_over_t_unfused"] = round(legs["fused"]["ms_per_call"] /
                                               legs["quantize_then_product"]["ms_per_call"], 4)
        res[f"n{N}"] = legs
    return res


def library_gemm_timing(args, qs, ss, qw, sw, ours):
    """The same MXFP4 x MXFP4 product through torch's scaled matmul (the vendor BLAS
    path; block-scaled products come out in bf16 only), timed the same way, with its
    relative difference to kq_mx_gemm's bf16 output (one bf16 unit in the last place
    on about half of the elements: the two round the fp32 sums differently);
    context only."""
    import torch
    try:
        wq, ws = qw.view(torch.float4_e2m1fn_x2).t(), sw.view(torch.float8_e8m0fnu).flatten()
        P = len(qs)
        aq = [q.view(torch.float4_e2m1fn_x2) for q in qs]
        as_ = [s.view(torch.float8_e8m0fnu).flatten() for s in ss]
        # `ours` holds the output of the graph's last step, on this set
        j_last = (max(8, args.steps // 10) - 1) % P
        lib_last = torch._scaled_mm(aq[j_last], wq, as_[j_last], ws, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        rel = float((lib_last.float() - ours.float()).norm() / ours.float().norm())

        def step(i):
            j = i % P
            torch._scaled_mm(aq[j], wq, as_[j], ws, out_dtype=torch.bfloat16)

        ms = timed_graph(step, max(8, args.steps // 10), min(args.warmup, 10))
        M, N, K = qs[0].shape[0], qw.shape[0], qs[0].shape[1] * 2
        return {"how": "torch._scaled_mm, float4_e2m1fn_x2 operands, float8_e8m0fnu block scales",
                "ms_per_call": round(ms, 6), "tflops": round(2.0 * M * N * K / (ms * 1e-3) / 1e12, 1),
                "rel_diff_vs_kq_mx_gemm": round(rel, 5)}
    except Exception as e:  # not every torch build has the fp4 scaled matmul
        return {"unavailable": f"{type(e).__name__}: {str(e)[:200]}"}


def weights_timing(args):
    """The weight side (W T^-1 then MXFP4 along the input channels) on the FLUX MLP
    up-projection W[12288, 3072] bf16, timed like the activation step over 4
    rotating buffer sets (300 MB, beyond the last-level cache)."""
    import torch

    import synth
    import online_activation_quantizer_amd as kq
    cfg = synth.get_weight_config("flux_w_mlp")
    sets = 4
    w0, p0 = synth.make_weights(cfg)
    g = torch.Generator(device="cuda")
    g.manual_seed(cfg.seed)
    ws = [torch.from_numpy(w0.view(np.int16)).cuda()]
    for _ in range(1, sets):
        ws.append((torch.randn((cfg.rows, cfg.d), generator=g, device="cuda") * cfg.std)
                  .to(torch.bfloat16).view(torch.int16))
    pd = torch.from_numpy(p0).cuda()
    qs = [torch.empty((cfg.rows, cfg.d // 2), dtype=torch.uint8, device="cuda") for _ in range(sets)]
    ss = [torch.empty((cfg.rows, cfg.d // 32), dtype=torch.uint8, device="cuda") for _ in range(sets)]

    def step(i):
        j = i % sets
        kq.kq_quantize_weights(ws[j], pd, q=qs[j], s=ss[j])

    steps = max(8, args.steps // 4)
    ms = (timed(step, steps, args.warmup, torch.cuda.current_stream()) if args.eager
          else timed_graph(step, steps, args.warmup))
    elems = cfg.rows * cfg.d
    gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    return {"workload": f"FLUX.1-schnell MLP up-projection weight {cfg.rows}x{cfg.d} bf16",
            "ms_per_call": round(ms, 6), "gelem_s": round(elems / (ms * 1e-3) / 1e9, 3),
            "gbs": round(gbs, 1), "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}


def cpu_leg(x0, p0, q0, s0, seconds):
    """The CPU leg, the only part of the bench that runs the oracle: the oracle timed
    on the host cores (cpu_baseline), the other rows' oracles on bounded samples,
    and the classification of one production step's output (q0, s0) against it."""
    out = {"cpu_baseline": cpu_baseline(x0, p0, seconds)}
    try:
        out["cpu_oracles"] = cpu_oracles(x0, p0, out["cpu_baseline"]["cores"])
    except Exception as e:  # the oracle is test infrastructure; its absence does not stop timing
        out["cpu_oracles"] = {"error": str(e)}
    try:
        import oracle
        _, _, y_o = oracle.quantize(x0, p0, want_y=True)
        st = oracle.classify(x0, y_o, q0, s0, 0, 1e-5)
        out["parity"] = {k: st[k] for k in ("exact", "excused", "unexcused", "elements")}
    except Exception as e:
        out["parity"] = {"error": str(e)}
    return out


def cpu_oracles(x0, p0, threads):
    """The oracle of every other row timed on bounded samples of the same workloads
    (host cores; about a second each), reported beside the GPU figures."""
    import oracle
    import synth

    def rate(fn, elems):
        t0 = time.perf_counter()
        fn()
        return elems / (time.perf_counter() - t0)

    rows = 256
    xs = np.ascontiguousarray(x0[:rows])
    d = x0.shape[1]
    out = {"threads": threads}
    one = sorted(rate(lambda: oracle.quantize(x0, p0, nthreads=1), x0.size) for _ in range(3))
    out["kq_quantize_1_thread_gelem_s"] = round(one[1] / 1e9, 5)
    out["kq_quantize_1_thread_sample"] = f"the full {x0.shape[0]}x{d} input, median of 3 passes"
    out["hq_quantize_gelem_s"] = round(rate(lambda: oracle.hadamard_quantize(xs, nthreads=threads), rows * d) / 1e9, 5)
    shift, scale = synth.make_modulation(1, d, np.random.default_rng(7))
    out["kq_norm_quantize_gelem_s"] = round(rate(
        lambda: oracle.norm_quantize(xs, p0, shift, scale, rows, 1e-6, nthreads=threads), rows * d) / 1e9, 5)
    w, pw = synth.make_weights(synth.get_weight_config("flux_w_mlp"))
    ws = np.ascontiguousarray(w[:rows])
    out["kq_quantize_weights_gelem_s"] = round(
        rate(lambda: oracle.quantize_weights(ws, pw, nthreads=threads), rows * d) / 1e9, 5)
    qa, sa, _ = oracle.quantize(xs, p0, nthreads=threads)
    qb, sb, _ = oracle.quantize_weights(ws, pw, nthreads=threads)
    out["w4a4_gemm_tflops"] = round(rate(lambda: oracle.mx_gemm(qa, sa, qb, sb), 2.0 * rows * rows * d) / 1e12, 6)
    out["sample"] = f"{rows} rows of each workload (the product: {rows} x {rows} x {d})"
    return out


def main():
    args = parse()
    global WARM_MS
    WARM_MS = args.warm_ms
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the quantizer needs no cross-GPU exchange: every (row, block) unit is independent, "
              "so each GPU quantizes its own shard of rows or of 32-channel blocks)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import synth
    import online_activation_quantizer_amd as kq

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    cfg = synth.get_config("flux")
    rows, d, nb = cfg.rows, cfg.d, cfg.nb
    elems = rows * d

    # pool of distinct buffer sets: set 0 from the host generator (parity-checked),
    # the rest drawn on the device with their own seeds
    x0, p0, m0 = synth.make_inputs(cfg)
    xs = [torch.from_numpy(x0.view(np.int16)).cuda()]
    ps = [torch.from_numpy(p0).cuda()]
    for i in range(1, args.pool):
        xs.append(synth.make_activations_device(cfg, cfg.seed + 1000 * i).view(torch.int16))
        ps.append(torch.from_numpy(synth.make_params(nb, np.random.default_rng(cfg.seed + 1000 * i))).cuda())
    qs = [torch.empty((rows, d // 2), dtype=torch.uint8, device="cuda") for _ in range(args.pool)]
    ss = [torch.empty((rows, d // 32), dtype=torch.uint8, device="cuda") for _ in range(args.pool)]
    m_dev = torch.from_numpy(m0).cuda()

    if args.variant == "mfma":
        ts = [kq.kq_expand_factors(p, kq.KQ_T_DENSE_BF16X3) for p in ps]
        tfmt, var = kq.KQ_T_DENSE_BF16X3, kq.KQ_MFMA
    else:
        ts, tfmt, var = ps, kq.KQ_T_PARAMS, kq.KQ_BUTTERFLY
    torch.cuda.synchronize()
    P = args.pool

    def kq_step(i):
        j = i % P
        kq.kq_quantize(xs[j], ts[j], tfmt, var, q=qs[j], s=ss[j])

    def sq_step(i):
        j = i % P
        kq.sq_quantize(xs[j], m_dev, q=qs[j], s=ss[j])

    def hq_step(i):
        j = i % P
        kq.hq_quantize(xs[j], q=qs[j], s=ss[j])

    if args.eager:
        ms = timed(kq_step, args.steps, args.warmup, stream)
        sq_ms = None if args.no_sq else timed(sq_step, args.steps, args.warmup, stream)
        hq_ms = None if args.no_sq else timed(hq_step, args.steps, args.warmup, stream)
    else:
        ms = timed_graph(kq_step, args.steps, args.warmup)
        sq_ms = None if args.no_sq else timed_graph(sq_step, args.steps, args.warmup)
        hq_ms = None if args.no_sq else timed_graph(hq_step, args.steps, args.warmup)

    # not the headline: independent steps on two streams, so that consecutive calls'
    # ramp-up and drain may overlap (graph replay only)
    ov_ms = None if args.no_overlap or args.eager else timed_graph_two_streams(kq_step, args.steps, args.warmup)
    weights = None if args.no_weights else weights_timing(args)
    norm = None if args.no_norm else norm_timing(args, cfg, xs, ps, qs, ss, ms)
    gemm = None if args.no_gemm else gemm_timing(args, qs, ss)
    if gemm is not None:
        gemm["few_tiles_split"] = gemm_split_timing(args)
        gemm["prologue_fused"] = gemm_fused_timing(args)
    mlp = None if args.no_mlp else mlp_timing(args)
    shard = None if args.no_shard or args.variant != "butterfly" else shard_timing(args, xs, ps)
    sweep = None if args.no_sweep else sweep_timing(args)
    quality = None
    if not args.no_quality:
        times = {"kq": round(ms * 1e3, 3)}
        if sq_ms is not None:
            times.update(sq=round(sq_ms * 1e3, 3), hq=round(hq_ms * 1e3, 3))
        quality = quality_leg(xs[0], ps[0], m_dev, times)
    ceiling = None if args.no_ceiling else stream_ceiling(args, xs, qs, ss, ms)

    gelem = elems / (ms * 1e-3) / 1e9
    gbs = elems * BYTES_PER_ELEM / (ms * 1e-3) / 1e9
    out = {
        "metric": METRIC,
        "value": round(gelem, 3),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 6),
        "timing": ms.summary(args.steps) if isinstance(ms, Timing) else None,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"FLUX.1-schnell-like joint-stream activations {rows}x{d} bf16, "
                               f"{nb} factor sets, {args.variant}",
                   "rows": rows, "d": d, "input": "bf16", "pool_sets": P,
                   "launch": "eager" if args.eager else "hip graph replay"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": measured_traffic() if args.variant == "butterfly" else None},
        "hbm_pct": round(100 * gbs / PEAK_HBM_GBS, 2),
    }
    if sq_ms is not None:
        sq_gbs = elems * BYTES_PER_ELEM / (sq_ms * 1e-3) / 1e9
        out["sq_baseline"] = {"ms_per_step": round(sq_ms, 6), "gbs": round(sq_gbs, 1),
                              "t_sq_over_t_kq": round(sq_ms / ms, 4), "timing": sq_ms.summary(args.steps)}
        hq_gbs = elems * BYTES_PER_ELEM / (hq_ms * 1e-3) / 1e9
        out["hadamard_baseline"] = {"ms_per_step": round(hq_ms, 6), "gbs": round(hq_gbs, 1),
                                    "t_hq_over_t_kq": round(hq_ms / ms, 4), "timing": hq_ms.summary(args.steps)}
        out["context"] = ("pages: on an MI350 the KroQuant quantizer kernel ran up to 14% faster "
                          "than a SmoothQuant kernel (shapes and timing method unstated)")
    if ov_ms is not None:
        ov_gbs = elems * BYTES_PER_ELEM / (ov_ms * 1e-3) / 1e9
        out["two_streams"] = {"ms_per_step": round(ov_ms, 6), "gbs": round(ov_gbs, 1),
                              "hbm_frac": round(ov_gbs / PEAK_HBM_GBS, 4),
                              "note": "independent steps alternating over two streams in one graph; "
                                      "not the headline, which times one call after another"}
    if ceiling is not None:
        out["stream_ceiling"] = ceiling
    if weights is not None:
        out["weights"] = weights
    if norm is not None:
        out["norm_fused"] = norm
    if gemm is not None:
        out["w4a4_gemm"] = gemm
    if mlp is not None:
        out["mlp_shape"] = mlp
    if shard is not None:
        out["shard_8way"] = shard
    if quality is not None:
        out["quality"] = quality
    if sweep is not None:
        out["sweep_28_calls"] = sweep
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu:
        kq_step(0)  # set 0 holds the host-generated input
        torch.cuda.synchronize()
        out.update(cpu_leg(x0, p0, qs[0].cpu().numpy(), ss[0].cpu().numpy(), args.cpu_seconds))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
