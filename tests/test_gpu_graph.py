"""The quantizer launched from a captured HIP graph: every replay (with eager
work and synchronizations between replays) must reproduce the eager result
bit for bit.  bench.py times its steps through such a graph."""
import numpy as np
import pytest

import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, say

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    cfg = synth.get_config("flux")
    say("[graph] flux x2 sets, kq + sq captured")
    sets = []
    for i in range(2):
        x, p, m = synth.make_inputs(cfg, rows=1024, seed=500 + i)
        sets.append((dev(x), dev(p), dev(m)))
    outs = [(torch.empty((1024, cfg.d // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((1024, cfg.d // 32), dtype=torch.uint8, device="cuda"),
             torch.empty((1024, cfg.d // 2), dtype=torch.uint8, device="cuda"),
             torch.empty((1024, cfg.d // 32), dtype=torch.uint8, device="cuda")) for _ in sets]
    eager = []
    for (x, p, m) in sets:
        q, s = kq.kq_quantize(x, p)
        q2, s2 = kq.sq_quantize(x, m)
        eager.append((q.clone(), s.clone(), q2.clone(), s2.clone()))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            for (x, p, m), (q, s, q2, s2) in zip(sets, outs):
                kq.kq_quantize(x, p, q=q, s=s)
                kq.sq_quantize(x, m, q=q2, s=s2)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(4):
        for o in outs:
            for t in o:
                t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            for a, b in zip(o, e):
                assert torch.equal(a, b), f"replay {rep} differs from eager"


def test_graph_replays_of_every_entry_point():
    """Weights, block Hadamard, fused normalization and the W4A4 product captured in one
    graph with the quantizer: every replay equals the eager run, bit for bit."""
    import torch
    cfg = synth.get_config("pixart")
    wcfg = synth.get_weight_config("pixart_w")
    say("[graph] every entry point, pixart shapes")
    x, p, _ = synth.make_inputs(cfg, rows=512, seed=77)
    w, _ = synth.make_weights(wcfg)
    shift, scale = synth.make_modulation(2, cfg.d, np.random.default_rng(78))
    xd, pd, wd, shd, scd = dev(x), dev(p), dev(w), dev(shift), dev(scale)

    def run(o=None):
        o = o or {}

        def qs(k):
            return dict(zip(("q", "s"), o[k])) if k in o else {}
        o["kq"] = kq.kq_quantize(xd, pd, **qs("kq"))
        o["w"] = kq.kq_quantize_weights(wd, pd, **qs("w"))
        o["hq"] = kq.hq_quantize(xd, **qs("hq"))
        o["norm"] = kq.kq_norm_quantize(xd, pd, shd, scd, 256, 1e-6, **qs("norm"))
        o["y"] = kq.kq_mx_gemm(o["kq"][0], o["kq"][1], o["w"][0], o["w"][1], out=o.get("y"))
        return o

    eager = run()
    torch.cuda.synchronize()
    ref = {k: (tuple(t.clone() for t in v) if isinstance(v, tuple) else v.clone()) for k, v in eager.items()}
    outs = {k: (tuple(torch.empty_like(t) for t in v) if isinstance(v, tuple) else torch.empty_like(v))
            for k, v in eager.items()}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g):
            run(outs)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for v in outs.values():
            for t in (v if isinstance(v, tuple) else (v,)):
                t.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in ref:
            a = outs[k] if isinstance(outs[k], tuple) else (outs[k],)
            b = ref[k] if isinstance(ref[k], tuple) else (ref[k],)
            for u, v in zip(a, b):
                assert torch.equal(u, v), f"replay {rep}: {k} differs from eager"


def test_norm_and_gemm_deterministic_across_streams():
    import torch
    cfg = synth.get_config("flux")
    say("[determinism] norm + gemm, two streams")
    x, p, _ = synth.make_inputs(cfg, rows=768, seed=91)
    shift, scale = synth.make_modulation(1, cfg.d, np.random.default_rng(92))
    xd, pd, shd, scd = dev(x), dev(p), dev(shift), dev(scale)
    q1, s1 = kq.kq_norm_quantize(xd, pd, shd, scd, 768, 1e-6)
    y1 = kq.kq_mx_gemm(q1, s1, q1[:300], s1[:300])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2, s2 = kq.kq_norm_quantize(xd, pd, shd, scd, 768, 1e-6)
        y2 = kq.kq_mx_gemm(q2, s2, q2[:300], s2[:300])
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2) and torch.equal(y1, y2)
