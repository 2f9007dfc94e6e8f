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
