"""The batched FLUX-like sweep: 28 layer-shaped calls alternating X[18432, 3072]
and X[18432, 12288] (bf16), each with its own inputs and factor set, run at full
size in the production launch configuration.  Inputs are drawn on the GPU
(seeded); sampled rows are checked against the oracle one by one."""
import numpy as np
import pytest

import oracle
import synth
from synth.configs import SWEEP_CALLS, sweep_call
import online_activation_quantizer_amd as kq
from gpu_util import host, say, verdict

pytestmark = pytest.mark.gpu


def test_sweep_28_calls_sampled_rows():
    import torch
    torch.cuda.synchronize()
    total_bad = 0
    for i in range(SWEEP_CALLS):
        cfg = sweep_call(i)
        say(f"[sweep] call {i}: {cfg.rows}x{cfg.d}")
        xd = synth.make_activations_device(cfg, cfg.seed)
        p = synth.make_params(cfg.nb, np.random.default_rng(cfg.seed))
        pd = torch.from_numpy(p).cuda()
        q, s = kq.kq_quantize(xd, pd)
        rng = np.random.default_rng(cfg.seed + 1)
        rows = np.unique(np.concatenate([[0, cfg.rows - 1], rng.choice(cfg.rows, 14, replace=False)]))
        ridx = torch.from_numpy(rows).cuda()
        x_s = host(xd.index_select(0, ridx).contiguous())
        q_s, s_s = host(q.index_select(0, ridx)), host(s.index_select(0, ridx))
        _, _, y_o = oracle.quantize(x_s, p, want_y=True)
        st = verdict(x_s, y_o, q_s, s_s)
        total_bad += st["unexcused"]
        assert st["pass"], (i, st)
        del xd, q, s
    assert total_bad == 0
