"""LayerNorm + adaptive-norm modulation fused ahead of the block transform and
MXFP4 (kq_norm_quantize) against the fp64 oracle, through the C ABI.

The transform's input is the normalized, modulated row h, so the fp32 rule is
applied to it: pre-quantization values within 1e-5 * max|h_block| of the oracle;
codes and scales exact outside that window (excused below 1e-4 of elements).
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say, verdict

pytestmark = pytest.mark.gpu

# (config, tokens per modulation vector or None for a plain LayerNorm)
CASES = [("tiny", 64), ("pixart", 1024), ("sana", None), ("flux", 4608), ("flux_mlp", 4608)]


def run_norm(x, p, shift, scale, rps, eps):
    import torch
    xd, pd = dev(x), dev(p)
    sh = None if shift is None else dev(shift)
    sc = None if scale is None else dev(scale)
    q, s = kq.kq_norm_quantize(xd, pd, sh, sc, rps, eps)
    q2, s2, yd = kq.kq_norm_debug(xd, pd, sh, sc, rps, eps)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "debug and production kernels disagree"
    return host(q), host(s), host(yd)


def check(x, p, shift, scale, rps, eps, label):
    q, s, y = run_norm(x, p, shift, scale, rps, eps)
    _, _, h_o, y_o = oracle.norm_quantize(x, p, shift, scale, rps, eps, want_y=True)
    st = verdict(h_o.astype(np.float32), y_o, q, s, y_c=y)
    say(f"  {label}: {st}")
    assert st["pass"], st


@pytest.mark.parametrize("name,rps", CASES)
def test_norm_parity(name, rps):
    cfg = synth.get_config(name)
    say(f"[norm parity] {name} {cfg.rows}x{cfg.d} {cfg.dtype} rows/sample={rps}")
    x, p, _ = synth.make_inputs(cfg)
    shift = scale = None
    if rps is not None:
        shift, scale = synth.make_modulation(-(-cfg.rows // rps), cfg.d, np.random.default_rng(cfg.seed + 77))
    check(x, p, shift, scale, rps, 1e-6, name)


@pytest.mark.parametrize("rows,d,rps,eps", [(1, 32, 1, 1e-6), (5, 96, 2, 0.0), (130, 3104, 7, 1e-5),
                                            (64, 64, 1000, 0.5), (3, 1024, 1, 1e-6),
                                            (9, 16384, 2, 1e-6), (4, 16352, 3, 1e-6)])
def test_norm_ragged_and_edge(rows, d, rps, eps):
    say(f"[norm edge] rows={rows} d={d} rps={rps} eps={eps}")
    rng = np.random.default_rng(rows + d)
    x = synth.bf16_bits_from_f32((rng.normal(size=(rows, d)) * 2 + rng.normal(0, 3, size=(rows, 1)))
                                 .astype(np.float32))
    p = synth.make_params(d // 32, rng)
    shift, scale = synth.make_modulation(-(-rows // rps), d, rng)
    check(x, p, shift, scale, rps, eps, f"{rows}x{d}")


def test_norm_constant_row_with_eps():
    # a constant row normalizes to exactly 0 (x - mu = 0): y = T_b shift, with eps > 0
    say("[norm constant row]")
    x = np.full((4, 64), 2.5, np.float32)
    p = synth.make_params(2, np.random.default_rng(3))
    shift, scale = synth.make_modulation(1, 64, np.random.default_rng(4))
    check(x, p, shift, scale, 4, 1e-6, "constant")


def test_norm_pitched_with_canaries():
    import torch
    say("[norm pitched]")
    rng = np.random.default_rng(9)
    full = synth.bf16_bits_from_f32(rng.normal(size=(33, 160)).astype(np.float32))
    p = synth.make_params(3, rng)
    xd = dev(full)[:, :96]
    q = torch.full((33, 64), 0x3C, dtype=torch.uint8, device="cuda")
    s = torch.full((33, 8), 0xC3, dtype=torch.uint8, device="cuda")
    kq.kq_norm_quantize(xd, dev(p), q=q[:, :48], s=s[:, :3])
    torch.cuda.synchronize()
    qh, sh = host(q), host(s)
    assert np.all(qh[:, 48:] == 0x3C) and np.all(sh[:, 3:] == 0xC3)
    x = np.ascontiguousarray(full[:, :96])
    _, _, h_o, y_o = oracle.norm_quantize(x, p, want_y=True)
    st = verdict(h_o.astype(np.float32), y_o, np.ascontiguousarray(qh[:, :48]), np.ascontiguousarray(sh[:, :3]))
    assert st["pass"], st
