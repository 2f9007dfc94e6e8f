"""Seeded random shapes, input dtypes, magnitudes and pitches for the quantizers
(kq_quantize, hq_quantize, sq_quantize, kq_quantize_weights) and the fused norm
(kq_norm_quantize), through the C ABI, against the fp64 oracle under the parity
rule; the same call through padded row pitches gives the same bytes and leaves the
padding of the outputs untouched.

Cases draw 1-1499 rows and 1-159 blocks (so the lane count, a multiple of nb, takes
many grid shapes and row strides), bf16 or fp32 input, Student-t values scaled by
2^-12 .. 2^12 (scale bytes far from 127) around a per-row mean, row pitches padded
by 0-3 x 16 bytes, code pitches by 0-2 x 16 bytes and scale pitches by 0-6 bytes.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say, verdict

pytestmark = pytest.mark.gpu

N_CASES = 12
CANARY_Q, CANARY_S = 0xA5, 0x5A


def draw(case):
    rng = np.random.default_rng(31337 + case)
    rows, nb = int(rng.integers(1, 1500)), int(rng.integers(1, 160))
    fp32 = bool(rng.integers(0, 2))
    mag = float(2.0 ** rng.uniform(-12, 12))
    d = 32 * nb
    xf = ((rng.standard_t(4, size=(rows, d)) + rng.normal(0, 2, size=(rows, 1))) * mag).astype(np.float32)
    x = xf if fp32 else synth.bf16_bits_from_f32(xf)
    pads = (int(rng.integers(0, 4)), int(rng.integers(0, 3)), int(rng.integers(0, 7)))
    return rng, x, fp32, pads


def pitched_input(x, fp32, pad16):
    """x in the leading columns of a device buffer 16 pad16 bytes wider per row whose
    padding holds huge finite values (never to be read)."""
    import torch
    rows, d = x.shape
    extra = pad16 * (4 if fp32 else 8)
    if fp32:
        buf = torch.full((rows, d + extra), 3.0e38, dtype=torch.float32, device="cuda")
    else:
        buf = torch.full((rows, d + extra), 0x7F7F, dtype=torch.int16, device="cuda")  # bf16 3.4e38
    buf[:, :d] = dev(x)
    return buf[:, :d]


def pitched_outputs(rows, nb, pq16, ps):
    import torch
    qb = torch.full((rows, 16 * nb + 16 * pq16), CANARY_Q, dtype=torch.uint8, device="cuda")
    sb = torch.full((rows, nb + ps), CANARY_S, dtype=torch.uint8, device="cuda")
    return qb, sb


def same_through_pitches(call, x, fp32, pads, q, s, label):
    """call(x_view, q_view, s_view) on padded buffers: the bytes of the contiguous call
    and untouched padding."""
    import torch
    rows, d = x.shape
    nb = d // 32
    xv = pitched_input(x, fp32, pads[0])
    qb, sb = pitched_outputs(rows, nb, pads[1], pads[2])
    call(xv, qb[:, :16 * nb], sb[:, :nb])
    torch.cuda.synchronize()
    qh, sh = host(qb), host(sb)
    assert np.array_equal(qh[:, :16 * nb], q) and np.array_equal(sh[:, :nb], s), f"{label}: pitched call differs"
    assert np.all(qh[:, 16 * nb:] == CANARY_Q) and np.all(sh[:, nb:] == CANARY_S), f"{label}: padding written"


@pytest.mark.parametrize("case", range(N_CASES))
def test_quantizers_random_shapes(case):
    import torch
    rng, x, fp32, pads = draw(case)
    rows, d = x.shape
    nb = d // 32
    say(f"[sweep {case}] {rows}x{d} {'fp32' if fp32 else 'bf16'} pads {pads}")
    xd = dev(x)
    # KroQuant transform
    p = synth.make_params(nb, rng)
    pd = dev(p)
    q, s = kq.kq_quantize(xd, pd)
    q2, s2, yd = kq.kq_transform_debug(xd, pd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, host(q), host(s), y_c=host(yd))
    say(f"  kq: {st}")
    assert st["pass"], st
    same_through_pitches(lambda xv, qv, sv: kq.kq_quantize(xv, pd, q=qv, s=sv), x, fp32, pads,
                         host(q), host(s), "kq")
    # block Hadamard
    q, s = kq.hq_quantize(xd)
    q2, s2, yd = kq.hq_transform_debug(xd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, y_o = oracle.hadamard_quantize(x, want_y=True)
    st = verdict(x, y_o, host(q), host(s), y_c=host(yd))
    say(f"  hq: {st}")
    assert st["pass"], st
    same_through_pitches(lambda xv, qv, sv: kq.hq_quantize(xv, q=qv, s=sv), x, fp32, pads,
                         host(q), host(s), "hq")
    # SmoothQuant
    m = np.exp(rng.normal(0, 0.5, size=d)).astype(np.float32)
    md = dev(m)
    q, s = kq.sq_quantize(xd, md)
    q2, s2, yd = kq.sq_transform_debug(xd, md)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, y_o = oracle.sq_quantize(x, m, want_y=True)
    st = verdict(x, y_o, host(q), host(s), y_c=host(yd))
    say(f"  sq: {st}")
    assert st["pass"], st
    same_through_pitches(lambda xv, qv, sv: kq.sq_quantize(xv, md, q=qv, s=sv), x, fp32, pads,
                         host(q), host(s), "sq")


@pytest.mark.parametrize("case", range(N_CASES))
def test_weights_random_shapes(case):
    """The weight side (W T^-1, then MXFP4) on the same draws, as weight matrices."""
    import torch
    rng, w, fp32, pads = draw(100 + case)
    rows, d = w.shape
    nb = d // 32
    say(f"[weights sweep {case}] {rows}x{d} {'fp32' if fp32 else 'bf16'} pads {pads}")
    p = synth.make_params(nb, rng)
    wd, pd = dev(w), dev(p)
    q, s = kq.kq_quantize_weights(wd, pd)
    q2, s2, yd = kq.kq_weights_debug(wd, pd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, y_o = oracle.quantize_weights(w, p, want_y=True)
    st = verdict(w, y_o, host(q), host(s), y_c=host(yd))
    say(f"  {st}")
    assert st["pass"], st
    same_through_pitches(lambda xv, qv, sv: kq.kq_quantize_weights(xv, pd, q=qv, s=sv), w, fp32, pads,
                         host(q), host(s), "weights")


@pytest.mark.parametrize("case", range(N_CASES))
def test_norm_random_shapes(case):
    """The fused norm on random row counts, widths (the half-wave kernel up to 4096
    channels, the LDS-meeting kernel above and for fp32), samples per call and eps."""
    import torch
    rng = np.random.default_rng(4711 + case)
    rows, nb = int(rng.integers(1, 700)), int(rng.integers(1, 200))
    fp32 = bool(rng.integers(0, 2))
    d = 32 * nb
    rps = int(rng.integers(1, rows + 1)) if rng.integers(0, 4) else None
    eps = float(rng.choice([0.0, 1e-6, 1e-5, 0.1]))
    xf = (rng.normal(size=(rows, d)) * rng.uniform(0.05, 20) + rng.normal(0, 3, size=(rows, 1))).astype(np.float32)
    x = xf if fp32 else synth.bf16_bits_from_f32(xf)
    p = synth.make_params(nb, rng)
    shift = scale = None
    if rps is not None:
        shift, scale = synth.make_modulation(-(-rows // rps), d, rng)
    say(f"[norm sweep {case}] {rows}x{d} {'fp32' if fp32 else 'bf16'} rps={rps} eps={eps}")
    xd, pd = dev(x), dev(p)
    sh = None if shift is None else dev(shift)
    sc = None if scale is None else dev(scale)
    q, s = kq.kq_norm_quantize(xd, pd, sh, sc, rps, eps)
    q2, s2, yd = kq.kq_norm_debug(xd, pd, sh, sc, rps, eps)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, h_o, y_o = oracle.norm_quantize(x, p, shift, scale, rps, eps, want_y=True)
    st = verdict(h_o.astype(np.float32), y_o, host(q), host(s), y_c=host(yd))
    say(f"  {st}")
    assert st["pass"], st
