"""Weight side of the HIP path (W T^-1 per 32-input-channel block, then MXFP4
along the input channels) against the fp64 oracle, through the C ABI.

Same rule as the activation side: pre-quantization values within 1e-5 * max|w_block|
of the oracle, E8M0 scales and E2M1 codes bit-exact except where the oracle's value
is within that tolerance of a decision boundary (below 1e-4 of elements).
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say, verdict

pytestmark = pytest.mark.gpu


def run_weights(w: np.ndarray, p: np.ndarray):
    import torch
    wd, pd = dev(w), dev(p)
    q, s = kq.kq_quantize_weights(wd, pd)
    q2, s2, yd = kq.kq_weights_debug(wd, pd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "debug and production kernels disagree"
    return host(q), host(s), host(yd)


@pytest.mark.parametrize("name", list(synth.WEIGHT_CONFIGS))
def test_weights_parity(name):
    cfg = synth.get_weight_config(name)
    say(f"[weights parity] {name} {cfg.rows}x{cfg.d} {cfg.dtype}")
    w, p = synth.make_weights(cfg)
    q, s, y = run_weights(w, p)
    _, _, y_o = oracle.quantize_weights(w, p, want_y=True)
    st = verdict(w, y_o, q, s, y_c=y)
    say(f"  {st}")
    assert st["pass"], st


def test_weights_identity_is_plain_mxfp4():
    cfg = synth.get_weight_config("pixart_w")
    say("[weights identity] pixart_w")
    w, _ = synth.make_weights(cfg)
    q, s, y = run_weights(w, synth.make_identity_params(cfg.nb))
    wf = synth.f32_from_bf16_bits(w)
    q_o, s_o = oracle.encode(wf.astype(np.float64))
    assert np.array_equal(y, wf)
    assert np.array_equal(q, q_o) and np.array_equal(s, s_o)


def test_weights_ragged_and_pitched():
    import torch
    say("[weights ragged] 37 x 96 in a 160-wide fp32 buffer")
    rng = np.random.default_rng(31)
    full = rng.normal(0, 0.05, size=(37, 160)).astype(np.float32)
    p = synth.make_params(3, rng)
    wd = dev(full)[:, :96]
    q = torch.full((37, 64), 0xAB, dtype=torch.uint8, device="cuda")
    s = torch.full((37, 16), 0xCD, dtype=torch.uint8, device="cuda")
    kq.kq_quantize_weights(wd, dev(p), q=q[:, :48], s=s[:, :3])
    torch.cuda.synchronize()
    qh, sh = host(q), host(s)
    assert np.all(qh[:, 48:] == 0xAB) and np.all(sh[:, 3:] == 0xCD)
    w = np.ascontiguousarray(full[:, :96])
    _, _, y_o = oracle.quantize_weights(w, p, want_y=True)
    st = verdict(w, y_o, np.ascontiguousarray(qh[:, :48]), np.ascontiguousarray(sh[:, :3]))
    assert st["pass"], st


def test_weight_and_activation_sides_cancel():
    """W' (T x) = W x on the GPU's own fp32 outputs of both sides (before
    quantization): the product of the two transformed operands matches the plain
    product within the fp32 error of two 6-operation transforms."""
    cfg_x = synth.get_config("pixart")
    cfg_w = synth.get_weight_config("pixart_w")
    say("[weights cancel] pixart activations x pixart_w weights")
    x, p, _ = synth.make_inputs(cfg_x, rows=512)
    w, _ = synth.make_weights(cfg_w)
    xd, wd, pd = dev(x), dev(w), dev(p)
    _, _, yx = kq.kq_transform_debug(xd, pd)
    _, _, yw = kq.kq_weights_debug(wd, pd)
    import torch
    torch.cuda.synchronize()
    yx, yw = host(yx).astype(np.float64), host(yw).astype(np.float64)
    xf = synth.f32_from_bf16_bits(x).astype(np.float64)
    wf = synth.f32_from_bf16_bits(w).astype(np.float64)
    lhs, rhs = yx @ yw.T, xf @ wf.T
    bound = 1e-5 * (np.abs(xf) @ np.abs(wf).T)
    err = np.abs(lhs - rhs)
    say(f"  max err / bound = {float(np.max(err / bound)):.3g}")
    assert np.all(err <= bound)
