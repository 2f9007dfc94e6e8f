"""The fixed block-Hadamard comparison transform (hq_quantize) against the fp64
oracle, through the C ABI; same rule as the learned transform (pre-quantization
values within 1e-5 * max|x_block|, codes and scales exact outside that window)."""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, run_kq, say, verdict

pytestmark = pytest.mark.gpu


def run_hq(x: np.ndarray):
    import torch
    xd = dev(x)
    q, s = kq.hq_quantize(xd)
    q2, s2, yd = kq.hq_transform_debug(xd)
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2), "debug and production kernels disagree"
    return host(q), host(s), host(yd)


@pytest.mark.parametrize("name", ["tiny", "pixart", "sana", "flux"])
def test_hadamard_parity(name):
    cfg = synth.get_config(name)
    say(f"[hadamard parity] {name} {cfg.rows}x{cfg.d} {cfg.dtype}")
    x, _, _ = synth.make_inputs(cfg)
    q, s, y = run_hq(x)
    _, _, y_o = oracle.hadamard_quantize(x, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y)
    say(f"  {st}")
    assert st["pass"], st


@pytest.mark.parametrize("rows", [1, 7, 300])
def test_hadamard_ragged_and_pitched(rows):
    import torch
    say(f"[hadamard ragged] rows={rows}")
    rng = np.random.default_rng(rows)
    full = synth.bf16_bits_from_f32(rng.normal(0, 3, size=(rows, 224)).astype(np.float32))
    xd = dev(full)[:, :160]
    q = torch.full((rows, 96), 0x5A, dtype=torch.uint8, device="cuda")
    s = torch.full((rows, 16), 0xA5, dtype=torch.uint8, device="cuda")
    kq.hq_quantize(xd, q=q[:, :80], s=s[:, :5])
    torch.cuda.synchronize()
    qh, sh = host(q), host(s)
    assert np.all(qh[:, 80:] == 0x5A) and np.all(sh[:, 5:] == 0xA5)
    x = np.ascontiguousarray(full[:, :160])
    _, _, y_o = oracle.hadamard_quantize(x, want_y=True)
    st = verdict(x, y_o, np.ascontiguousarray(qh[:, :80]), np.ascontiguousarray(sh[:, :5]))
    assert st["pass"], st


def test_hadamard_twice_is_identity_on_gpu():
    import torch
    say("[hadamard involution]")
    rng = np.random.default_rng(5)
    x = rng.normal(size=(64, 256)).astype(np.float32)
    _, _, y = kq.hq_transform_debug(dev(x))
    _, _, z = kq.hq_transform_debug(y)
    torch.cuda.synchronize()
    err = np.abs(host(z) - x).max()
    say(f"  max |H H x - x| = {err:.3g}")
    assert err <= 1e-6 * np.abs(x).max()


def test_45_degree_rotation_factors_match_hadamard_up_to_signs():
    """The Kronecker product of five 45-degree rotations [[c, s], [-s, c]] is the
    Sylvester Hadamard H_32 / sqrt(32) with some rows negated, so the butterfly with
    those factors and the Hadamard path must give the same scales and the same code
    magnitudes (sign bits may differ), except where fp32 rounding of the two
    evaluation orders straddles a decision boundary.  Against the oracle: no
    unexcused mismatch and the pre-quantization bound everywhere.  The excused
    count is a known excess over the 1e-4 that every workload's own factors stay
    under: 1,903 of 14,155,776 elements (1.34e-4), measured; this input and the
    kernel's arithmetic are deterministic, so the assert holds it to 1.4e-4.  The
    rotations spread each block's outlier over all 32 values (so the window, 1e-5
    of the block's largest input, is wide next to them) and the butterfly rounds
    five times where the Hadamard path's sums are exact."""
    import torch
    cfg = synth.get_config("flux")
    say("[rotation vs hadamard] flux")
    x, _, _ = synth.make_inputs(cfg)
    pr = synth.make_rotation_params(cfg.nb)
    qk, sk, yk = run_kq(x, pr)
    xd = dev(x)
    qh, sh = kq.hq_quantize(xd)
    torch.cuda.synchronize()
    qh, sh = host(qh), host(sh)
    mag = lambda q: np.stack([q & 7, (q >> 4) & 7], -1)
    scale_diff = np.count_nonzero(sk != sh)
    code_diff = np.count_nonzero(mag(qk) != mag(qh))
    say(f"  scale bytes differing {scale_diff} of {sk.size}, code magnitudes {code_diff} of {x.size}")
    assert scale_diff <= 1e-4 * sk.size and code_diff <= 1e-4 * x.size
    _, _, y_o = oracle.quantize(x, pr, want_y=True)
    st = verdict(x, y_o, qk, sk, y_c=yk)
    say(f"  oracle: {st}")
    assert st["unexcused"] == 0 and st["prequant_violations"] == 0, st
    assert st["excused"] <= 1.4e-4 * st["elements"], st
