"""Parity of the matrix-core variant (bf16 input, T_b as three bf16 parts, fp32
accumulation) with the fp64 oracle.

Its tolerance is the bf16 matrix-core rule: pre-quantization values within
8e-3 * max|y_block| of the oracle; codes and scales bit-exact except within that
tolerance of a decision boundary, below 1e-4 of elements.  The three-part split
carries fp32 accuracy in T, so the test also reports the fp32 rule's counts.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, run_kq, say, verdict

pytestmark = pytest.mark.gpu

MFMA_TOL = (1, 8e-3)


@pytest.mark.parametrize("name", ["pixart", "sana", "flux", "flux_mlp"])
def test_mfma_parity_full_config(name):
    cfg = synth.get_config(name)
    say(f"[mfma parity] {name} {cfg.rows}x{cfg.d}")
    x, p, _ = synth.make_inputs(cfg)
    q, s, y = run_kq(x, p, variant=kq.KQ_MFMA)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y, tol=MFMA_TOL)
    st32 = verdict(x, y_o, q, s, y_c=y)
    say(f"  bf16 rule {st}\n  fp32 rule {st32}")
    assert st["pass"], st


def test_mfma_identity_is_plain_mxfp4_exactly():
    cfg = synth.get_config("pixart")
    say("[mfma identity] pixart")
    x, _, _ = synth.make_inputs(cfg, rows=1000)
    q, s, y = run_kq(x, synth.make_identity_params(cfg.nb), variant=kq.KQ_MFMA)
    q_o, s_o = oracle.encode(synth.f32_from_bf16_bits(x).astype(np.float64))
    assert np.array_equal(y, synth.f32_from_bf16_bits(x))
    assert np.array_equal(s, s_o) and np.array_equal(q, q_o)


@pytest.mark.parametrize("rows", [1, 31, 33, 100])
@pytest.mark.parametrize("d", [32, 96, 3104])
def test_mfma_ragged(rows, d):
    say(f"[mfma ragged] rows={rows} d={d}")
    rng = np.random.default_rng(rows * 31 + d)
    x = synth.bf16_bits_from_f32(rng.normal(size=(rows, d)).astype(np.float32) * 4)
    p = synth.make_params(d // 32, rng)
    q, s, y = run_kq(x, p, variant=kq.KQ_MFMA)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y, tol=MFMA_TOL)
    assert st["pass"], st


def test_mfma_pitched_with_canaries():
    """Padded pitches on x, q and s: the padding of x holds huge values that must never
    be read, and the bytes past d/2 and d/32 in q and s must stay untouched; the
    result equals the unpitched call byte for byte.  97 blocks leave a last group of
    one block, 77 rows a partial last tile."""
    import torch
    rows, d = 77, 3104
    say(f"[mfma pitch] rows={rows} d={d}")
    rng = np.random.default_rng(97)
    x = synth.bf16_bits_from_f32(rng.normal(size=(rows, d)).astype(np.float32) * 4)
    p = synth.make_params(d // 32, rng)
    q0, s0, _ = run_kq(x, p, debug=False, variant=kq.KQ_MFMA)
    xw = np.zeros((rows, d + 64), np.uint16)
    xw[:, :d] = x
    xw[:, d:] = synth.bf16_bits_from_f32(np.full((rows, 64), 3e38, np.float32))
    t = kq.kq_expand_factors(dev(p), kq.KQ_T_DENSE_BF16X3)
    qbuf = torch.full((rows, d // 2 + 48), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows, d // 32 + 9), 0x5A, dtype=torch.uint8, device="cuda")
    kq.kq_quantize(dev(xw)[:, :d], t, kq.KQ_T_DENSE_BF16X3, kq.KQ_MFMA, q=qbuf[:, : d // 2], s=sbuf[:, : d // 32])
    torch.cuda.synchronize()
    qb, sb = qbuf.cpu().numpy(), sbuf.cpu().numpy()
    assert np.array_equal(qb[:, : d // 2], q0) and np.array_equal(sb[:, : d // 32], s0)
    assert np.all(qb[:, d // 2:] == 0xA5) and np.all(sb[:, d // 32:] == 0x5A)


def test_mfma_rejects_fp32_input():
    x = np.zeros((4, 64), np.float32)
    p = synth.make_identity_params(2)
    with pytest.raises(kq.KQError):
        run_kq(x, p, variant=kq.KQ_MFMA)
