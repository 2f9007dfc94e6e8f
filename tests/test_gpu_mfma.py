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


def test_mfma_rejects_fp32_input():
    x = np.zeros((4, 64), np.float32)
    p = synth.make_identity_params(2)
    with pytest.raises(kq.KQError):
        run_kq(x, p, variant=kq.KQ_MFMA)
