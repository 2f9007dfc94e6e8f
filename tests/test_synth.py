"""The seeded input generators: determinism and the stated value model."""
import numpy as np

import synth


def test_deterministic_and_seeded():
    cfg = synth.get_config("pixart")
    a = synth.make_inputs(cfg, rows=32)
    b = synth.make_inputs(cfg, rows=32)
    c = synth.make_inputs(cfg, rows=32, seed=99)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
    assert not np.array_equal(a[0], c[0])


def test_shapes_and_dtypes():
    for name, cfg in synth.CONFIGS.items():
        x, p, m = synth.make_inputs(cfg, rows=4)
        assert x.shape == (4, cfg.d)
        assert x.dtype == (np.uint16 if cfg.dtype == "bf16" else np.float32)
        assert p.shape == (cfg.nb, 5, 3) and p.dtype == np.float32
        assert m.shape == (cfg.d,) and m.dtype == np.float32
        assert np.all(p[..., 1] > 0)


def test_outlier_channels_and_bf16_rounding():
    cfg = synth.get_config("flux")
    assert cfg.n_outliers == 31
    x, _, _ = synth.make_inputs(cfg, rows=512)
    xf = synth.f32_from_bf16_bits(x)
    col = np.abs(xf).mean(axis=0)
    big = np.sort(col)[::-1]
    # 31 outlier channels are ~40x the rest
    assert big[30] > 10 * np.median(col) and big[31] < 3 * np.median(col)
    # bf16 round trip is the identity on already-rounded values
    assert np.array_equal(synth.bf16_bits_from_f32(xf), x)
    # round to nearest even at a tie: 1 + 2^-8 is halfway between bf16 1 and 1 + 2^-7
    assert synth.bf16_bits_from_f32(np.array([1 + 2 ** -8], np.float32))[0] == 0x3F80
    assert synth.bf16_bits_from_f32(np.array([1 + 3 * 2 ** -8], np.float32))[0] == 0x3F82


def test_factor_distribution():
    p = synth.make_params(20000, np.random.default_rng(0))
    assert abs(p[..., 0].std() - 0.5) < 0.01 and abs(p[..., 2].std() - 0.5) < 0.01
    assert abs(np.log(p[..., 1]).std() - 0.3) < 0.01


def test_weights_seeded_and_shaped():
    cfg = synth.get_weight_config("tiny_w")
    w1, p1 = synth.make_weights(cfg)
    w2, p2 = synth.make_weights(cfg)
    assert w1.shape == (cfg.rows, cfg.d) and w1.dtype == np.float32
    assert p1.shape == (cfg.nb, 5, 3)
    assert np.array_equal(w1, w2) and np.array_equal(p1, p2)
    assert 0.01 < float(np.std(w1)) < 0.04
    wb, _ = synth.make_weights(synth.get_weight_config("pixart_w"))
    assert wb.dtype == np.uint16
