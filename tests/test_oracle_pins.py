"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Sources: KroQuant abstract (arXiv 2607.21446) and its researchpod summary (method
paragraph) for the block transform; OCP MX v1.0 for MXFP4.  Each test names
the fact it checks.  No GPU is used.
"""
import os
import subprocess

import numpy as np
import pytest

import synth

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def rand_params(nb, seed):
    return synth.make_params(nb, np.random.default_rng(seed))


def f32_block(vals, d=32):
    x = np.zeros((1, d), np.float32)
    x[0, : len(vals)] = vals
    return x


# ---------------------------------------------------------------- factors / T_b

def test_factor_is_l_times_u(oq):
    # L = [[1,0],[l,1]], U = [[u,v],[0,1/u]]  ->  L U = [[u, v],[l u, l v + 1/u]]
    l, u, v = 0.7, 1.9, -0.35
    F = oq.factor(l, u, v)
    assert np.allclose(F, [[u, v], [l * u, l * v + 1 / u]], rtol=0, atol=1e-15)
    Fi = oq.factor_inverse(l, u, v)
    assert np.allclose(F @ Fi, np.eye(2), atol=1e-14)


def test_kron_matches_numpy(oq):
    rng = np.random.default_rng(5)
    A, B = rng.normal(size=(2, 3)), rng.normal(size=(4, 2))
    assert np.array_equal(oq.kron(A, B), np.kron(A, B))


def test_expand_is_kron_product_in_order(oq):
    # T_b = F1 (x) F2 (x) F3 (x) F4 (x) F5 (researchpod summary, method paragraph),
    # checked against numpy.kron of the closed-form factors.
    p = rand_params(3, 11)
    T = oq.expand(p)
    for b in range(3):
        Fs = [np.array([[u, v], [l * u, l * v + 1.0 / u]], np.float64)
              for (l, u, v) in p[b].astype(np.float64)]
        ref = Fs[0]
        for F in Fs[1:]:
            ref = np.kron(ref, F)
        np.testing.assert_allclose(T[b], ref, rtol=1e-14, atol=1e-14)


def test_p1_unit_determinant(oq):
    # det F = u (l v + 1/u) - v l u = 1 and det(A (x) B) = det(A)^m det(B)^n  ->  det T_b = 1
    p = rand_params(64, 1)
    T = oq.expand(p)
    for b in range(64):
        assert abs(oq.det(T[b]) - 1.0) <= 1e-12
        assert abs(np.linalg.det(T[b]) - 1.0) <= 1e-10


def test_p2_kron_of_inverses_is_inverse(oq):
    # (F1 (x) ... (x) F5)^-1 = F1^-1 (x) ... (x) F5^-1 (the inverse goes to the weights)
    p = rand_params(32, 2)
    T, Ti = oq.expand(p), oq.expand(p, inverse=True)
    for b in range(32):
        err = np.abs(T[b] @ Ti[b] - np.eye(32)).max()
        assert err <= 1e-12 * max(1.0, np.abs(T[b]).max() * np.abs(Ti[b]).max())


def test_rotation_factors_give_an_orthogonal_transform(oq):
    # L U = [[c, s], [-s, c]] for (l, u, v) = (-s/c, c, s); a Kronecker product of
    # orthogonal factors is orthogonal, so T_b T_b^T = I and the inverse is T_b^T
    # (up to the float32 rounding of the parameters)
    import synth
    for p in (synth.make_rotation_params(8), synth.make_rotation_params(16, np.random.default_rng(4))):
        T, Ti = oq.expand(p), oq.expand(p, inverse=True)
        for b in range(p.shape[0]):
            assert np.abs(T[b] @ T[b].T - np.eye(32)).max() < 5e-6
            assert np.abs(Ti[b] - T[b].T).max() < 5e-6
    c = s = np.sqrt(0.5)
    F1 = np.array([[c, s], [-s, c]])
    T = oq.expand(synth.make_rotation_params(1))[0]
    ref = F1
    for _ in range(4):
        ref = np.kron(ref, F1)
    assert np.abs(T - ref).max() < 1e-6


def test_p6_parameter_count_below_half_of_per_channel():
    # abstract: fewer than half the parameters of per-channel scaling.
    per_block = 5 * 3  # five factors, three free parameters (l, u, v) each
    assert per_block / 32 < 0.5
    assert 5 * 4 / 32 > 0.5  # a general 2x2 factor would not satisfy the claim


def test_p5_dense_equals_factored(oq):
    rng = np.random.default_rng(3)
    p = rand_params(4, 3)
    x = rng.normal(size=(8, 128)).astype(np.float32) * 10
    yd = oq.transform_dense(x, oq.expand(p))
    yf = oq.transform_factored(x, p)
    # bound the rounding by the absolute dense sum
    T = oq.expand(p)
    bound = np.zeros_like(yd)
    for b in range(4):
        bound[:, 32 * b:32 * b + 32] = np.abs(x[:, 32 * b:32 * b + 32].astype(np.float64)) @ np.abs(T[b]).T
    assert np.all(np.abs(yd - yf) <= 1e-12 * bound + 1e-300)


def test_p10_single_factor_closed_forms(oq):
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 64)).astype(np.float32)
    for k in range(5):
        p = synth.make_identity_params(2)
        l, u, v = 0.4, 1.7, -0.9
        p[:, k] = (l, u, v)
        l, u, v = (float(t) for t in p[0, k])  # the fp32 values the oracle reads
        F = np.array([[u, v], [l * u, l * v + 1 / u]], np.float64)
        y = oq.transform_dense(x, oq.expand(p))
        st = 16 >> k  # F_{k+1} acts on bit 4 - k
        ref = x.astype(np.float64).copy()
        for i in range(64):
            if (i % 32) & st:
                continue
            a, c = x[:, i].astype(np.float64), x[:, i + st].astype(np.float64)
            ref[:, i] = F[0, 0] * a + F[0, 1] * c
            ref[:, i + st] = F[1, 0] * a + F[1, 1] * c
        np.testing.assert_allclose(y, ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------------ MXFP4 encode

def load_golden():
    path = os.path.join(HERE, "golden", "worked_examples.txt")
    ex, cur = [], None
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, _, rest = line.partition(" ")
        if key == "example":
            cur = {"name": rest}
        elif key == "params":
            cur["params"] = np.array(rest.split(), np.float32).reshape(1, 5, 3)
        elif key == "x":
            cur["x"] = np.array(rest.split(), np.float32).reshape(1, 32)
        elif key == "S":
            cur["S"] = int(rest)
        elif key == "Q":
            cur["Q"] = [int(c, 16) for c in rest.split()]
        elif key == "end":
            ex.append(cur)
    return ex


GOLDEN = load_golden()


@pytest.mark.parametrize("ex", GOLDEN, ids=[e["name"] for e in GOLDEN])
def test_p9_worked_examples(oq, ex):
    q, s, _ = oq.quantize(ex["x"], ex["params"])
    assert int(s[0, 0]) == ex["S"]
    codes = [(q[0, i // 2] >> (4 * (i & 1))) & 0xF for i in range(32)]
    assert codes == ex["Q"]


def test_scale_rule_points(oq):
    # e = floor(log2 amax) - 2, clamped to [-127, 127]; zero -> -127; NaN/Inf -> marker
    assert oq.scale_exp(0.0) == -127
    assert oq.scale_exp(1.0) == -2
    assert oq.scale_exp(np.nextafter(1.0, 0)) == -3
    assert oq.scale_exp(6.0) == 0 and oq.scale_exp(8.0) == 1 and oq.scale_exp(7.999) == 0
    assert oq.scale_exp(2.0 ** -200) == -127
    assert oq.scale_exp(2.0 ** 200) == 127
    assert oq.scale_exp(float("inf")) == 128 and oq.scale_exp(float("nan")) == 128


def test_p4_e2m1_exhaustive_against_argmin(tmp_path):
    """Every finite fp32 value, plus fp64 ulps around every midpoint, against an
    independently written arg-min over the E2M1 grid (tests/native/e2m1_sweep.c)."""
    exe = tmp_path / "e2m1_sweep"
    lib_dir = os.path.join(ROOT, "oracle")
    subprocess.run(["gcc", "-O2", "-o", str(exe), os.path.join(HERE, "native", "e2m1_sweep.c"),
                    "-L", lib_dir, "-l:liboracle_kq.so", f"-Wl,-rpath,{lib_dir}", "-lpthread", "-lm"],
                   check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "sweep_bad=0" in res.stdout and "ulp_bad=0" in res.stdout


def test_p3_identity_factors_reduce_to_plain_mxfp4(oq):
    # T_b = I: the quantizer is plain MXFP4 of x, bit for bit.
    cfg = synth.get_config("pixart")
    x, _, _ = synth.make_inputs(cfg, rows=64)
    q, s, y = oq.quantize(x, synth.make_identity_params(cfg.nb), want_y=True)
    xf = synth.f32_from_bf16_bits(x).astype(np.float64)
    assert np.array_equal(y, xf)
    q2, s2 = oq.encode(xf)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_p7_power_of_two_shifts_scale_only(oq):
    rng = np.random.default_rng(7)
    x = rng.normal(size=(16, 96)).astype(np.float32)
    p = rand_params(3, 7)
    q0, s0, _ = oq.quantize(x, p)
    for k in (-20, -3, 1, 5, 20):
        qk, sk, _ = oq.quantize((x * np.float32(2.0 ** k)).astype(np.float32), p)
        assert np.array_equal(qk, q0)
        assert np.array_equal(sk.astype(int), s0.astype(int) + k)


def test_p8_negation_flips_sign_bits(oq):
    rng = np.random.default_rng(8)
    x = rng.normal(size=(16, 96)).astype(np.float32)
    p = rand_params(3, 8)
    q0, s0, y0 = oq.quantize(x, p, want_y=True)
    q1, s1, _ = oq.quantize(-x, p)
    assert np.array_equal(s0, s1)
    assert np.all(y0 != 0)  # no zeros, so every nibble's sign flips
    assert np.array_equal(q1, q0 ^ 0x88)


def test_p11_row_independence_and_pitch(oq):
    cfg = synth.get_config("tiny")
    x, p, _ = synth.make_inputs(cfg, rows=40)
    q, s, _ = oq.quantize(x, p)
    for rows in (0, 1, 31, 33):
        qr, sr, _ = oq.quantize(np.ascontiguousarray(x[:rows]), p)
        assert np.array_equal(qr, q[:rows]) and np.array_equal(sr, s[:rows])
    wide = np.zeros((40, cfg.d + 64), np.float32)
    wide[:, : cfg.d] = x
    wide[:, cfg.d:] = 1e30  # must never be read
    qw, sw, _ = oq.quantize(wide[:, : cfg.d], p)
    assert np.array_equal(qw, q) and np.array_equal(sw, s)


def test_nonfinite_block_marker(oq):
    x = f32_block([1.0, 2.0])
    x[0, 5] = np.nan
    q, s, _ = oq.quantize(x, synth.make_identity_params(1))
    assert s[0, 0] == 0xFF and not q.any()


def test_sq_oracle_reduces(oq):
    rng = np.random.default_rng(9)
    x = rng.normal(size=(8, 64)).astype(np.float32)
    ones = np.ones(64, np.float32)
    q1, s1, _ = oq.sq_quantize(x, ones)
    q2, s2, _ = oq.quantize(x, synth.make_identity_params(2))
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)
    q3, s3, _ = oq.sq_quantize(x, np.full(64, 0.25, np.float32))
    assert np.array_equal(q3, q1) and np.array_equal(s3.astype(int), s1.astype(int) - 2)
    # per-channel multiply: channel c only sees mult[c]
    m = np.exp(rng.normal(size=64)).astype(np.float32)
    _, _, y = oq.sq_quantize(x, m, want_y=True)
    assert np.array_equal(y, x.astype(np.float64) * m.astype(np.float64))


# ---------------------------------------------------------------- parity rule

def test_classify_counts_planted_mismatches(oq):
    """The parity accounting itself: exact outputs pass; a code moved by one step
    at a value far from any boundary is unexcused; one at a value within tol of a
    boundary is excused; a scale off by one away from a power of two is unexcused."""
    x = f32_block([7.9, 6, 5, 3.5, 2.5, 1.75, 1.25, 0.75, 0.25, -0.25, 3.0, 1.0])
    p = synth.make_identity_params(1)
    q, s, y = oq.quantize(x, p, want_y=True)
    st = oq.classify(x, y, q, s, 0, 1e-5)
    assert st["exact"] == 32 and st["unexcused"] == 0 and st["excused"] == 0
    # channel 2 holds 5.0, exactly on the 4|6 boundary: code 7 is excusable
    q2 = q.copy()
    q2[0, 1] = (q2[0, 1] & 0xF0) | 7
    st = oq.classify(x, y, q2, s, 0, 1e-5)
    assert st["excused"] == 1 and st["unexcused"] == 0
    # channel 10 holds 3.0, far from any boundary: code 6 is not excusable
    q3 = q.copy()
    q3[0, 5] = (q3[0, 5] & 0xF0) | 6
    st = oq.classify(x, y, q3, s, 0, 1e-5)
    assert st["unexcused"] == 1 and st["first_unexcused"] == 10
    # scale off by one with amax 7.9 (not near 8): unexcused block
    s4 = s.copy()
    s4[0, 0] += 1
    st = oq.classify(x, y, q, s4, 0, 1e-5)
    assert st["unexcused_scale_blocks"] == 1 and st["unexcused"] == 32
    # amax within tol of 8: the higher scale is excused, codes judged at that scale
    xe = f32_block([np.nextafter(np.float32(8), np.float32(0)), 1.0])
    qe, se, ye = oq.quantize(xe, p, want_y=True)
    assert se[0, 0] == 127
    xs = f32_block([8.0, 1.0])
    qs_, ss_, _ = oq.quantize(xs, p)
    st = oq.classify(xe, ye, qs_, ss_, 0, 1e-5)
    assert st["excused_scale_blocks"] == 1 and st["unexcused"] == 0 and st["excused"] == 32
    # pre-quant check
    yc = y.astype(np.float32).copy()
    yc[0, 3] += 1e-3
    st = oq.classify(x, y, q, s, 0, 1e-5, y_c=yc)
    assert st["prequant_violations"] == 1
    assert abs(st["max_norm_prequant_err"] - 1e-3 / 7.9) < 1e-6


# ------------------------------------------------------------------ weight side

def test_weight_transform_undoes_the_activation_transform(oq):
    # abstract: the inverse transform goes to the weights, so W' (T x) = W x.
    rng = np.random.default_rng(21)
    p = rand_params(4, 21)
    w = rng.normal(size=(6, 128)).astype(np.float32)
    x = rng.normal(size=(5, 128)).astype(np.float32)
    wp = oq.weight_transform(w, p)
    tx = oq.transform_dense(x, oq.expand(p))
    lhs = tx @ wp.T
    rhs = x.astype(np.float64) @ w.astype(np.float64).T
    scale = np.abs(x.astype(np.float64)) @ np.abs(w.astype(np.float64)).T
    assert np.all(np.abs(lhs - rhs) <= 1e-11 * np.maximum(scale, 1.0))


def test_weight_transform_against_numpy_inverse(oq):
    # an independent inverse (numpy.linalg.inv of the dense T_b) gives the same W'
    rng = np.random.default_rng(22)
    p = rand_params(3, 22)
    w = rng.normal(size=(4, 96)).astype(np.float32)
    T = oq.expand(p)
    ref = np.concatenate([w[:, 32 * b:32 * b + 32].astype(np.float64) @ np.linalg.inv(T[b])
                          for b in range(3)], axis=1)
    np.testing.assert_allclose(oq.weight_transform(w, p), ref, rtol=1e-9, atol=1e-9)


def test_weight_identity_and_encoding(oq):
    rng = np.random.default_rng(23)
    w = rng.normal(size=(8, 64)).astype(np.float32)
    ident = synth.make_identity_params(2)
    assert np.array_equal(oq.weight_transform(w, ident), w.astype(np.float64))
    q, s, y = oq.quantize_weights(w, ident, want_y=True)
    q2, s2 = oq.encode(w.astype(np.float64))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


# ------------------------------------------------------------------ fixed Hadamard comparison

def test_hadamard_columns_match_scipy(oq):
    # unit inputs read the transform's columns; scipy builds the Sylvester matrix independently
    from scipy.linalg import hadamard
    x = np.zeros((32, 64), np.float32)
    for j in range(32):
        x[j, j] = 1.0
        x[j, 32 + j] = -2.0
    _, _, y = oq.hadamard_quantize(x, want_y=True)
    H = hadamard(32) / np.sqrt(32.0)
    np.testing.assert_allclose(y[:, :32], H.T, rtol=0, atol=1e-15)
    np.testing.assert_allclose(y[:, 32:], -2.0 * H.T, rtol=0, atol=1e-15)


def test_hadamard_is_an_orthonormal_involution(oq):
    from scipy.linalg import hadamard
    rng = np.random.default_rng(41)
    x = rng.normal(size=(16, 96)).astype(np.float32)
    _, _, y = oq.hadamard_quantize(x, want_y=True)
    xb, yb = x.astype(np.float64).reshape(16, 3, 32), y.reshape(16, 3, 32)
    np.testing.assert_allclose(np.sum(yb ** 2, -1), np.sum(xb ** 2, -1), rtol=1e-13)  # Parseval
    # applying it again returns the input (H / sqrt(32) is symmetric and orthogonal)
    y32 = y.astype(np.float32)
    _, _, z = oq.hadamard_quantize(y32, want_y=True)
    H = hadamard(32) / np.sqrt(32.0)
    ref = (y32.astype(np.float64).reshape(16, 3, 32) @ H.T).reshape(16, 96)
    np.testing.assert_allclose(z, ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(z, x.astype(np.float64), rtol=0, atol=1e-6 * np.abs(x).max())


def test_hadamard_constant_block_and_encoding(oq):
    # a constant block concentrates on channel 0: sqrt(32) * c, the rest 0
    x = np.full((2, 32), 0.75, np.float32)
    q, s, y = oq.hadamard_quantize(x, want_y=True)
    expect = np.zeros(32)
    expect[0] = np.sqrt(32.0) * 0.75
    np.testing.assert_allclose(y[0], expect, atol=1e-15)
    q2, s2 = oq.encode(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_hadamard_exact_cancellation_is_positive_zero(oq):
    # x = (1, 1, 0, ...): every odd-indexed coefficient is (1 - 1)/sqrt(32) = 0 exactly, a
    # +0 in exact arithmetic, so its code is 0x0 (a negative zero would encode 0x8)
    x = np.zeros((1, 32), np.float32)
    x[0, :2] = 1.0
    q, s, y = oq.hadamard_quantize(x, want_y=True)
    assert np.all(y[0, 1::2] == 0.0) and not np.any(np.signbit(y[0, 1::2]))
    assert np.all((q[0] >> 4) == 0)  # odd channels sit in the high nibbles


# ------------------------------------------------------------------ fused normalization

def test_norm_closed_form_row(oq):
    # x = 0, 1, ..., 31: mean 15.5, biased variance (32^2 - 1) / 12 = 85.25
    x = np.arange(32, dtype=np.float32).reshape(1, 32)
    q, s, h, y = oq.norm_quantize(x, synth.make_identity_params(1), eps=0.0, want_y=True)
    expect = (np.arange(32) - 15.5) / np.sqrt(85.25)
    np.testing.assert_allclose(h[0], expect, rtol=0, atol=1e-14)
    np.testing.assert_allclose(y[0], expect, rtol=0, atol=1e-14)  # identity factors
    q2, s2 = oq.encode(y)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_norm_moments_and_eps(oq):
    rng = np.random.default_rng(51)
    x = (rng.normal(size=(6, 96)) * 3 + 5).astype(np.float32)
    p = synth.make_identity_params(3)
    _, _, h, _ = oq.norm_quantize(x, p, eps=0.0)
    np.testing.assert_allclose(h.mean(1), 0.0, atol=1e-13)
    np.testing.assert_allclose((h ** 2).mean(1), 1.0, rtol=1e-13)
    eps = 0.5
    _, _, he, _ = oq.norm_quantize(x, p, eps=eps)
    var = x.astype(np.float64).var(1)
    np.testing.assert_allclose((he ** 2).mean(1), var / (var + eps), rtol=1e-12)


def test_norm_shift_invariance_and_modulation_per_sample(oq):
    rng = np.random.default_rng(52)
    x = (rng.integers(-64, 64, size=(7, 64)) / 8.0).astype(np.float32)  # exact after + 3
    p = synth.make_params(2, rng)
    _, _, h0, y0 = oq.norm_quantize(x, p, want_y=True)
    _, _, h1, _ = oq.norm_quantize((x + 3).astype(np.float32), p)
    np.testing.assert_allclose(h1, h0, rtol=0, atol=1e-12)
    scale = rng.normal(0, 0.3, size=(3, 64)).astype(np.float32)
    shift = rng.normal(0, 0.5, size=(3, 64)).astype(np.float32)
    _, _, hm, ym = oq.norm_quantize(x, p, shift=shift, scale=scale, rows_per_sample=3, want_y=True)
    g = np.arange(7) // 3  # rows 0-2 sample 0, 3-5 sample 1, 6 sample 2
    np.testing.assert_allclose(hm, h0 * (1 + scale[g].astype(np.float64)) + shift[g], rtol=0, atol=1e-12)
    # the transform of the modulated rows, by numpy from the dense T_b
    T = oq.expand(p)
    ref = np.einsum("bij,rbj->rbi", T, hm.reshape(7, 2, 32)).reshape(7, 64)
    np.testing.assert_allclose(ym, ref, rtol=0, atol=1e-12 * np.abs(ref).max())


# ------------------------------------------------------------------ W4A4 product

def test_dequantize_table_and_round_trip(oq):
    # every code at a few scales against the E2M1 table of the OCP MX spec
    table = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    q = np.zeros((3, 16), np.uint8)
    for i in range(16):
        q[:, i // 2] |= np.uint8(i << (4 * (i % 2)))  # code i at channel i
    q[:, 8:] = q[:, :8]
    s = np.array([[127], [130], [120]], np.uint8)
    v = oq.dequantize(q, s)
    for r, e in enumerate([0, 3, -7]):
        for c in range(32):
            code = c % 16
            mag = table[code & 7] * 2.0 ** e
            assert v[r, c] == (-mag if code & 8 else mag)
    # blocks whose largest code is 6 (value 4) or 7 (value 6) re-encode to themselves
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 16, size=(20, 64)).astype(np.uint8)
    codes[:, ::32] = 7
    qq = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ss = rng.integers(100, 150, size=(20, 2)).astype(np.uint8)
    q2, s2 = oq.encode(oq.dequantize(qq, ss))
    assert np.array_equal(q2, qq) and np.array_equal(s2, ss)


def test_mx_gemm_on_grid_values_is_the_plain_product(oq):
    # values already on the MXFP4 grid survive quantization exactly, so the W4A4 product
    # of their encodings equals numpy's product of the original values
    rng = np.random.default_rng(62)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])

    def on_grid(rows, d):
        v = rng.choice(grid, size=(rows, d)) * rng.choice([-1, 1], size=(rows, d))
        v[:, ::32] = 6.0  # every block's amax is 6: scale 2^0 ... then scaled per block
        e = rng.integers(-4, 5, size=(rows, d // 32))
        return v * np.repeat(2.0 ** e, 32, axis=1)

    a, b = on_grid(9, 128), on_grid(7, 128)
    qa, sa = oq.encode(a)
    qb, sb = oq.encode(b)
    Y, Yabs = oq.mx_gemm(qa, sa, qb, sb)
    assert np.array_equal(Y, a @ b.T)
    assert np.array_equal(Yabs, np.abs(a) @ np.abs(b).T)
    Ysub, _ = oq.mx_gemm(qa, sa, qb, sb, rows=[8, 0], cols=[3])
    assert np.array_equal(Ysub[:, 0], (a @ b.T)[[8, 0], 3])
