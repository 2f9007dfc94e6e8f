"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Rule (fp32 transform): pre-quantization values within 1e-5 * max|x_block| of the
oracle everywhere; E8M0 scales and E2M1 codes bit-exact except where the
oracle's value lies within that tolerance of a decision boundary (counted, and
below 1e-4 of elements); nothing else may differ.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, run_kq, say, verdict

pytestmark = pytest.mark.gpu

CONFIGS = ["tiny", "pixart", "sana", "flux", "flux_mlp"]


@pytest.mark.parametrize("name", CONFIGS)
def test_kq_parity_full_config(name):
    cfg = synth.get_config(name)
    say(f"[kq parity] {name} {cfg.rows}x{cfg.d} {cfg.dtype}")
    x, p, _ = synth.make_inputs(cfg)
    q, s, y = run_kq(x, p)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y)
    say(f"  {st}")
    assert st["pass"], st


@pytest.mark.parametrize("name", ["tiny", "pixart", "flux"])
def test_sq_parity(name):
    cfg = synth.get_config(name)
    say(f"[sq parity] {name}")
    x, _, m = synth.make_inputs(cfg)
    xd, md = dev(x), dev(m)
    q, s = kq.sq_quantize(xd, md)
    q2, s2, yd = kq.sq_transform_debug(xd, md)
    import torch
    torch.cuda.synchronize()
    assert torch.equal(q, q2) and torch.equal(s, s2)
    _, _, y_o = oracle.sq_quantize(x, m, want_y=True)
    st = verdict(x, y_o, host(q), host(s), y_c=host(yd))
    say(f"  {st}")
    assert st["pass"], st


@pytest.mark.parametrize("rows,nb", [(1, 1), (33, 97), (5, 300), (257, 3)])
def test_sq_ragged_and_wide(rows, nb):
    """SmoothQuant on shapes whose grid has lanes past the last row (they join the
    workgroup's multiplier staging and stop) and on more blocks than a workgroup's
    lanes (300: each workgroup stages the slice its lanes cover)."""
    say(f"[sq ragged] rows={rows} nb={nb}")
    rng = np.random.default_rng(rows * 31 + nb)
    x = synth.bf16_bits_from_f32((rng.normal(size=(rows, 32 * nb)) * 3).astype(np.float32))
    m = synth.make_sq_mult(32 * nb, rng)
    q, s = kq.sq_quantize(dev(x), dev(m))
    _, _, y_o = oracle.sq_quantize(x, m, want_y=True)
    st = verdict(x, y_o, host(q), host(s))
    assert st["pass"], st


def test_identity_factors_are_plain_mxfp4_exactly():
    cfg = synth.get_config("pixart")
    say("[identity] pixart")
    x, _, _ = synth.make_inputs(cfg)
    p = synth.make_identity_params(cfg.nb)
    q, s, y = run_kq(x, p)
    q_o, s_o = oracle.encode(synth.f32_from_bf16_bits(x).astype(np.float64))
    assert np.array_equal(y, synth.f32_from_bf16_bits(x))
    assert np.array_equal(s, s_o)
    assert np.array_equal(q, q_o)


def test_encoder_black_box_every_fp32_in_range():
    """Every fp32 magnitude in [2^-3, 8) (both signs) through the product path with
    identity factors at scale 2^0, against the oracle's element encoder: exact."""
    say("[encoder sweep] fp32 [0.125, 8)")
    lo, hi = np.float32(0.125).view(np.uint32), np.float32(8.0).view(np.uint32)
    vals = np.arange(lo, hi, dtype=np.uint32).view(np.float32)
    vals = vals * np.where(np.arange(vals.size) % 2 == 0, 1, -1).astype(np.float32)
    per = 31
    nblk = -(-vals.size // per)
    blocks = np.zeros((nblk, 32), np.float32)
    blocks[:, 0] = 7.99  # anchors every block's amax in [7.99, 8): scale 2^0
    flat = blocks[:, 1:].reshape(-1)
    flat[: vals.size] = vals
    blocks[:, 1:] = flat.reshape(nblk, per)
    d = 2048
    rows = -(-nblk // (d // 32))
    x = np.zeros((rows * (d // 32), 32), np.float32)
    x[:nblk] = blocks
    x[nblk:, 0] = 7.99
    x = x.reshape(rows, d)
    q, s, _ = run_kq(x, synth.make_identity_params(d // 32), debug=False)
    q_o, s_o = oracle.encode(x.astype(np.float64))
    assert np.all(s_o == 127)
    assert np.array_equal(s, s_o)
    bad = np.count_nonzero(q != q_o)
    assert bad == 0, f"{bad} code bytes differ"


def _nibbles(q: np.ndarray) -> np.ndarray:
    return np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[0], -1)


@pytest.mark.parametrize("k", [-149, -140, -127, -126, -110, -100, -30, 0, 30, 100, 115, 125])
def test_extreme_scales(k):
    """Blocks scaled by 2^k (fp32 input): scale bytes from 0 to 252.  Identity factors
    (no rounding in the transform) must match the oracle at every k, subnormal and
    signed-zero inputs included: scales bit for bit, codes bit for bit except the
    sign of a zero code on a +-0 input.  (The oracle's sums start from +0, so a -0.0
    input gives y = +0 there; the shears keep -0 where every partner is negative or
    -0.  A zero y sits on the code boundary at 0, so the parity rule excuses either
    sign, and this test asserts that those are the only excused cases.)  Random
    factors run where fp32 arithmetic keeps its relative precision (|x| above the
    subnormal range, so the 1e-5 * max|x| rule is attainable) and below 2^116 (so
    |T_b x| < 2^128)."""
    say(f"[extreme scale] 2^{k}")
    rng = np.random.default_rng(1000 + k)
    x = (rng.normal(size=(64, 256)) * 2.0 ** k).astype(np.float32)
    zeros = x == 0
    say(f"[extreme scale] 2^{k}: {int(np.count_nonzero(zeros & np.signbit(x)))} inputs -0.0, "
        f"{int(np.count_nonzero(zeros & ~np.signbit(x)))} +0.0")
    p = synth.make_identity_params(8)
    q, s, y = run_kq(x, p)
    q_o, s_o, y_o = oracle.quantize(x, p, want_y=True)
    assert np.array_equal(y[~zeros].view(np.uint32), x[~zeros].view(np.uint32))
    assert np.all(y[zeros] == 0)
    assert np.array_equal(s, s_o)
    n_g, n_o = _nibbles(q), _nibbles(q_o)
    diff = n_g != n_o
    assert np.all((n_g ^ n_o)[diff] == 8), "a code differs in more than the sign bit"
    assert np.all(zeros[diff]), "a sign differs on a nonzero input"
    st = oracle.classify(x, y_o, q, s, 0, 1e-5, y_c=y)
    assert st["unexcused"] == 0 and st["prequant_violations"] == 0, st
    assert st["excused"] == np.count_nonzero(diff), (st, int(np.count_nonzero(diff)))
    if not np.any(zeros & np.signbit(x)):
        assert np.array_equal(q, q_o)
    if -120 <= k <= 115:
        p = synth.make_params(8, rng)
        q, s, y = run_kq(x, p)
        _, _, y_o = oracle.quantize(x, p, want_y=True)
        st = verdict(x, y_o, q, s, y_c=y)
        assert st["pass"], st


def test_zero_nan_inf_blocks():
    say("[special blocks]")
    x = np.ones((4, 128), np.float32)
    x[0, :32] = 0.0
    x[1, 40] = np.nan
    x[2, 70] = np.inf
    x[3, 100] = -np.inf
    p = synth.make_identity_params(4)
    q, s, _ = run_kq(x, p, debug=False)
    q_o, s_o = oracle.encode(x.astype(np.float64))
    assert s[0, 0] == 0 and not q[0, :16].any()
    assert s[1, 1] == 0xFF and s[2, 2] == 0xFF and s[3, 3] == 0xFF
    assert np.array_equal(s, s_o) and np.array_equal(q, q_o)


@pytest.mark.parametrize("rows", [1, 2, 31, 33, 257])
@pytest.mark.parametrize("d", [32, 96, 3104])
def test_ragged_shapes_match_oracle(rows, d):
    """Row counts around tile edges and block counts of 1, 3 and 97 (prime) blocks."""
    say(f"[ragged] rows={rows} d={d}")
    rng = np.random.default_rng(rows * 7919 + d)
    x = synth.bf16_bits_from_f32(rng.standard_t(3, size=(rows, d)).astype(np.float32) * 3)
    p = synth.make_params(d // 32, rng)
    q, s, y = run_kq(x, p)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y)
    assert st["pass"], st


@pytest.mark.parametrize("rows,nb", [(3, 4096), (2, 4099)])
def test_wide_rows_match_oracle(rows, nb):
    """Very wide rows: 4096 blocks, and a prime 4099 blocks (the lane count must be a
    multiple of nb, so the grid holds far more lanes than units)."""
    say(f"[wide] rows={rows} nb={nb}")
    rng = np.random.default_rng(nb)
    x = synth.bf16_bits_from_f32((rng.normal(size=(rows, 32 * nb)) * 3).astype(np.float32))
    p = synth.make_params(nb, rng)
    q, s, y = run_kq(x, p)
    _, _, y_o = oracle.quantize(x, p, want_y=True)
    st = verdict(x, y_o, q, s, y_c=y)
    assert st["pass"], st


def test_eight_way_shards_equal_the_full_call():
    """One GPU's share at 8-way sharding of the FLUX layer: each token shard X[576,
    3072] and each channel shard X[4608, 384] with its 12 factor sets gives exactly the
    matching rows / columns of the full call (every (row, block) unit is independent),
    and one shard of each kind passes the oracle rule on its own."""
    cfg = synth.get_config("flux")
    say("[shards] flux 8 token shards 576x3072, 8 channel shards 4608x384")
    x, p, _ = synth.make_inputs(cfg)
    q_full, s_full, _ = run_kq(x, p, debug=False)
    tr, tc, tb = cfg.rows // 8, cfg.d // 8, cfg.nb // 8
    for k in range(8):
        rows = slice(k * tr, (k + 1) * tr)
        qt, st, _ = run_kq(np.ascontiguousarray(x[rows]), p, debug=False)
        assert np.array_equal(qt, q_full[rows]) and np.array_equal(st, s_full[rows]), k
        xc = np.ascontiguousarray(x[:, k * tc:(k + 1) * tc])
        pc = np.ascontiguousarray(p[k * tb:(k + 1) * tb])
        qc, sc, _ = run_kq(xc, pc, debug=False)
        assert np.array_equal(qc, q_full[:, k * tc // 2:(k + 1) * tc // 2]), k
        assert np.array_equal(sc, s_full[:, k * tb:(k + 1) * tb]), k
    for xs, ps in [(np.ascontiguousarray(x[3 * tr:4 * tr]), p),
                   (np.ascontiguousarray(x[:, 5 * tc:6 * tc]), np.ascontiguousarray(p[5 * tb:6 * tb]))]:
        q, s, y = run_kq(xs, ps)
        _, _, y_o = oracle.quantize(xs, ps, want_y=True)
        st = verdict(xs, y_o, q, s, y_c=y)
        say(f"  {xs.shape}: {st}")
        assert st["pass"], st


def test_row_subsets_and_pitches_with_canaries():
    import torch
    cfg = synth.get_config("sana")
    say("[pitch] sana rows 300, padded x/q/s pitches, canaries")
    x, p, _ = synth.make_inputs(cfg, rows=300)
    q_full, s_full, _ = run_kq(x, p, debug=False)
    d = cfg.d
    xw = np.zeros((300, d + 64), np.uint16)
    xw[:, :d] = x
    xw[:, d:] = synth.bf16_bits_from_f32(np.full((300, 64), 3e38, np.float32))  # never read
    xd = dev(xw)[:, :d]
    pd = dev(p)
    qbuf = torch.full((300, d // 2 + 48), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((300, d // 32 + 9), 0x5A, dtype=torch.uint8, device="cuda")
    kq.kq_quantize(xd, pd, kq.KQ_T_PARAMS, kq.KQ_AUTO, q=qbuf[:, : d // 2], s=sbuf[:, : d // 32])
    qb, sb = host(qbuf), host(sbuf)
    assert np.array_equal(qb[:, : d // 2], q_full) and np.array_equal(sb[:, : d // 32], s_full)
    assert np.all(qb[:, d // 2:] == 0xA5) and np.all(sb[:, d // 32:] == 0x5A)
    for r0, r1 in [(0, 1), (5, 36), (299, 300)]:
        qs, ss, _ = run_kq(np.ascontiguousarray(x[r0:r1]), p, debug=False)
        assert np.array_equal(qs, q_full[r0:r1]) and np.array_equal(ss, s_full[r0:r1])


def test_deterministic_and_side_stream():
    import torch
    cfg = synth.get_config("pixart")
    say("[determinism] pixart, side stream")
    x, p, _ = synth.make_inputs(cfg, rows=1024)
    xd, pd = dev(x), dev(p)
    q1, s1 = kq.kq_quantize(xd, pd)
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        q2, s2 = kq.kq_quantize(xd, pd, stream=st)
    st.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def test_expand_dense_f32_and_bf16x3():
    import torch
    say("[expand] 384 blocks")
    p = synth.make_params(384, np.random.default_rng(55))
    pd = dev(p)
    Tf = host(kq.kq_expand_factors(pd, kq.KQ_T_DENSE_F32)).reshape(384, 32, 32).astype(np.float64)
    T_o = oracle.expand(p)
    # error bound of the fp32 evaluation: each factor entry carries at most 3 roundings
    # (l*v, 1/u, their sum) and the product of five entries 4 more, so
    # |T_gpu - T| <= 16 eps * kron_k(|F_k| with |l v| + |1/u| in the (1,1) slot)
    bound = np.ones((384, 1, 1))
    for k in range(5):
        l, u, v = (p[:, k, i].astype(np.float64) for i in range(3))
        A = np.stack([np.stack([np.abs(u), np.abs(v)], -1),
                      np.stack([np.abs(l * u), np.abs(l * v) + np.abs(1 / u)], -1)], -2)
        bound = np.einsum("bij,bkl->bikjl", bound, A).reshape(384, bound.shape[1] * 2, -1)
    assert np.all(np.abs(Tf - T_o) <= 16 * 2.0 ** -24 * bound)
    T3 = kq.kq_expand_factors(pd, kq.KQ_T_DENSE_BF16X3)
    parts = host(T3).reshape(3, 384, 32, 32).astype(np.uint32) << 16
    hi, mid, lo = (parts[i].view(np.float32).astype(np.float64) for i in range(3))
    # the three bf16 parts sum exactly to the fp32 dense entry
    assert np.array_equal(hi + mid + lo, Tf)
    assert np.all(np.abs(mid) <= np.abs(hi) * 2.0 ** -8) and np.all(np.abs(lo) <= np.abs(mid) * 2.0 ** -8 + 0)
    # the five 2x2 factors F = L U: u and v as given, l u rounded once, l v + 1/u three times
    F = host(kq.kq_expand_factors(pd, kq.KQ_T_FACTORS_2X2_F32)).reshape(384, 5, 2, 2).astype(np.float64)
    for b in (0, 1, 77, 383):
        for k in range(5):
            l, u, v = (float(t) for t in p[b, k])
            F_o = oracle.factor(l, u, v)
            tol = np.array([[0.0, 0.0], [abs(l * u), 2 * (abs(l * v) + abs(1 / u))]]) * 2.0 ** -24
            assert np.all(np.abs(F[b, k] - F_o) <= tol), (b, k, F[b, k], F_o)
    torch.cuda.synchronize()
