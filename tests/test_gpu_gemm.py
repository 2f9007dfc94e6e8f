"""W4A4 product on the gfx950 scaled matrix cores (kq_mx_gemm) against the fp64
reference (decode both MXFP4 operands, multiply), through the C ABI.

Tolerance: every product of two decoded MXFP4 values is exact; the hardware sums
64 of them per instruction and the K/64 instruction results accumulate in fp32,
so |Y_gpu - Y_ref| <= (K/64 + 2) * 2^-23 * sum_k |a_k b_k| bounds the rounding
(twice the sequential-summation bound, for the unknown order inside an
instruction).  bf16 output is the round-to-nearest-even of the fp32 result.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def random_mx(rows, K, rng, lo=118, hi=136):
    codes = rng.integers(0, 16, size=(rows, K), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    s = rng.integers(lo, hi, size=(rows, K // 32), dtype=np.uint8)
    return q, s


def tol(K, Yabs, parts=2):
    """fp32 rounding bound of the product: one rounding per 64-wide MFMA step, one
    per addition of a K part's sums when a tile is split into `parts` parts (the
    unsplit product counted as two parts, one rounding of slack)."""
    return (K / 64 + parts) * 2.0 ** -23 * Yabs


def check(Y, Yref, Yabs, K, label, parts=2):
    err = np.abs(Y.astype(np.float64) - Yref)
    bound = tol(K, Yabs, parts)
    ratio = float(np.max(err / np.maximum(bound, 1e-300)))
    say(f"  {label}: max err/bound = {ratio:.3g}")
    assert np.all(err <= bound), label


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (37, 45, 96), (128, 128, 128), (130, 257, 1152),
                                   (300, 200, 2240), (64, 512, 3072), (300, 1024, 256),
                                   (129, 2048, 608)])
def test_mx_gemm_random_codes(M, N, K):
    import torch
    say(f"[mx gemm] {M}x{N}x{K}")
    rng = np.random.default_rng(M * 7 + N * 13 + K)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    Y = kq.kq_mx_gemm(dev(qa), dev(sa), dev(qb), dev(sb))
    torch.cuda.synchronize()
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    check(host(Y), Yref, Yabs, K, f"{M}x{N}x{K}")


def test_mx_gemm_several_tiles_per_workgroup():
    """More 256 x 256 output tiles than workgroups (the grid is persistent and a
    workgroup's step sequence crosses tile boundaries), ragged M and K; fp32 against
    the reference, bf16 (four-wide stores) against the rounded fp32 result."""
    import torch
    M, N, K = 2321, 8192, 320
    say(f"[mx gemm several tiles per workgroup] {M}x{N}x{K}")
    rng = np.random.default_rng(11)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    y32 = kq.kq_mx_gemm(*args)
    y16 = kq.kq_mx_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    check(host(y32), Yref, Yabs, K, f"{M}x{N}x{K}")


def test_mx_gemm_several_tiles_byte_scales_and_odd_n():
    """The persistent grid's other paths: scale rows read byte by byte (K below 128,
    scale pointer and pitch not word-aligned) and N not a multiple of 4 (one output
    per store), with more tiles than workgroups."""
    import torch
    M, N, K = 2100, 8190, 96
    say(f"[mx gemm byte scales, odd N] {M}x{N}x{K}")
    rng = np.random.default_rng(12)
    qa, sa_full = random_mx(M, K + 32, rng)   # one spare block per row: pitch 4, data at byte 1
    qb, sb_full = random_mx(N, K + 32, rng)
    qa, qb = np.ascontiguousarray(qa[:, :K // 2]), np.ascontiguousarray(qb[:, :K // 2])
    sa_d, sb_d = dev(sa_full)[:, 1:1 + K // 32], dev(sb_full)[:, 1:1 + K // 32]
    args = (dev(qa), sa_d, dev(qb), sb_d)
    y32 = kq.kq_mx_gemm(*args)
    y16 = kq.kq_mx_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    sa, sb = np.ascontiguousarray(sa_full[:, 1:1 + K // 32]), np.ascontiguousarray(sb_full[:, 1:1 + K // 32])
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    check(host(y32), Yref, Yabs, K, f"{M}x{N}x{K}")


def test_mx_gemm_bf16_output_is_rounded_fp32():
    import torch
    say("[mx gemm bf16]")
    rng = np.random.default_rng(5)
    qa, sa = random_mx(200, 1152, rng)
    qb, sb = random_mx(150, 1152, rng)
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    y32 = kq.kq_mx_gemm(*args)
    y16 = kq.kq_mx_gemm(*args, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)


def test_mx_gemm_pitched_operands_and_output():
    import torch
    say("[mx gemm pitched]")
    rng = np.random.default_rng(6)
    qa_full, sa_full = random_mx(50, 256, rng)   # pitches 128 / 8 bytes, K used: 192
    qb_full, sb_full = random_mx(40, 256, rng)
    K = 192
    out = torch.full((50, 48), 7.0, dtype=torch.float32, device="cuda")
    qa, sa = dev(qa_full)[:, :K // 2], dev(sa_full)[:, :K // 32]
    qb, sb = dev(qb_full)[:, :K // 2], dev(sb_full)[:, :K // 32]
    kq.kq_mx_gemm(qa, sa, qb, sb, out=out[:, :40])
    torch.cuda.synchronize()
    o = host(out)
    assert np.all(o[:, 40:] == 7.0)
    Yref, Yabs = oracle.mx_gemm(np.ascontiguousarray(qa_full[:, :K // 2]), np.ascontiguousarray(sa_full[:, :K // 32]),
                                np.ascontiguousarray(qb_full[:, :K // 2]), np.ascontiguousarray(sb_full[:, :K // 32]))
    check(o[:, :40], Yref, Yabs, K, "pitched")


@pytest.mark.parametrize("factors", ["random", "identity"])
def test_w4a4_pipeline_pixart(factors):
    """Activations through kq_quantize, weights through kq_quantize_weights (same
    factors), then the product: parity of the product on the GPU's own codes; with
    identity factors the whole pipeline is plain MXFP4 W4A4, bit for bit."""
    import torch
    cfg, wcfg = synth.get_config("pixart"), synth.get_weight_config("pixart_w")
    say(f"[w4a4 pipeline] pixart 512 tokens x pixart_w, {factors} factors")
    x, p, _ = synth.make_inputs(cfg, rows=512)
    w, _ = synth.make_weights(wcfg)
    if factors == "identity":
        p = synth.make_identity_params(cfg.nb)
    pd = dev(p)
    qx, sx = kq.kq_quantize(dev(x), pd)
    qw, sw = kq.kq_quantize_weights(dev(w), pd)
    Y = kq.kq_mx_gemm(qx, sx, qw, sw)
    torch.cuda.synchronize()
    qx, sx, qw, sw = host(qx), host(sx), host(qw), host(sw)
    Yref, Yabs = oracle.mx_gemm(qx, sx, qw, sw)
    check(host(Y), Yref, Yabs, cfg.d, "pipeline product")
    xf = synth.f32_from_bf16_bits(x).astype(np.float64)
    wf = synth.f32_from_bf16_bits(w).astype(np.float64)
    exact = xf @ wf.T
    rel = np.linalg.norm(Yref - exact) / np.linalg.norm(exact)
    say(f"  W4A4 relative error vs W x ({factors} factors, uncalibrated): {rel:.4f}")
    if factors == "identity":
        qxo, sxo = oracle.encode(xf)
        qwo, swo = oracle.encode(wf)
        assert np.array_equal(qx, qxo) and np.array_equal(sx, sxo)
        assert np.array_equal(qw, qwo) and np.array_equal(sw, swo)


def test_mx_gemm_flux_mlp_full_size():
    """FLUX MLP up-projection at full size (4608 x 12288 x 3072) on the quantizer's own
    outputs: every fp32 output against the reference, and the bf16 output (the
    LDS-staged path bench.py times) equal to the rounded fp32 one."""
    import torch
    cfg, wcfg = synth.get_config("flux"), synth.get_weight_config("flux_w_mlp")
    say("[mx gemm full size] 4608 x 12288 x 3072, every output")
    x, p, _ = synth.make_inputs(cfg)
    w, _ = synth.make_weights(wcfg)
    pd = dev(p)
    qx, sx = kq.kq_quantize(dev(x), pd)
    qw, sw = kq.kq_quantize_weights(dev(w), pd)
    y32 = kq.kq_mx_gemm(qx, sx, qw, sw)
    y16 = kq.kq_mx_gemm(qx, sx, qw, sw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    Yref, Yabs = oracle.mx_gemm(host(qx), host(sx), host(qw), host(sw))
    check(host(y32), Yref, Yabs, cfg.d, "4608 x 12288")
