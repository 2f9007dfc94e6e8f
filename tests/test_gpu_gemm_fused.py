"""W4A4 product with the quantizer in its prologue (kq_mx_gemm_fused), through the
C ABI, against the oracle chain: the quantizer's oracle, then the product's.

The fused kernel quantizes the activations with the quantizer's own transform and
encoder, so its codes are kq_quantize's bit for bit, and it multiplies them with
the same instruction in the same K order as kq_mx_gemm.  So the fused output equals
kq_mx_gemm on kq_quantize's output exactly (fp32 and bf16).  Tied to the oracle:
the GPU's codes pass the quantizer's parity rule against oracle.quantize, and the
product of those codes is within kq_mx_gemm's tolerance of oracle.mx_gemm on them;
on the rows where the GPU's codes equal the oracle's (all but the rows holding an
excused element), the fused output is within that tolerance of oracle.mx_gemm on the
oracle's own codes.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say, verdict
from test_gpu_gemm import check, random_mx

pytestmark = pytest.mark.gpu


def activations(M, K, rng):
    """bf16 bits of N(0, 1) rows with a few 30x outlier channels (the pages' kind of
    activation), and factor parameters for K / 32 blocks."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 30.0
    bits = (x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16
    return bits.astype(np.uint16), synth.make_params(K // 32, rng)


def run(M, N, K, seed, label, oracle_rows=None):
    import torch
    rng = np.random.default_rng(seed)
    x, p = activations(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    xd, pd, qbd, sbd = dev(x), dev(p), dev(qb), dev(sb)
    say(f"[mx gemm fused] {label}: {M}x{N}x{K}")
    y32 = kq.kq_mx_gemm_fused(xd, pd, qbd, sbd)
    y16 = kq.kq_mx_gemm_fused(xd, pd, qbd, sbd, out_dtype=torch.bfloat16)
    qa, sa = kq.kq_quantize(xd, pd)
    u32 = kq.kq_mx_gemm(qa, sa, qbd, sbd)
    u16 = kq.kq_mx_gemm(qa, sa, qbd, sbd, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32, u32), f"{label}: fused fp32 differs from the unfused pair"
    assert torch.equal(y16, u16), f"{label}: fused bf16 differs from the unfused pair"
    # the oracle chain
    rows = np.arange(M) if oracle_rows is None else oracle_rows
    xs = np.ascontiguousarray(x[rows])
    qo, so, yo = oracle.quantize(xs, p, want_y=True)
    qg, sg = host(qa)[rows], host(sa)[rows]
    st = verdict(xs, yo, qg, sg)
    assert st["pass"], f"{label}: quantizer parity {st}"
    Yref, Yabs = oracle.mx_gemm(qg, sg, qb, sb)
    y = host(y32)[rows]
    check(y, Yref, Yabs, K, f"{label} (GPU codes)")
    same = np.all(qo == qg, axis=1) & np.all(so == sg, axis=1)
    say(f"  rows with codes equal to the oracle's: {int(same.sum())} of {len(rows)}")
    assert same.mean() > 0.5
    Yo, Yoabs = oracle.mx_gemm(qo[same], so[same], qb, sb)
    check(y[same], Yo, Yoabs, K, f"{label} (oracle codes)")


@pytest.mark.parametrize("M,N,K", [(1, 1, 32), (37, 45, 96), (128, 256, 256), (300, 520, 2336),
                                   (129, 2048, 608), (257, 1030, 1152)])
def test_fused_small(M, N, K):
    """Ragged M and N (N = 1030 takes the one-output-per-store path), a K tail
    inside the last step (2336 = 9 steps + 4 blocks), one block (K = 32)."""
    run(M, N, K, M * 3 + N * 7 + K, "small")


def test_fused_largest_k():
    """K = 16384, every block's constants on chip (512 blocks)."""
    run(64, 512, 16384, 5, "largest K")


def test_fused_flux_mlp_full_size():
    """FLUX MLP up-projection at full size (4608 x 12288 x 3072): equal to the unfused
    pair on every output; the oracle chain on a 256-row sample."""
    run(4608, 12288, 3072, 9, "flux 4608x12288x3072",
        oracle_rows=np.sort(np.random.default_rng(1).choice(4608, 256, replace=False)))


FLAG_BYTES = 4096
FUSED_TILE_BYTES = 128 * 256 * 4
FUSED_MIN_STEPS_PER_PART = 3


def fused_parts_expected(M, N, K):
    """The rule the library states for the fused product's 128 x 256 tiles: the
    largest of 2, 4 and 8 parts with that many times the tiles (rounded up to 8) on
    the compute units (one workgroup each) and at least 3 K steps per part."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    full = max(8, cus // 8 * 8)
    tiles = ((M + 127) // 128) * ((N + 255) // 256)
    n8 = (tiles + 7) // 8 * 8
    p = min(full // n8, ((K + 255) // 256) // FUSED_MIN_STEPS_PER_PART)
    p = 8 if p >= 8 else 4 if p >= 4 else 2 if p >= 2 else p
    return (p if p >= 2 and tiles <= FLAG_BYTES // 4 else 1), tiles


@pytest.mark.parametrize("M,N,K,want", [(4608, 256, 3072, 4), (1000, 300, 4096, 4), (300, 256, 8192, 8),
                                        (129, 600, 2400, 2), (64, 1030, 1600, 2)])
def test_fused_split(M, N, K, want):
    """Few tiles: each 128 x 256 tile in K parts through a workspace (the FLUX MLP
    up-projection's first 256 weight rows; ragged M, N and K; N = 1030 takes the
    one-output-per-store path).  Against the oracle chain on the GPU's codes within
    the product's bound with one rounding per part, bf16 equal to the rounded fp32,
    the flags left at zero, and the unsplit fused product within the same bound."""
    import torch
    parts, tiles = fused_parts_expected(M, N, K)
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert parts == want
    n = kq.kq_mx_gemm_fused_workspace_size(M, N, K)
    assert n == (FLAG_BYTES + parts * tiles * FUSED_TILE_BYTES if parts > 1 else 0), (n, parts, tiles)
    ws = torch.zeros(max(n, FLAG_BYTES), dtype=torch.uint8, device="cuda")
    rng = np.random.default_rng(M + N * 3 + K * 7)
    x, p = activations(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    xd, pd, qbd, sbd = dev(x), dev(p), dev(qb), dev(sb)
    say(f"[mx gemm fused split] {M}x{N}x{K}, {parts} parts")
    y32 = kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, ws)
    y16 = kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, ws, out_dtype=torch.bfloat16)
    whole = kq.kq_mx_gemm_fused(xd, pd, qbd, sbd)
    qa, sa = kq.kq_quantize(xd, pd)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
    Yref, Yabs = oracle.mx_gemm(host(qa), host(sa), qb, sb)
    check(host(y32), Yref, Yabs, K, f"split {M}x{N}x{K} (GPU codes)", parts=max(2, parts))
    check(host(whole), Yref, Yabs, K, f"unsplit {M}x{N}x{K} (GPU codes)")


def test_fused_split_calls_in_a_row_and_no_workspace():
    """Two split calls in a row on one workspace, the second smaller; no workspace:
    the unsplit fused product, bit for bit."""
    import torch
    shapes = [(1000, 300, 4096), (300, 256, 8192)]
    n = max(kq.kq_mx_gemm_fused_workspace_size(*sh) for sh in shapes)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(shapes):
        rng = np.random.default_rng(50 + i)
        x, p = activations(M, K, rng)
        qb, sb = random_mx(N, K, rng)
        xd, pd, qbd, sbd = dev(x), dev(p), dev(qb), dev(sb)
        y = kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, ws)
        qa, sa = kq.kq_quantize(xd, pd)
        torch.cuda.synchronize()
        assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
        Yref, Yabs = oracle.mx_gemm(host(qa), host(sa), qb, sb)
        check(host(y), Yref, Yabs, K, f"shared workspace call {i}", parts=8)
        if i == 0:
            a = kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, None)
            b = kq.kq_mx_gemm_fused(xd, pd, qbd, sbd)
            torch.cuda.synchronize()
            assert torch.equal(a, b)


def test_fused_rejects():
    import torch
    x = torch.zeros((8, 64), dtype=torch.bfloat16, device="cuda")
    p = torch.zeros(2 * 15, dtype=torch.float32, device="cuda")
    qb = torch.zeros((8, 32), dtype=torch.uint8, device="cuda")
    sb = torch.zeros((8, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.kq_mx_gemm_fused(x.float(), p, qb, sb)
    assert e.value.status == kq.KQ_ERR_DTYPE
    big = torch.zeros((1, 16416), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.kq_mx_gemm_fused(big, torch.zeros(513 * 15, device="cuda"),
                            torch.zeros((1, 8208), dtype=torch.uint8, device="cuda"),
                            torch.zeros((1, 513), dtype=torch.uint8, device="cuda"))
    assert e.value.status == kq.KQ_ERR_SHAPE


@pytest.mark.parametrize("case", range(8))
def test_fused_split_random_shapes_and_pitches(case):
    """Seeded random shapes with few tiles (M in [1, 1200), N in [1, 700), K a
    multiple of 32 in [768, 10240)), activation, weight and output pitches padded:
    fp32 within the bound for the rule's part count against the oracle on the GPU's
    codes (kq_quantize of the same pitched rows), bf16 the rounded fp32, nothing
    written past N in a row, the flags left at zero."""
    import torch
    from test_gpu_gemm_split import pitched, sentinel_outputs, padding_untouched
    rng = np.random.default_rng(4242 + case)
    M, N, K = int(rng.integers(1, 1200)), int(rng.integers(1, 700)), 32 * int(rng.integers(24, 320))
    px, pb, psb, po = 8 * int(rng.integers(0, 3)), 16 * int(rng.integers(0, 3)), int(rng.integers(0, 6)), \
        int(rng.integers(0, 9))
    parts, _ = fused_parts_expected(M, N, K)
    say(f"[mx gemm fused split sweep {case}] {M}x{N}x{K}, {parts} parts, pads {px} {pb} {psb} {po}")
    x, p = activations(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    xw = torch.zeros((M, K + px), dtype=torch.int16, device="cuda")
    xw[:, :K] = dev(x)
    xd, pd = xw[:, :K], dev(p)
    qbd, sbd = pitched(qb, pb, 0xA5), pitched(sb, psb, 0x88)
    n = kq.kq_mx_gemm_fused_workspace_size(M, N, K)
    ws = torch.zeros(max(n, FLAG_BYTES), dtype=torch.uint8, device="cuda") if n > 0 else None
    o32, o16 = sentinel_outputs(M, N, po)
    kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, ws, out=o32[:, :N])
    kq.kq_mx_gemm_fused_ws(xd, pd, qbd, sbd, ws, out=o16[:, :N])
    qa, sa = kq.kq_quantize(xd, pd)
    torch.cuda.synchronize()
    assert torch.equal(o32[:, :N].to(torch.bfloat16), o16[:, :N])
    assert padding_untouched(o32, o16, N), "a store past N"
    if ws is not None:
        assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
    Yref, Yabs = oracle.mx_gemm(host(qa), host(sa), qb, sb)
    check(host(o32[:, :N].contiguous()), Yref, Yabs, K, f"fused sweep {case}", parts=max(2, parts))
