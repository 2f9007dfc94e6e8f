"""W4A4 product with its tiles split in K (kq_mx_gemm_ws) against the fp64
reference, through the C ABI.

When the 256 x 256 output tiles leave at least half of the compute units idle and
a tile has at least 10 K steps (256 values each), each tile is computed as S parts
of K on S workgroups that meet through the caller's workspace: S is the largest
power of two (2, 4 or 8) of parts that fit the compute units, each of at least 5
K steps.  Every part's
fp32 sums are added in part order, one rounding per addition more than the
unsplit product: the bound is (K/64 + S) 2^-23 sum_k |a_k b_k| (the unsplit
product's tests use S = 2).  The workspace's flag words start at zero and every
call leaves them zero, so calls in a row, on shapes of different sizes, share one
workspace.
"""
import numpy as np
import pytest

import oracle
import synth
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say
from test_gpu_gemm import check, random_mx

pytestmark = pytest.mark.gpu

FLAG_BYTES = 4096
TILE_BYTES = 256 * 256 * 4
MIN_STEPS_PER_PART = 5  # K steps per part from which the library splits
MAX_PARTS = 8


def cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def tiles(M, N):
    return ((M + 255) // 256) * ((N + 255) // 256)


def parts_expected(M, N, K, max_slots=None):
    """The rule the library states: one workgroup per compute unit (a multiple of
    8); the largest power of two of parts per tile that fits that grid (tiles
    rounded up to 8), with parts of at least 5 K steps, at most 8, and no more
    than the workspace's part slots; split when that is at least two.  Returns 1
    for whole tiles."""
    full = max(8, cus() // 8 * 8)
    n8 = (tiles(M, N) + 7) // 8 * 8
    p = min(full // n8, ((K + 255) // 256) // MIN_STEPS_PER_PART, MAX_PARTS)
    if max_slots is not None:
        p = min(p, max_slots // tiles(M, N))
    p = 8 if p >= 8 else 4 if p >= 4 else 2 if p >= 2 else p
    return p if p >= 2 and tiles(M, N) <= FLAG_BYTES // 4 else 1


def workspace_for(M, N, K):
    import torch
    n = kq.kq_mx_gemm_workspace_size(M, N, K)
    parts = parts_expected(M, N, K)
    assert n == (FLAG_BYTES + parts * tiles(M, N) * TILE_BYTES if parts > 1 else 0), (M, N, K, n, parts)
    return torch.zeros(max(n, FLAG_BYTES), dtype=torch.uint8, device="cuda"), parts


def run_case(M, N, K, ws, parts, seed, label):
    import torch
    rng = np.random.default_rng(seed)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    y32 = kq.kq_mx_gemm_ws(*args, ws)
    y16 = kq.kq_mx_gemm_ws(*args, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16), label
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    check(host(y32), Yref, Yabs, K, label, parts=max(2, parts))
    assert int(ws[:FLAG_BYTES].count_nonzero()) == 0, f"{label}: flags not left at zero"


@pytest.mark.parametrize("M,N,K", [(1, 1, 2560), (512, 512, 2560), (300, 520, 2336), (257, 257, 2592),
                                   (1000, 776, 3072), (64, 1030, 2400), (256, 2048, 2560)])
def test_split_halves(M, N, K):
    """Fewer tiles than half the compute units and 10-14 K steps: every tile in two
    parts of K (ragged M, N and K included; N = 1030 takes the one-output-per-store
    path; 2048 columns deal the tiles to the XCDs)."""
    say(f"[mx gemm split halves] {M}x{N}x{K}")
    ws, parts = workspace_for(M, N, K)
    assert parts == 2
    run_case(M, N, K, ws, parts, M * 5 + N * 3 + K, f"halves {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,want", [(300, 700, 5120, 4), (1024, 1024, 5120, 4), (700, 1500, 6400, 4),
                                        (512, 512, 12288, 8), (257, 300, 10240, 8), (33, 2000, 8160, 4),
                                        (1, 300, 7424, 4), (300, 700, 4000, 2)])
def test_split_many_parts(M, N, K, want):
    """Longer K: four and eight parts per tile (ragged M, N and K; K steps that do
    not divide evenly among the parts; one row); three parts' worth of K runs in
    two."""
    say(f"[mx gemm split {want} parts] {M}x{N}x{K}")
    ws, parts = workspace_for(M, N, K)
    if cus() == 256:
        assert parts == want
    run_case(M, N, K, ws, parts, M * 11 + N * 7 + K, f"{parts} parts {M}x{N}x{K}")


def test_split_calls_in_a_row_share_the_workspace():
    """Three calls on one workspace, the later ones on smaller shapes: each call
    finds the flags at zero and leaves them so."""
    import torch
    shapes = [(1000, 776, 3072), (512, 512, 2560), (1, 1, 2560)]
    n = max(kq.kq_mx_gemm_workspace_size(*s) for s in shapes)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(shapes):
        say(f"[mx gemm split, shared workspace] call {i}: {M}x{N}x{K}")
        run_case(M, N, K, ws, parts_expected(M, N, K), 100 + i, f"shared workspace call {i}")


def test_split_unsplit_when_no_workspace_or_nothing_to_split():
    """No workspace: the unsplit product, bit for bit; tiles of 9 K steps, or more
    tiles than half the compute units, need no workspace."""
    import torch
    M, N, K = 512, 512, 512
    rng = np.random.default_rng(3)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    a = kq.kq_mx_gemm(*args)
    b = kq.kq_mx_gemm_ws(*args, None)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert kq.kq_mx_gemm_workspace_size(M, N, 2304) == 0       # 9 K steps: no split
    full = max(8, cus() // 8 * 8)
    assert kq.kq_mx_gemm_workspace_size(256, (full // 2 + 8) * 256, 3072) == 0  # over half the grid


def test_split_workspace_too_small_is_rejected():
    import torch
    M, N, K = 512, 512, 2560
    rng = np.random.default_rng(4)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    need = kq.kq_mx_gemm_workspace_size(M, N, K)
    ws = torch.zeros(need - 256, dtype=torch.uint8, device="cuda")
    with pytest.raises(kq.KQError) as e:
        kq.kq_mx_gemm_ws(dev(qa), dev(sa), dev(qb), dev(sb), ws)
    assert e.value.status == kq.KQ_ERR_VALUE


def test_split_flux_down_projection_1024_tokens():
    """FLUX MLP down-projection for 1024 tokens (1024 x 3072 x 12288: 48 tiles of
    48 K steps, in four parts on 192 workgroups), on the quantizer's own outputs:
    every fp32 output against the reference, and bf16 (the LDS-staged path) equal
    to the rounded fp32."""
    import torch
    cfg, wcfg = synth.get_config("flux_mlp"), synth.get_weight_config("flux_w_down")
    say("[mx gemm split full size] 1024 x 3072 x 12288, every output")
    x, p, _ = synth.make_inputs(cfg, rows=1024)
    w, _ = synth.make_weights(wcfg)
    pd = dev(p)
    qx, sx = kq.kq_quantize(dev(x), pd)
    qw, sw = kq.kq_quantize_weights(dev(w), pd)
    M, N, K = 1024, wcfg.rows, cfg.d
    ws, parts = workspace_for(M, N, K)
    assert parts >= 2
    y32 = kq.kq_mx_gemm_ws(qx, sx, qw, sw, ws)
    y16 = kq.kq_mx_gemm_ws(qx, sx, qw, sw, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
    Yref, Yabs = oracle.mx_gemm(host(qx), host(sx), host(qw), host(sw))
    check(host(y32), Yref, Yabs, K, f"split 1024 x 3072 x 12288 ({parts} parts)", parts=parts)


def sweep_cases(n, seed=20261203):
    """Seeded random shapes and pitches: M, N in [1, 1200), K a multiple of 32 in
    [1536, 11520) (6-45 K steps, so 1, 2, 4 or 8 parts), code-row pitches padded by
    0-32 bytes, scale pitches by 0-5 bytes (word-aligned or not), output pitches by
    0-8 elements."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        M, N = int(rng.integers(1, 1200)), int(rng.integers(1, 1200))
        K = 32 * int(rng.integers(48, 360))
        pads = (16 * int(rng.integers(0, 3)), int(rng.integers(0, 6)), 16 * int(rng.integers(0, 3)),
                int(rng.integers(0, 6)), int(rng.integers(0, 9)))
        out.append((M, N, K) + pads)
    return out


def pitched(a, extra, fill):
    """The uint8 matrix a in the leading columns of a device buffer `extra` bytes
    wider per row (the row pitch), the padding filled with `fill`: the view."""
    import torch
    rows, cols = a.shape
    whole = torch.full((rows, cols + extra), fill, dtype=torch.uint8, device="cuda")
    whole[:, :cols] = dev(a)
    return whole[:, :cols]


SENTINEL_F32, SENTINEL_BF16 = 0x7FC0DEAD, 0x7FAD  # NaN payloads no product writes


def sentinel_outputs(M, N, extra):
    """fp32 and bf16 output buffers of row pitch N + extra filled with NaN
    sentinels, and their M x N views."""
    import torch
    o32 = torch.full((M, N + extra), SENTINEL_F32, dtype=torch.int32, device="cuda").view(torch.float32)
    o16 = torch.full((M, N + extra), SENTINEL_BF16, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    return o32, o16


def padding_untouched(o32, o16, N):
    import torch
    return (bool(torch.all(o32.view(torch.int32)[:, N:] == SENTINEL_F32))
            and bool(torch.all(o16.view(torch.int16)[:, N:] == SENTINEL_BF16)))


@pytest.mark.parametrize("case", range(10))
def test_split_random_shapes_and_pitches(case):
    """Seeded random shapes, padded operand and output pitches: fp32 within the bound
    for the part count the rule gives, bf16 the rounded fp32, nothing written past N
    in a row, the flags left at zero."""
    import torch
    M, N, K, pa, psa, pb, psb, po = sweep_cases(10)[case]
    parts = parts_expected(M, N, K)
    say(f"[mx gemm split sweep {case}] {M}x{N}x{K}, {parts} parts, pads {pa} {psa} {pb} {psb} {po}")
    rng = np.random.default_rng(1000 + case)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    args = (pitched(qa, pa, 0x5A), pitched(sa, psa, 0x77), pitched(qb, pb, 0xA5), pitched(sb, psb, 0x88))
    n = kq.kq_mx_gemm_workspace_size(M, N, K)
    ws = torch.zeros(max(n, FLAG_BYTES), dtype=torch.uint8, device="cuda") if n > 0 else None
    o32, o16 = sentinel_outputs(M, N, po)
    kq.kq_mx_gemm_ws(*args, ws, out=o32[:, :N])
    kq.kq_mx_gemm_ws(*args, ws, out=o16[:, :N])
    torch.cuda.synchronize()
    assert torch.equal(o32[:, :N].to(torch.bfloat16), o16[:, :N])
    assert padding_untouched(o32, o16, N), "a store past N"
    if ws is not None:
        assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    check(host(o32[:, :N].contiguous()), Yref, Yabs, K, f"sweep {case}", parts=max(2, parts))
