"""W4A4 product with its tiles split in K (kq_mx_gemm_ws) against the fp64
reference, through the C ABI.

When the 256 x 256 output tiles leave at least half of the compute units idle and
a tile has at least 10 K steps (256 values each), each tile is computed as two
halves of K on two workgroups that meet through the caller's workspace.  The fp32
sum of the two half sums has one more rounding than the unsplit product, inside
the same bound as kq_mx_gemm's tests, (K/64 + 2) 2^-23 sum_k |a_k b_k|.  The
workspace's flag words start at zero and every call leaves them zero, so calls in
a row, on shapes of different sizes, share one workspace.
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
MIN_STEPS = 10  # K steps per tile from which the library splits


def cus():
    import torch
    return torch.cuda.get_device_properties(0).multi_processor_count


def tiles(M, N):
    return ((M + 255) // 256) * ((N + 255) // 256)


def split_expected(M, N, K):
    """The rule the library states: one workgroup per compute unit (a multiple of
    8); split when twice the tiles (rounded up to 8) fit in that grid and a tile
    has at least 10 K steps."""
    full = max(8, cus() // 8 * 8)
    n8 = (tiles(M, N) + 7) // 8 * 8
    return 2 * n8 <= full and tiles(M, N) <= FLAG_BYTES // 4 and (K + 255) // 256 >= MIN_STEPS


def workspace_for(M, N, K):
    import torch
    n = kq.kq_mx_gemm_workspace_size(M, N, K)
    split = split_expected(M, N, K)
    assert n == (FLAG_BYTES + tiles(M, N) * TILE_BYTES if split else 0), (M, N, K, n, split)
    return torch.zeros(max(n, FLAG_BYTES), dtype=torch.uint8, device="cuda"), split


def run_case(M, N, K, ws, seed, label):
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
    check(host(y32), Yref, Yabs, K, label)
    assert int(ws[:FLAG_BYTES].count_nonzero()) == 0, f"{label}: flags not left at zero"


@pytest.mark.parametrize("M,N,K", [(1, 1, 2560), (512, 512, 2560), (300, 520, 2336), (257, 257, 2592),
                                   (1000, 776, 3072), (64, 1030, 2400), (256, 2048, 2560)])
def test_split_halves(M, N, K):
    """Fewer tiles than half the compute units: every tile in two halves of K
    (ragged M, N and K included; N = 1030 takes the one-output-per-store path;
    2048 columns deal the tiles to the XCDs)."""
    say(f"[mx gemm split halves] {M}x{N}x{K}")
    ws, split = workspace_for(M, N, K)
    assert split
    run_case(M, N, K, ws, M * 5 + N * 3 + K, f"halves {M}x{N}x{K}")


def test_split_calls_in_a_row_share_the_workspace():
    """Three calls on one workspace, the later ones on smaller shapes: each call
    finds the flags at zero and leaves them so."""
    import torch
    shapes = [(1000, 776, 3072), (512, 512, 2560), (1, 1, 2560)]
    n = max(kq.kq_mx_gemm_workspace_size(*s) for s in shapes)
    ws = torch.zeros(n, dtype=torch.uint8, device="cuda")
    for i, (M, N, K) in enumerate(shapes):
        say(f"[mx gemm split, shared workspace] call {i}: {M}x{N}x{K}")
        run_case(M, N, K, ws, 100 + i, f"shared workspace call {i}")


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
    48 K steps, 96 workgroups), on the quantizer's own outputs: every fp32 output
    against the reference, and bf16 (the LDS-staged path) equal to the rounded
    fp32."""
    import torch
    cfg, wcfg = synth.get_config("flux_mlp"), synth.get_weight_config("flux_w_down")
    say("[mx gemm split full size] 1024 x 3072 x 12288, every output")
    x, p, _ = synth.make_inputs(cfg, rows=1024)
    w, _ = synth.make_weights(wcfg)
    pd = dev(p)
    qx, sx = kq.kq_quantize(dev(x), pd)
    qw, sw = kq.kq_quantize_weights(dev(w), pd)
    M, N, K = 1024, wcfg.rows, cfg.d
    ws, split = workspace_for(M, N, K)
    assert split
    y32 = kq.kq_mx_gemm_ws(qx, sx, qw, sw, ws)
    y16 = kq.kq_mx_gemm_ws(qx, sx, qw, sw, ws, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(y32.to(torch.bfloat16), y16)
    assert int(ws[:FLAG_BYTES].count_nonzero()) == 0
    Yref, Yabs = oracle.mx_gemm(host(qx), host(sx), host(qw), host(sw))
    check(host(y32), Yref, Yabs, K, "split 1024 x 3072 x 12288")
