"""kq_mx_gemm_static (the product's entry point that allocates nothing: its split
tiles meet through the library's static device array) against kq_mx_gemm_ws (the
same product through a caller's workspace), through the C ABI: two calls in a
row on shapes that split, the second smaller, then one that does not split.
On these shapes both entry points run the same kernels on the same schedule, so
the outputs are equal bit for bit.  Where the static array holds fewer part
slots than the caller's workspace would use, the static entry splits the tiles
into fewer K parts, and both meet the product's fp32 bound against the
reference."""
import numpy as np
import pytest

import oracle
import online_activation_quantizer_amd as kq
from gpu_util import dev, host, say
from test_gpu_gemm import check, random_mx

pytestmark = pytest.mark.gpu


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    return dev(qa), dev(sa), dev(qb), dev(sb)


@pytest.mark.parametrize("out_dtype", ["float32", "bfloat16"])
def test_static_workspace_matches_caller_workspace(out_dtype):
    import torch
    dt = getattr(torch, out_dtype)
    shapes = [(1000, 776, 3072), (257, 257, 2592), (4096, 1152, 1152)]
    for i, (M, N, K) in enumerate(shapes):
        say(f"[mx gemm static] call {i}: {M}x{N}x{K} {out_dtype}")
        n = kq.kq_mx_gemm_workspace_size(M, N, K)
        assert (n > 0) == (i < 2)
        args = operands(M, N, K, 40 + i)
        ws = torch.zeros(max(n, 4096), dtype=torch.uint8, device="cuda")
        want = kq.kq_mx_gemm_ws(*args, ws, out_dtype=dt)
        got = kq.kq_mx_gemm_static(*args, out_dtype=dt)
        torch.cuda.synchronize()
        assert torch.equal(got, want), f"call {i}"
        assert float(got.float().abs().sum()) > 0


def test_static_workspace_with_fewer_parts_than_the_caller_workspace():
    """1024 x 2048 x 10240: 32 tiles of 40 K steps.  With a caller's workspace the
    tiles run in 8 parts (256 part slots, 64 MiB); the static array holds 128
    slots, so the static entry runs them in 4 parts.  Two calls in a row."""
    import torch
    M, N, K = 1024, 2048, 10240
    rng = np.random.default_rng(77)
    qa, sa = random_mx(M, K, rng)
    qb, sb = random_mx(N, K, rng)
    args = (dev(qa), dev(sa), dev(qb), dev(sb))
    n = kq.kq_mx_gemm_workspace_size(M, N, K)
    cu = torch.cuda.get_device_properties(0).multi_processor_count
    if cu == 256:
        assert n == 4096 + 8 * 32 * 256 * 256 * 4
    ws = torch.zeros(max(n, 4096), dtype=torch.uint8, device="cuda")
    Yref, Yabs = oracle.mx_gemm(qa, sa, qb, sb)
    for call in range(2):
        say(f"[mx gemm static, fewer parts] call {call}: {M}x{N}x{K}")
        want = kq.kq_mx_gemm_ws(*args, ws)
        got = kq.kq_mx_gemm_static(*args)
        torch.cuda.synchronize()
        check(host(want), Yref, Yabs, K, f"caller workspace, call {call}", parts=8)
        check(host(got), Yref, Yabs, K, f"static array, call {call}", parts=8)
