"""kq_mx_gemm_static (the product's entry point that allocates nothing: its split
tiles meet through the library's static device array) against kq_mx_gemm_ws (the
same product through a caller's workspace), through the C ABI: two calls in a
row on shapes that split, the second smaller, then one that does not split.
Both entry points run the same kernels on the same schedule, so the outputs are
equal bit for bit."""
import numpy as np
import pytest

import online_activation_quantizer_amd as kq
from gpu_util import dev, say
from test_gpu_gemm import random_mx

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
