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
