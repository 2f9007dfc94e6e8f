"""The Python binding's checks of what the C ABI's plain pointers cannot carry:
device, dtype and size of every tensor.  Each case expects one specific status,
raised before any library call (so never KQ_ERR_HIP, which a missing GPU would
also give).  Runs on the CPU: shapes and dtypes are checked before the device."""
import pytest

torch = pytest.importorskip("torch")

import online_activation_quantizer_amd as kq  # noqa: E402


def status_of(fn, *a, **kw):
    with pytest.raises(kq.KQError) as ei:
        fn(*a, **kw)
    assert ei.value.status != kq.KQ_ERR_HIP
    return ei.value.status


def bf16(rows, d):
    return torch.zeros((rows, d), dtype=torch.bfloat16)


def params(nb):
    return torch.zeros((nb, 5, 3), dtype=torch.float32)


def test_host_tensors_are_refused_before_the_library():
    x, p = bf16(4, 64), params(2)
    assert status_of(kq.kq_quantize, x, p) == kq.KQ_ERR_DEVICE
    assert status_of(kq.kq_transform_debug, x, p) == kq.KQ_ERR_DEVICE
    assert status_of(kq.sq_quantize, x, torch.ones(64)) == kq.KQ_ERR_DEVICE
    assert status_of(kq.hq_quantize, x) == kq.KQ_ERR_DEVICE
    assert status_of(kq.kq_quantize_weights, x, p) == kq.KQ_ERR_DEVICE
    assert status_of(kq.kq_norm_quantize, x, p) == kq.KQ_ERR_DEVICE
    assert status_of(kq.kq_expand_factors, p, kq.KQ_T_DENSE_F32) == kq.KQ_ERR_DEVICE
    qa, sa = torch.zeros((4, 32), dtype=torch.uint8), torch.zeros((4, 2), dtype=torch.uint8)
    assert status_of(kq.kq_mx_gemm, qa, sa, qa, sa) == kq.KQ_ERR_DEVICE


def test_factor_parameters_sized_for_another_width():
    x = bf16(4, 64)
    assert status_of(kq.kq_quantize, x, params(3)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, params(1)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize_weights, x, params(3)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_norm_quantize, x, params(1)) == kq.KQ_ERR_SHAPE
    # non-contiguous parameters would be read past their view
    p = torch.zeros((4, 5, 3), dtype=torch.float32)[::2]
    assert status_of(kq.kq_quantize, x, p) == kq.KQ_ERR_SHAPE


def test_transform_dtypes_and_expanded_sizes():
    x = bf16(4, 64)
    assert status_of(kq.kq_quantize, x, params(2).double()) == kq.KQ_ERR_DTYPE
    dense = torch.zeros(2 * 1024, dtype=torch.float32)
    assert status_of(kq.kq_quantize, x, dense[:2000], kq.KQ_T_DENSE_F32) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, dense, kq.KQ_T_DENSE_BF16X3) == kq.KQ_ERR_DTYPE
    b3 = torch.zeros(3 * 2 * 1024 - 8, dtype=torch.int16)
    assert status_of(kq.kq_quantize, x, b3, kq.KQ_T_DENSE_BF16X3, kq.KQ_MFMA) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, dense, 7) == kq.KQ_ERR_FORMAT


def test_outputs_smaller_than_the_input():
    x, p = bf16(8, 64), params(2)
    q, s = torch.zeros((8, 32), dtype=torch.uint8), torch.zeros((8, 2), dtype=torch.uint8)
    assert status_of(kq.kq_quantize, x, p, q=q[:7], s=s) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, p, q=q[:, :31], s=s) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, p, q=q, s=s[:, :1]) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, x, p, q=q.int(), s=s) == kq.KQ_ERR_DTYPE
    y = torch.zeros((8, 64), dtype=torch.float32)
    assert status_of(kq.kq_transform_debug, x, p, y=y[:, :63]) == kq.KQ_ERR_SHAPE
    assert status_of(kq.hq_transform_debug, x, y=y.double()) == kq.KQ_ERR_DTYPE
    assert status_of(kq.hq_quantize, x, q=q, s=s[:5]) == kq.KQ_ERR_SHAPE


def test_multipliers_and_modulation_sizes():
    x, p = bf16(8, 64), params(2)
    assert status_of(kq.sq_quantize, x, torch.ones(32)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.sq_quantize, x, torch.ones(64, dtype=torch.float64)) == kq.KQ_ERR_DTYPE
    sh = torch.zeros((2, 64), dtype=torch.float32)
    assert status_of(kq.kq_norm_quantize, x, p, sh, None) == kq.KQ_ERR_NULL
    # 8 rows at 4 rows per sample need 2 modulation vectors
    assert status_of(kq.kq_norm_quantize, x, p, sh[:1], sh[:1], 4) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_norm_quantize, x, p, sh, sh, 4) == kq.KQ_ERR_DEVICE


def test_input_shapes():
    assert status_of(kq.kq_quantize, torch.zeros((4, 48), dtype=torch.bfloat16), params(1)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, torch.zeros(64, dtype=torch.bfloat16), params(2)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_quantize, bf16(64, 4).t(), params(2)) == kq.KQ_ERR_SHAPE


def test_mx_gemm_operands_and_output():
    qa, sa = torch.zeros((4, 32), dtype=torch.uint8), torch.zeros((4, 2), dtype=torch.uint8)
    qb, sb = torch.zeros((3, 32), dtype=torch.uint8), torch.zeros((3, 2), dtype=torch.uint8)
    assert status_of(kq.kq_mx_gemm, qa, sa, qb, sb, out=torch.zeros((4, 2))) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_mx_gemm, qa, sa, qb, sb, out=torch.zeros((4, 3), dtype=torch.float16)) == kq.KQ_ERR_DTYPE
    assert status_of(kq.kq_mx_gemm, qa.int(), sa, qb, sb) == kq.KQ_ERR_DTYPE
    assert status_of(kq.kq_mx_gemm, qa, sa, qb, sb, out=torch.zeros((4, 3))) == kq.KQ_ERR_DEVICE


def test_expand_output_size():
    p = params(2)
    assert status_of(kq.kq_expand_factors, p, kq.KQ_T_DENSE_F32, out=torch.zeros(2047)) == kq.KQ_ERR_SHAPE
    assert status_of(kq.kq_expand_factors, p, kq.KQ_T_DENSE_BF16X3, out=torch.zeros(6144)) == kq.KQ_ERR_DTYPE
    assert status_of(kq.kq_expand_factors, p, kq.KQ_T_PARAMS) == kq.KQ_ERR_FORMAT
    assert status_of(kq.kq_expand_factors, torch.zeros((2, 15)), kq.KQ_T_DENSE_F32) == kq.KQ_ERR_SHAPE
