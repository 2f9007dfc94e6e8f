"""KroQuant online activation quantizer for AMD gfx950 (MI350 / MI355X).

The compute path is the HIP library ``libkq.so`` (C ABI in ``include/kq.h``);
this package only marshals arguments to it.  There is no CPU fallback: when
the library is missing or fails to load, every call raises.
"""
from .kq import (  # noqa: F401
    KQ_AUTO, KQ_BF16, KQ_BUTTERFLY, KQ_FP32, KQ_MFMA, KQ_T_DENSE_BF16X3, KQ_T_DENSE_F32,
    KQ_T_PARAMS, KQ_T_FACTORS_2X2_F32, KQError, STATUS, kq_expand_factors, kq_quantize, kq_transform_debug, lib,
    sq_quantize, sq_transform_debug, expanded_numel, EXPORTED_SYMBOLS, kq_quantize_weights,
    kq_weights_debug, hq_quantize, hq_transform_debug, kq_norm_quantize, kq_norm_debug, kq_mx_gemm,
    kq_mx_gemm_workspace_size, kq_mx_gemm_ws, kq_mx_gemm_static, kq_mx_gemm_fused,
    kq_mx_gemm_fused_ws, kq_mx_gemm_fused_workspace_size,
    KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN, KQ_ERR_DTYPE, KQ_ERR_FORMAT, KQ_ERR_VARIANT,
    KQ_ERR_HIP, KQ_ERR_VALUE, KQ_ERR_DEVICE,
)
