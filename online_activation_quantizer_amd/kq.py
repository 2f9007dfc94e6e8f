"""ctypes binding of libkq.so: same names as the C ABI, argument marshalling only.

Tensors are torch tensors on the current HIP device; the binding passes their
``data_ptr()`` and torch's current stream (unless a stream is given) and raises
:class:`KQError` on any non-zero status.  Every step of the computation runs in
the library's kernels.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkq.so")

KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN = 0, -1, -2, -3
KQ_ERR_DTYPE, KQ_ERR_FORMAT, KQ_ERR_VARIANT, KQ_ERR_HIP, KQ_ERR_VALUE = -4, -5, -6, -7, -8
STATUS = {0: "KQ_OK", -1: "KQ_ERR_NULL", -2: "KQ_ERR_SHAPE", -3: "KQ_ERR_ALIGN",
          -4: "KQ_ERR_DTYPE", -5: "KQ_ERR_FORMAT", -6: "KQ_ERR_VARIANT", -7: "KQ_ERR_HIP",
          -8: "KQ_ERR_VALUE"}
KQ_BF16, KQ_FP32 = 0, 1
KQ_T_PARAMS, KQ_T_DENSE_F32, KQ_T_DENSE_BF16X3 = 0, 1, 2
KQ_AUTO, KQ_BUTTERFLY, KQ_MFMA = 0, 1, 2

EXPORTED_SYMBOLS = ("kq_expand_factors", "kq_quantize", "sq_quantize", "kq_transform_debug",
                    "sq_transform_debug", "kq_quantize_weights", "kq_weights_debug",
                    "hq_quantize", "hq_transform_debug", "kq_norm_quantize", "kq_norm_debug",
                    "kq_mx_gemm", "kq_status_string", "kq_last_hip_error")


class KQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        detail = ""
        if status == KQ_ERR_HIP and _lib is not None:
            detail = f" (hipError_t {_lib.kq_last_hip_error()})"
        super().__init__(f"{what}: {STATUS.get(status, status)}{detail}")


_lib = None


def lib():
    """Load libkq.so (built in-tree by ``online_activation_quantizer_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KQError(KQ_ERR_HIP, f"libkq.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.kq_expand_factors.argtypes = [P, I64, I, P, P]
        L.kq_quantize.argtypes = [P, I, I64, I64, I64, P, I, P, I64, P, I64, I, P]
        L.sq_quantize.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P]
        L.kq_transform_debug.argtypes = [P, I, I64, I64, I64, P, I, P, I64, P, I64, I, P, I64, P]
        L.sq_transform_debug.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P, I64, P]
        L.kq_quantize_weights.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P]
        L.kq_weights_debug.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P, I64, P]
        L.hq_quantize.argtypes = [P, I, I64, I64, I64, P, I64, P, I64, P]
        L.hq_transform_debug.argtypes = [P, I, I64, I64, I64, P, I64, P, I64, P, I64, P]
        F = ctypes.c_float
        L.kq_norm_quantize.argtypes = [P, I, I64, I64, I64, P, P, I64, F, P, P, I64, P, I64, P]
        L.kq_norm_debug.argtypes = [P, I, I64, I64, I64, P, P, I64, F, P, P, I64, P, I64, P, I64, P]
        L.kq_mx_gemm.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, P, I64, I, P]
        L.kq_status_string.argtypes = [I]
        L.kq_status_string.restype = ctypes.c_char_p
        L.kq_last_hip_error.argtypes = []
        for name in EXPORTED_SYMBOLS:
            if name not in ("kq_status_string",):
                getattr(L, name).restype = I
        _lib = L
    return _lib


def _check(rc: int, what: str):
    if rc != KQ_OK:
        raise KQError(rc, what)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(x) -> int:
    import torch
    if x.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return KQ_BF16
    if x.dtype == torch.float32:
        return KQ_FP32
    raise KQError(KQ_ERR_DTYPE, f"unsupported input dtype {x.dtype}")


def _row_pitch(a) -> int:
    """Row pitch in elements of a 2-D tensor whose columns are contiguous."""
    if a.dim() != 2 or (a.shape[1] > 1 and a.stride(1) != 1):
        raise KQError(KQ_ERR_SHAPE, "expected a 2-D tensor with unit column stride")
    return a.stride(0)


def expanded_numel(nb: int, tfmt: int) -> int:
    """Elements of an expanded transform (float32 for DENSE_F32, bf16 words for BF16X3)."""
    return {KQ_T_DENSE_F32: nb * 1024, KQ_T_DENSE_BF16X3: 3 * nb * 1024}[tfmt]


def kq_expand_factors(params, tfmt: int, out=None, stream=None):
    """params: float32 [nb, 5, 3] device tensor -> expanded transform tensor."""
    import torch
    nb = params.shape[0]
    if out is None:
        dt = torch.float32 if tfmt == KQ_T_DENSE_F32 else torch.int16
        out = torch.empty(expanded_numel(nb, tfmt) if tfmt in (KQ_T_DENSE_F32, KQ_T_DENSE_BF16X3) else 1,
                          dtype=dt, device=params.device)
    _check(lib().kq_expand_factors(params.data_ptr(), nb, tfmt, out.data_ptr(), _stream(stream)),
           "kq_expand_factors")
    return out


def _outputs(x, q, s):
    import torch
    rows, d = x.shape
    if q is None:
        q = torch.empty((rows, d // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, d // 32), dtype=torch.uint8, device=x.device)
    return q, s


def kq_quantize(x, t, tfmt: int = KQ_T_PARAMS, variant: int = KQ_AUTO, q=None, s=None, stream=None):
    """MXFP4 codes q [rows, d/2] and E8M0 scales s [rows, d/32] of T_b-transformed x."""
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    _check(lib().kq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), t.data_ptr(), tfmt,
                             q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s), variant,
                             _stream(stream)), "kq_quantize")
    return q, s


def sq_quantize(x, mult, q=None, s=None, stream=None):
    """SmoothQuant baseline: MXFP4 of x * mult (mult = 1/s_c, float32 [d])."""
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    _check(lib().sq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), mult.data_ptr(),
                             q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)),
           "sq_quantize")
    return q, s


def kq_transform_debug(x, t, tfmt: int = KQ_T_PARAMS, variant: int = KQ_AUTO, q=None, s=None, y=None,
                       stream=None):
    """kq_quantize that also returns the float32 pre-quantization values y [rows, d]."""
    import torch
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=x.device)
    _check(lib().kq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), t.data_ptr(),
                                    tfmt, q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                    variant, y.data_ptr(), _row_pitch(y), _stream(stream)),
           "kq_transform_debug")
    return q, s, y


def sq_transform_debug(x, mult, q=None, s=None, y=None, stream=None):
    import torch
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=x.device)
    _check(lib().sq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), mult.data_ptr(),
                                    q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                    y.data_ptr(), _row_pitch(y), _stream(stream)),
           "sq_transform_debug")
    return q, s, y


def kq_quantize_weights(w, params, q=None, s=None, stream=None):
    """MXFP4 (q [N, d/2], s [N, d/32]) of W T^-1 for weights w [N, d] (blocks along d)."""
    q, s = _outputs(w, q, s)
    rows, d = w.shape
    _check(lib().kq_quantize_weights(w.data_ptr(), _dtype_code(w), rows, d, _row_pitch(w),
                                     params.data_ptr(), q.data_ptr(), _row_pitch(q), s.data_ptr(),
                                     _row_pitch(s), _stream(stream)), "kq_quantize_weights")
    return q, s


def kq_weights_debug(w, params, q=None, s=None, y=None, stream=None):
    """kq_quantize_weights that also returns the float32 W T^-1 [N, d]."""
    import torch
    q, s = _outputs(w, q, s)
    rows, d = w.shape
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=w.device)
    _check(lib().kq_weights_debug(w.data_ptr(), _dtype_code(w), rows, d, _row_pitch(w), params.data_ptr(),
                                  q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                  y.data_ptr(), _row_pitch(y), _stream(stream)), "kq_weights_debug")
    return q, s, y


def hq_quantize(x, q=None, s=None, stream=None):
    """MXFP4 of the fixed block-Hadamard transform H x_b / sqrt(32) (comparison transform)."""
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    _check(lib().hq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), q.data_ptr(),
                             _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)), "hq_quantize")
    return q, s


def hq_transform_debug(x, q=None, s=None, y=None, stream=None):
    """hq_quantize that also returns the float32 transformed values y [rows, d]."""
    import torch
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=x.device)
    _check(lib().hq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), q.data_ptr(),
                                    _row_pitch(q), s.data_ptr(), _row_pitch(s), y.data_ptr(), _row_pitch(y),
                                    _stream(stream)), "hq_transform_debug")
    return q, s, y


def _ptr_or_null(t):
    return None if t is None else t.data_ptr()


def kq_norm_quantize(x, params, shift=None, scale=None, rows_per_sample=None, eps: float = 1e-6,
                     q=None, s=None, stream=None):
    """LayerNorm + (1 + scale) * . + shift per sample, block transform, MXFP4 (x before normalization)."""
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    rps = rows if rows_per_sample is None else rows_per_sample
    _check(lib().kq_norm_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), _ptr_or_null(shift),
                                  _ptr_or_null(scale), max(1, rps), eps, params.data_ptr(), q.data_ptr(),
                                  _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)),
           "kq_norm_quantize")
    return q, s


def kq_norm_debug(x, params, shift=None, scale=None, rows_per_sample=None, eps: float = 1e-6, q=None,
                  s=None, y=None, stream=None):
    """kq_norm_quantize that also returns the float32 transformed values y [rows, d]."""
    import torch
    q, s = _outputs(x, q, s)
    rows, d = x.shape
    rps = rows if rows_per_sample is None else rows_per_sample
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=x.device)
    _check(lib().kq_norm_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), _ptr_or_null(shift),
                               _ptr_or_null(scale), max(1, rps), eps, params.data_ptr(), q.data_ptr(),
                               _row_pitch(q), s.data_ptr(), _row_pitch(s), y.data_ptr(), _row_pitch(y),
                               _stream(stream)), "kq_norm_debug")
    return q, s, y


def kq_mx_gemm(qa, sa, qb, sb, out=None, out_dtype=None, stream=None):
    """W4A4 product out[m][n] = sum_k deq(A)[m][k] deq(B)[n][k] of two MXFP4 operands
    (codes [rows, K/2], scales [rows, K/32]); out float32 (default) or bfloat16."""
    import torch
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    if qb.shape[1] != qa.shape[1] or tuple(sa.shape) != (M, K // 32) or tuple(sb.shape) != (N, K // 32):
        raise KQError(KQ_ERR_SHAPE, "kq_mx_gemm: codes [rows, K/2] and scales [rows, K/32] of both operands "
                                    "must agree on K")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qa.device)
    code = {torch.float32: KQ_FP32, torch.bfloat16: KQ_BF16}.get(out.dtype)
    if code is None:
        raise KQError(KQ_ERR_DTYPE, f"unsupported output dtype {out.dtype}")
    _check(lib().kq_mx_gemm(qa.data_ptr(), _row_pitch(qa), sa.data_ptr(), _row_pitch(sa), qb.data_ptr(),
                            _row_pitch(qb), sb.data_ptr(), _row_pitch(sb), M, N, K, out.data_ptr(),
                            _row_pitch(out), code, _stream(stream)), "kq_mx_gemm")
    return out
