"""ctypes binding of libkq.so: same names as the C ABI, argument marshalling only.

Tensors are torch tensors on one HIP device; the binding passes their
``data_ptr()`` and torch's current stream (unless a stream is given) and raises
:class:`KQError` on any non-zero status.  Every step of the computation runs in
the library's kernels.

The C library sees plain pointers and sizes only, so before any call the binding
checks what the pointers cannot carry: every tensor is on the input's device
(KQ_ERR_DEVICE, a status of this binding only), of the dtype the entry point
reads (KQ_ERR_DTYPE), and large enough for what the kernels read or write
(KQ_ERR_SHAPE).  Shapes and dtypes are checked first, the device last.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkq.so")

KQ_OK, KQ_ERR_NULL, KQ_ERR_SHAPE, KQ_ERR_ALIGN = 0, -1, -2, -3
KQ_ERR_DTYPE, KQ_ERR_FORMAT, KQ_ERR_VARIANT, KQ_ERR_HIP, KQ_ERR_VALUE = -4, -5, -6, -7, -8
# raised by this binding only (the C ABI cannot tell host from device pointers)
KQ_ERR_DEVICE = -9
STATUS = {0: "KQ_OK", -1: "KQ_ERR_NULL", -2: "KQ_ERR_SHAPE", -3: "KQ_ERR_ALIGN",
          -4: "KQ_ERR_DTYPE", -5: "KQ_ERR_FORMAT", -6: "KQ_ERR_VARIANT", -7: "KQ_ERR_HIP",
          -8: "KQ_ERR_VALUE", -9: "KQ_ERR_DEVICE"}
KQ_BF16, KQ_FP32 = 0, 1
KQ_T_PARAMS, KQ_T_DENSE_F32, KQ_T_DENSE_BF16X3, KQ_T_FACTORS_2X2_F32 = 0, 1, 2, 3
KQ_AUTO, KQ_BUTTERFLY, KQ_MFMA = 0, 1, 2

EXPORTED_SYMBOLS = ("kq_expand_factors", "kq_quantize", "sq_quantize", "kq_transform_debug",
                    "sq_transform_debug", "kq_quantize_weights", "kq_weights_debug",
                    "hq_quantize", "hq_transform_debug", "kq_norm_quantize", "kq_norm_debug",
                    "kq_mx_gemm", "kq_mx_gemm_fused", "kq_mx_gemm_workspace_size", "kq_mx_gemm_ws",
                    "kq_mx_gemm_static", "kq_mx_gemm_fused_workspace_size", "kq_mx_gemm_fused_ws",
                    "kq_status_string", "kq_last_hip_error")


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
        L.kq_mx_gemm_workspace_size.argtypes = [I64, I64, I64, ctypes.POINTER(I64)]
        L.kq_mx_gemm_ws.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, P, I64, I, P, I64, P]
        L.kq_mx_gemm_static.argtypes = [P, I64, P, I64, P, I64, P, I64, I64, I64, I64, P, I64, I, P]
        L.kq_mx_gemm_fused.argtypes = [P, I, I64, P, P, I64, P, I64, I64, I64, I64, P, I64, I, P]
        L.kq_mx_gemm_fused_workspace_size.argtypes = [I64, I64, I64, ctypes.POINTER(I64)]
        L.kq_mx_gemm_fused_ws.argtypes = [P, I, I64, P, P, I64, P, I64, I64, I64, I64, P, I64, I, P, I64, P]
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


def _fail(status: int, msg: str):
    raise KQError(status, msg)


def _is16(t) -> bool:
    import torch
    return t.dtype in (torch.bfloat16, torch.int16, torch.uint16, torch.float16)


def _need_2d(what: str, name: str, t, rows: int, cols: int, dtype):
    """t: 2-D, unit column stride, dtype `dtype`, at least rows x cols."""
    if t.dtype != dtype:
        _fail(KQ_ERR_DTYPE, f"{what}: {name} must be {dtype}, got {t.dtype}")
    _row_pitch(t)
    if t.shape[0] < rows or t.shape[1] < cols:
        _fail(KQ_ERR_SHAPE, f"{what}: {name} is {tuple(t.shape)}, needs at least ({rows}, {cols})")


def _need_flat(what: str, name: str, t, numel: int, dtype_ok, dtype_name: str):
    """t: contiguous, exactly `numel` elements of an accepted dtype."""
    if not dtype_ok(t):
        _fail(KQ_ERR_DTYPE, f"{what}: {name} must be {dtype_name}, got {t.dtype}")
    if not t.is_contiguous():
        _fail(KQ_ERR_SHAPE, f"{what}: {name} must be contiguous")
    if t.numel() != numel:
        _fail(KQ_ERR_SHAPE, f"{what}: {name} has {t.numel()} elements, needs {numel}")


def _f32(t) -> bool:
    import torch
    return t.dtype == torch.float32


def _need_device(what: str, ref, **tensors):
    """Every given tensor on the HIP device of `ref` (which must be a HIP tensor)."""
    if not ref.is_cuda:
        _fail(KQ_ERR_DEVICE, f"{what}: tensors must be on a HIP device, got {ref.device}")
    for name, t in tensors.items():
        if t is not None and t.device != ref.device:
            _fail(KQ_ERR_DEVICE, f"{what}: {name} is on {t.device}, the input on {ref.device}")


def _need_input(what: str, x):
    if x.dim() != 2:
        _fail(KQ_ERR_SHAPE, f"{what}: input must be 2-D, got {tuple(x.shape)}")
    _dtype_code(x)
    _row_pitch(x)


def _need_transform(what: str, t, nb: int, tfmt: int):
    if tfmt == KQ_T_PARAMS:
        _need_flat(what, "params", t, nb * 15, _f32, "float32 [d/32, 5, 3]")
    elif tfmt == KQ_T_DENSE_F32:
        _need_flat(what, "transform", t, nb * 1024, _f32, "float32 [d/32, 32, 32]")
    elif tfmt == KQ_T_DENSE_BF16X3:
        _need_flat(what, "transform", t, 3 * nb * 1024, _is16, "16-bit [3, d/32, 32, 32]")
    else:
        _fail(KQ_ERR_FORMAT, f"{what}: unknown transform format {tfmt}")


def _need_outputs(what: str, x, q, s, y=None):
    import torch
    rows, d = x.shape
    _need_2d(what, "q", q, rows, d // 2, torch.uint8)
    _need_2d(what, "s", s, rows, d // 32, torch.uint8)
    if y is not None:
        _need_2d(what, "y", y, rows, d, torch.float32)


def expanded_numel(nb: int, tfmt: int) -> int:
    """Elements of an expanded transform (float32 for DENSE_F32 and FACTORS_2X2_F32, bf16
    words for BF16X3)."""
    return {KQ_T_DENSE_F32: nb * 1024, KQ_T_DENSE_BF16X3: 3 * nb * 1024, KQ_T_FACTORS_2X2_F32: nb * 20}[tfmt]


def kq_expand_factors(params, tfmt: int, out=None, stream=None):
    """params: float32 [nb, 5, 3] device tensor -> expanded transform tensor."""
    import torch
    what = "kq_expand_factors"
    if params.dim() != 3 or tuple(params.shape[1:]) != (5, 3):
        _fail(KQ_ERR_SHAPE, f"{what}: params must be [nb, 5, 3], got {tuple(params.shape)}")
    nb = params.shape[0]
    _need_flat(what, "params", params, nb * 15, _f32, "float32")
    if tfmt not in (KQ_T_DENSE_F32, KQ_T_DENSE_BF16X3, KQ_T_FACTORS_2X2_F32):
        _fail(KQ_ERR_FORMAT, f"{what}: format {tfmt} is not an expanded format")
    f32 = tfmt != KQ_T_DENSE_BF16X3
    if out is None:
        out = torch.empty(expanded_numel(nb, tfmt), dtype=torch.float32 if f32 else torch.int16,
                          device=params.device if params.is_cuda else "cpu")
    _need_flat(what, "out", out, expanded_numel(nb, tfmt), _f32 if f32 else _is16,
               "float32" if f32 else "16-bit")
    _need_device(what, params, out=out)
    _check(lib().kq_expand_factors(params.data_ptr(), nb, tfmt, out.data_ptr(), _stream(stream)),
           "kq_expand_factors")
    return out


def _outputs(x, q, s, what="kq"):
    """Checks the input's shape and dtype and allocates the outputs not given."""
    import torch
    _need_input(what, x)
    rows, d = x.shape
    if d % 32:
        _fail(KQ_ERR_SHAPE, f"{what}: d = {d} is not a multiple of 32")
    if q is None:
        q = torch.empty((rows, d // 2), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((rows, d // 32), dtype=torch.uint8, device=x.device)
    _need_outputs(what, x, q, s)
    return q, s


def _y_out(x, y, what):
    import torch
    rows, d = x.shape
    if y is None:
        y = torch.empty((rows, d), dtype=torch.float32, device=x.device)
    _need_2d(what, "y", y, rows, d, torch.float32)
    return y


def kq_quantize(x, t, tfmt: int = KQ_T_PARAMS, variant: int = KQ_AUTO, q=None, s=None, stream=None):
    """MXFP4 codes q [rows, d/2] and E8M0 scales s [rows, d/32] of T_b-transformed x."""
    q, s = _outputs(x, q, s, "kq_quantize")
    rows, d = x.shape
    _need_transform("kq_quantize", t, d // 32, tfmt)
    _need_device("kq_quantize", x, t=t, q=q, s=s)
    _check(lib().kq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), t.data_ptr(), tfmt,
                             q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s), variant,
                             _stream(stream)), "kq_quantize")
    return q, s


def sq_quantize(x, mult, q=None, s=None, stream=None):
    """SmoothQuant baseline: MXFP4 of x * mult (mult = 1/s_c, float32 [d])."""
    q, s = _outputs(x, q, s, "sq_quantize")
    rows, d = x.shape
    _need_flat("sq_quantize", "mult", mult, d, _f32, "float32 [d]")
    _need_device("sq_quantize", x, mult=mult, q=q, s=s)
    _check(lib().sq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), mult.data_ptr(),
                             q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)),
           "sq_quantize")
    return q, s


def kq_transform_debug(x, t, tfmt: int = KQ_T_PARAMS, variant: int = KQ_AUTO, q=None, s=None, y=None,
                       stream=None):
    """kq_quantize that also returns the float32 pre-quantization values y [rows, d]."""
    what = "kq_transform_debug"
    q, s = _outputs(x, q, s, what)
    rows, d = x.shape
    _need_transform(what, t, d // 32, tfmt)
    y = _y_out(x, y, what)
    _need_device(what, x, t=t, q=q, s=s, y=y)
    _check(lib().kq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), t.data_ptr(),
                                    tfmt, q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                    variant, y.data_ptr(), _row_pitch(y), _stream(stream)),
           "kq_transform_debug")
    return q, s, y


def sq_transform_debug(x, mult, q=None, s=None, y=None, stream=None):
    what = "sq_transform_debug"
    q, s = _outputs(x, q, s, what)
    rows, d = x.shape
    _need_flat(what, "mult", mult, d, _f32, "float32 [d]")
    y = _y_out(x, y, what)
    _need_device(what, x, mult=mult, q=q, s=s, y=y)
    _check(lib().sq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), mult.data_ptr(),
                                    q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                    y.data_ptr(), _row_pitch(y), _stream(stream)),
           "sq_transform_debug")
    return q, s, y


def kq_quantize_weights(w, params, q=None, s=None, stream=None):
    """MXFP4 (q [N, d/2], s [N, d/32]) of W T^-1 for weights w [N, d] (blocks along d)."""
    what = "kq_quantize_weights"
    q, s = _outputs(w, q, s, what)
    rows, d = w.shape
    _need_transform(what, params, d // 32, KQ_T_PARAMS)
    _need_device(what, w, params=params, q=q, s=s)
    _check(lib().kq_quantize_weights(w.data_ptr(), _dtype_code(w), rows, d, _row_pitch(w),
                                     params.data_ptr(), q.data_ptr(), _row_pitch(q), s.data_ptr(),
                                     _row_pitch(s), _stream(stream)), "kq_quantize_weights")
    return q, s


def kq_weights_debug(w, params, q=None, s=None, y=None, stream=None):
    """kq_quantize_weights that also returns the float32 W T^-1 [N, d]."""
    what = "kq_weights_debug"
    q, s = _outputs(w, q, s, what)
    rows, d = w.shape
    _need_transform(what, params, d // 32, KQ_T_PARAMS)
    y = _y_out(w, y, what)
    _need_device(what, w, params=params, q=q, s=s, y=y)
    _check(lib().kq_weights_debug(w.data_ptr(), _dtype_code(w), rows, d, _row_pitch(w), params.data_ptr(),
                                  q.data_ptr(), _row_pitch(q), s.data_ptr(), _row_pitch(s),
                                  y.data_ptr(), _row_pitch(y), _stream(stream)), "kq_weights_debug")
    return q, s, y


def hq_quantize(x, q=None, s=None, stream=None):
    """MXFP4 of the fixed block-Hadamard transform H x_b / sqrt(32) (comparison transform)."""
    q, s = _outputs(x, q, s, "hq_quantize")
    rows, d = x.shape
    _need_device("hq_quantize", x, q=q, s=s)
    _check(lib().hq_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), q.data_ptr(),
                             _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)), "hq_quantize")
    return q, s


def hq_transform_debug(x, q=None, s=None, y=None, stream=None):
    """hq_quantize that also returns the float32 transformed values y [rows, d]."""
    what = "hq_transform_debug"
    q, s = _outputs(x, q, s, what)
    y = _y_out(x, y, what)
    rows, d = x.shape
    _need_device(what, x, q=q, s=s, y=y)
    _check(lib().hq_transform_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), q.data_ptr(),
                                    _row_pitch(q), s.data_ptr(), _row_pitch(s), y.data_ptr(), _row_pitch(y),
                                    _stream(stream)), "hq_transform_debug")
    return q, s, y


def _ptr_or_null(t):
    return None if t is None else t.data_ptr()


def _need_modulation(what, x, shift, scale, rps):
    """shift and scale: both absent, or float32 [ceil(rows / rps), d] contiguous."""
    if (shift is None) != (scale is None):
        _fail(KQ_ERR_NULL, f"{what}: shift and scale must be given together")
    if shift is None:
        return
    rows, d = x.shape
    if rps < 1:
        _fail(KQ_ERR_SHAPE, f"{what}: rows_per_sample must be >= 1")
    samples = max(1, -(-rows // rps))
    for name, t in (("shift", shift), ("scale", scale)):
        _need_flat(what, name, t, samples * d, _f32, f"float32 [{samples}, {d}]")


def kq_norm_quantize(x, params, shift=None, scale=None, rows_per_sample=None, eps: float = 1e-6,
                     q=None, s=None, stream=None):
    """LayerNorm + (1 + scale) * . + shift per sample, block transform, MXFP4 (x before normalization)."""
    what = "kq_norm_quantize"
    q, s = _outputs(x, q, s, what)
    rows, d = x.shape
    rps = rows if rows_per_sample is None else rows_per_sample
    _need_modulation(what, x, shift, scale, rps)
    _need_transform(what, params, d // 32, KQ_T_PARAMS)
    _need_device(what, x, shift=shift, scale=scale, params=params, q=q, s=s)
    _check(lib().kq_norm_quantize(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), _ptr_or_null(shift),
                                  _ptr_or_null(scale), max(1, rps), eps, params.data_ptr(), q.data_ptr(),
                                  _row_pitch(q), s.data_ptr(), _row_pitch(s), _stream(stream)),
           "kq_norm_quantize")
    return q, s


def kq_norm_debug(x, params, shift=None, scale=None, rows_per_sample=None, eps: float = 1e-6, q=None,
                  s=None, y=None, stream=None):
    """kq_norm_quantize that also returns the float32 transformed values y [rows, d]."""
    what = "kq_norm_debug"
    q, s = _outputs(x, q, s, what)
    rows, d = x.shape
    rps = rows if rows_per_sample is None else rows_per_sample
    _need_modulation(what, x, shift, scale, rps)
    _need_transform(what, params, d // 32, KQ_T_PARAMS)
    y = _y_out(x, y, what)
    _need_device(what, x, shift=shift, scale=scale, params=params, q=q, s=s, y=y)
    _check(lib().kq_norm_debug(x.data_ptr(), _dtype_code(x), rows, d, _row_pitch(x), _ptr_or_null(shift),
                               _ptr_or_null(scale), max(1, rps), eps, params.data_ptr(), q.data_ptr(),
                               _row_pitch(q), s.data_ptr(), _row_pitch(s), y.data_ptr(), _row_pitch(y),
                               _stream(stream)), "kq_norm_debug")
    return q, s, y


def _mx_gemm(what, qa, sa, qb, sb, out, out_dtype, workspace, stream):
    import torch
    for name, t in (("qa", qa), ("sa", sa), ("qb", qb), ("sb", sb)):
        if t.dim() != 2:
            _fail(KQ_ERR_SHAPE, f"{what}: {name} must be 2-D, got {tuple(t.shape)}")
        if t.dtype != torch.uint8:
            _fail(KQ_ERR_DTYPE, f"{what}: {name} must be uint8, got {t.dtype}")
        _row_pitch(t)
    M, N, K = qa.shape[0], qb.shape[0], qa.shape[1] * 2
    if qb.shape[1] != qa.shape[1] or tuple(sa.shape) != (M, K // 32) or tuple(sb.shape) != (N, K // 32):
        raise KQError(KQ_ERR_SHAPE, f"{what}: codes [rows, K/2] and scales [rows, K/32] of both operands "
                                    "must agree on K")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=qa.device)
    code = {torch.float32: KQ_FP32, torch.bfloat16: KQ_BF16}.get(out.dtype)
    if code is None:
        raise KQError(KQ_ERR_DTYPE, f"unsupported output dtype {out.dtype}")
    if out.dim() != 2 or tuple(out.shape) != (M, N):
        _fail(KQ_ERR_SHAPE, f"{what}: out is {tuple(out.shape)}, needs ({M}, {N})")
    _row_pitch(out)
    args = (qa.data_ptr(), _row_pitch(qa), sa.data_ptr(), _row_pitch(sa), qb.data_ptr(), _row_pitch(qb),
            sb.data_ptr(), _row_pitch(sb), M, N, K, out.data_ptr(), _row_pitch(out), code)
    if workspace is False or workspace == "static":
        _need_device(what, qa, sa=sa, qb=qb, sb=sb, out=out)
        fn = lib().kq_mx_gemm if workspace is False else lib().kq_mx_gemm_static
        _check(fn(*args, _stream(stream)), what)
        return out
    if workspace is None:
        _need_device(what, qa, sa=sa, qb=qb, sb=sb, out=out)
        _check(lib().kq_mx_gemm_ws(*args, None, 0, _stream(stream)), what)
        return out
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        _fail(KQ_ERR_DTYPE, f"{what}: workspace must be a contiguous 1-D uint8 tensor")
    _need_device(what, qa, sa=sa, qb=qb, sb=sb, out=out, workspace=workspace)
    _check(lib().kq_mx_gemm_ws(*args, workspace.data_ptr(), workspace.numel(), _stream(stream)), what)
    return out


def kq_mx_gemm(qa, sa, qb, sb, out=None, out_dtype=None, stream=None):
    """W4A4 product out[m][n] = sum_k deq(A)[m][k] deq(B)[n][k] of two MXFP4 operands
    (codes [rows, K/2], scales [rows, K/32]); out float32 (default) or bfloat16."""
    return _mx_gemm("kq_mx_gemm", qa, sa, qb, sb, out, out_dtype, False, stream)


def kq_mx_gemm_fused(x, params, qb, sb, out=None, out_dtype=None, stream=None):
    """The W4A4 product with the quantizer in its prologue: out = deq(Q(T x))
    deq(B)^T from bf16 x [M, K], its float32 factor parameters [K/32, 5, 3] and the
    weights' MXFP4 operand (codes [N, K/2], scales [N, K/32]); equal to
    kq_mx_gemm(*kq_quantize(x, params), qb, sb) bit for bit."""
    return _mx_gemm_fused("kq_mx_gemm_fused", x, params, qb, sb, out, out_dtype, False, stream)


def kq_mx_gemm_fused_ws(x, params, qb, sb, workspace, out=None, out_dtype=None, stream=None):
    """kq_mx_gemm_fused with each 128 x 256 output tile split into 2, 4 or 8 parts
    of K through ``workspace`` when the library's rule splits the shape (uint8
    device tensor of kq_mx_gemm_fused_workspace_size bytes whose first 4096 bytes
    are zero before the first call; every call leaves them zero).
    ``workspace=None`` runs the unsplit product."""
    return _mx_gemm_fused("kq_mx_gemm_fused_ws", x, params, qb, sb, out, out_dtype, workspace, stream)


def kq_mx_gemm_fused_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace kq_mx_gemm_fused_ws uses for an M x N x K product on the
    current device."""
    n = ctypes.c_int64(0)
    _check(lib().kq_mx_gemm_fused_workspace_size(M, N, K, ctypes.byref(n)), "kq_mx_gemm_fused_workspace_size")
    return n.value


def _mx_gemm_fused(what, x, params, qb, sb, out, out_dtype, workspace, stream):
    import torch
    _need_input(what, x)
    if _dtype_code(x) != KQ_BF16:
        _fail(KQ_ERR_DTYPE, f"{what}: x must be bf16, got {x.dtype}")
    M, K = x.shape
    if K % 32 != 0:
        _fail(KQ_ERR_SHAPE, f"{what}: K = {K} is not a multiple of 32")
    _need_flat(what, "params", params, K // 32 * 15, _f32, "float32 [K/32, 5, 3]")
    for name, t in (("qb", qb), ("sb", sb)):
        if t.dim() != 2:
            _fail(KQ_ERR_SHAPE, f"{what}: {name} must be 2-D, got {tuple(t.shape)}")
        if t.dtype != torch.uint8:
            _fail(KQ_ERR_DTYPE, f"{what}: {name} must be uint8, got {t.dtype}")
        _row_pitch(t)
    N = qb.shape[0]
    if qb.shape[1] != K // 2 or tuple(sb.shape) != (N, K // 32):
        _fail(KQ_ERR_SHAPE, f"{what}: weights need codes [N, K/2] and scales [N, K/32] for K = {K}")
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype or torch.float32, device=x.device)
    code = {torch.float32: KQ_FP32, torch.bfloat16: KQ_BF16}.get(out.dtype)
    if code is None:
        _fail(KQ_ERR_DTYPE, f"unsupported output dtype {out.dtype}")
    if out.dim() != 2 or tuple(out.shape) != (M, N):
        _fail(KQ_ERR_SHAPE, f"{what}: out is {tuple(out.shape)}, needs ({M}, {N})")
    _row_pitch(out)
    args = (x.data_ptr(), KQ_BF16, _row_pitch(x), params.data_ptr(), qb.data_ptr(), _row_pitch(qb),
            sb.data_ptr(), _row_pitch(sb), M, N, K, out.data_ptr(), _row_pitch(out), code)
    if workspace is False:
        _need_device(what, x, params=params, qb=qb, sb=sb, out=out)
        _check(lib().kq_mx_gemm_fused(*args, _stream(stream)), what)
        return out
    if workspace is None:
        _need_device(what, x, params=params, qb=qb, sb=sb, out=out)
        _check(lib().kq_mx_gemm_fused_ws(*args, None, 0, _stream(stream)), what)
        return out
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        _fail(KQ_ERR_DTYPE, f"{what}: workspace must be a contiguous 1-D uint8 tensor")
    _need_device(what, x, params=params, qb=qb, sb=sb, out=out, workspace=workspace)
    _check(lib().kq_mx_gemm_fused_ws(*args, workspace.data_ptr(), workspace.numel(), _stream(stream)), what)
    return out


def kq_mx_gemm_static(qa, sa, qb, sb, out=None, out_dtype=None, stream=None):
    """kq_mx_gemm_ws through the library's static device workspace: allocates
    nothing (beyond ``out`` when it is not given).  Calls that overlap on one device
    race."""
    return _mx_gemm("kq_mx_gemm_static", qa, sa, qb, sb, out, out_dtype, "static", stream)


def kq_mx_gemm_workspace_size(M: int, N: int, K: int) -> int:
    """Bytes of workspace kq_mx_gemm_ws uses for an M x N x K product on the current device."""
    n = ctypes.c_int64(0)
    _check(lib().kq_mx_gemm_workspace_size(M, N, K, ctypes.byref(n)), "kq_mx_gemm_workspace_size")
    return n.value


def kq_mx_gemm_ws(qa, sa, qb, sb, workspace, out=None, out_dtype=None, stream=None):
    """kq_mx_gemm with each output tile split into 2, 4 or 8 parts of K through
    ``workspace`` when the library's rule splits the shape (uint8 device tensor of
    kq_mx_gemm_workspace_size bytes whose first 4096 bytes are zero before the
    first call; every call leaves them zero).  ``workspace=None`` runs the unsplit
    product."""
    return _mx_gemm("kq_mx_gemm_ws", qa, sa, qb, sb, out, out_dtype, workspace, stream)
