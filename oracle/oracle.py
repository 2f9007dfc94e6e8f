"""ctypes front end of the C++ fp64 oracle (``kq_oracle.cpp``).

TEST INFRASTRUCTURE ONLY.  Each function mirrors one C entry point; the
arithmetic lives in the C++ file, whose header names the passages it follows.
The pages print no numeric worked example for this path, so every function is
pinned by closed forms, invariants, brute force and hand-derived examples in the
tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liboracle_kq.so")
# The mutation tests point the pins at deliberately broken builds of the oracle.
_LIB_OVERRIDE = os.environ.get("KQ_ORACLE_LIB")
SOURCES = [os.path.join(HERE, "kq_oracle.cpp")]

BF16, FP32 = 0, 1
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with g++ (-O2, no FMA contraction) into liboracle_kq.so."""
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    tmp = LIB_PATH + ".tmp"
    cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", "-pthread", "-Wall", "-Wextra", "-o", tmp] + SOURCES
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


def lib():
    global _lib
    if _lib is None:
        path = _LIB_OVERRIDE or LIB_PATH
        if not _LIB_OVERRIDE and not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(path)
        P, I64, I, D = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
        L.oq_factor.argtypes = [D, D, D, P]
        L.oq_factor_inverse.argtypes = [D, D, D, P]
        L.oq_kron.argtypes = [P, I, I, P, I, I, P]
        L.oq_expand.argtypes = [P, I64, I, P]
        L.oq_det.argtypes = [P, I]
        L.oq_det.restype = D
        L.oq_transform_dense.argtypes = [P, I, I64, I64, I64, P, P]
        L.oq_transform_factored.argtypes = [P, I, I64, I64, I64, P, P]
        L.oq_scale_exp.argtypes = [D]
        L.oq_e2m1_code.argtypes = [D, I]
        L.oq_e2m1_value.argtypes = [I, I]
        L.oq_e2m1_value.restype = D
        L.oq_encode.argtypes = [P, I64, I64, P, I64, P, I64]
        L.oq_quantize.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P, I]
        L.oq_sq_quantize.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P, I]
        L.oq_hadamard_quantize.argtypes = [P, I, I64, I64, I64, P, I64, P, I64, P, I]
        L.oq_norm_quantize.argtypes = [P, I, I64, I64, I64, P, P, I64, ctypes.c_double, P, P, I64, P, I64,
                                       P, P, I]
        L.oq_dequantize.argtypes = [P, I64, P, I64, I64, I64, P]
        L.oq_weight_transform.argtypes = [P, I, I64, I64, I64, P, P]
        L.oq_quantize_weights.argtypes = [P, I, I64, I64, I64, P, P, I64, P, I64, P, I]
        L.oq_classify.argtypes = [P, I, I64, I64, I64, P, I, D, P, I64, P, I64, P, I64, P]
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def _x_info(x: np.ndarray):
    """(dtype code, rows, ldx) of an input held as uint16 bf16 bits or float32."""
    if x.dtype == np.uint16:
        dt = BF16
    elif x.dtype == np.float32:
        dt = FP32
    else:
        raise TypeError("oracle input must be uint16 (bf16 bits) or float32")
    if x.ndim != 2 or x.strides[1] != x.itemsize or x.strides[0] % x.itemsize:
        raise ValueError("oracle input must be a 2-D array with unit column stride")
    return dt, x.shape[0], x.strides[0] // x.itemsize


def factor(l, u, v):
    F = np.zeros(4, np.float64)
    lib().oq_factor(l, u, v, _ptr(F))
    return F.reshape(2, 2)


def factor_inverse(l, u, v):
    F = np.zeros(4, np.float64)
    lib().oq_factor_inverse(l, u, v, _ptr(F))
    return F.reshape(2, 2)


def kron(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    A = np.ascontiguousarray(A, np.float64)
    B = np.ascontiguousarray(B, np.float64)
    C = np.zeros((A.shape[0] * B.shape[0], A.shape[1] * B.shape[1]), np.float64)
    lib().oq_kron(_ptr(A), A.shape[0], A.shape[1], _ptr(B), B.shape[0], B.shape[1], _ptr(C))
    return C


def expand(params: np.ndarray, inverse: bool = False) -> np.ndarray:
    p = np.ascontiguousarray(params, np.float32)
    nb = p.shape[0]
    assert p.shape == (nb, 5, 3)
    T = np.zeros((nb, 32, 32), np.float64)
    _check(lib().oq_expand(_ptr(p), nb, int(inverse), _ptr(T)), "expand")
    return T


def det(A: np.ndarray) -> float:
    A = np.ascontiguousarray(A, np.float64)
    return lib().oq_det(_ptr(A), A.shape[0])


def transform_dense(x: np.ndarray, T: np.ndarray) -> np.ndarray:
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    Tm = np.ascontiguousarray(T, np.float64)
    y = np.zeros((rows, d), np.float64)
    _check(lib().oq_transform_dense(_ptr(x), dt, rows, d, ldx, _ptr(Tm), _ptr(y)), "transform_dense")
    return y


def transform_factored(x: np.ndarray, params: np.ndarray) -> np.ndarray:
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    p = np.ascontiguousarray(params, np.float32)
    y = np.zeros((rows, d), np.float64)
    _check(lib().oq_transform_factored(_ptr(x), dt, rows, d, ldx, _ptr(p), _ptr(y)), "transform_factored")
    return y


def scale_exp(amax: float) -> int:
    return lib().oq_scale_exp(float(amax))


def e2m1_code(y: float, e: int) -> int:
    return lib().oq_e2m1_code(float(y), int(e))


def e2m1_value(code: int, e: int) -> float:
    return lib().oq_e2m1_value(int(code), int(e))


def encode(y: np.ndarray):
    y = np.ascontiguousarray(y, np.float64)
    rows, d = y.shape
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    _check(lib().oq_encode(_ptr(y), rows, d, _ptr(q), d // 2, _ptr(s), d // 32), "encode")
    return q, s


def quantize(x: np.ndarray, params: np.ndarray, want_y: bool = False, nthreads: int = 0):
    """Returns (q [rows, d/2] uint8, s [rows, d/32] uint8, y fp64 or None)."""
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    p = np.ascontiguousarray(params, np.float32)
    assert p.shape == (d // 32, 5, 3)
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    y = np.zeros((rows, d), np.float64) if want_y else None
    rc = lib().oq_quantize(_ptr(x), dt, rows, d, ldx, _ptr(p), _ptr(q), d // 2, _ptr(s), d // 32,
                           _ptr(y) if want_y else None, nthreads)
    _check(rc, "quantize")
    return q, s, y


def sq_quantize(x: np.ndarray, mult: np.ndarray, want_y: bool = False, nthreads: int = 0):
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    m = np.ascontiguousarray(mult, np.float32)
    assert m.shape == (d,)
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    y = np.zeros((rows, d), np.float64) if want_y else None
    rc = lib().oq_sq_quantize(_ptr(x), dt, rows, d, ldx, _ptr(m), _ptr(q), d // 2, _ptr(s), d // 32,
                              _ptr(y) if want_y else None, nthreads)
    _check(rc, "sq_quantize")
    return q, s, y


def hadamard_quantize(x: np.ndarray, want_y: bool = False, nthreads: int = 0):
    """(q, s, y fp64 or None) of the fixed block-Hadamard comparison transform."""
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    y = np.zeros((rows, d), np.float64) if want_y else None
    rc = lib().oq_hadamard_quantize(_ptr(x), dt, rows, d, ldx, _ptr(q), d // 2, _ptr(s), d // 32,
                                    _ptr(y) if want_y else None, nthreads)
    _check(rc, "hadamard_quantize")
    return q, s, y


def norm_quantize(x: np.ndarray, params: np.ndarray, shift=None, scale=None, rows_per_sample=None,
                  eps: float = 1e-6, want_y: bool = False, nthreads: int = 0):
    """(q, s, h fp64, y fp64 or None): LayerNorm (no affine) + adaptive-norm modulation
    (1 + scale) * . + shift per sample, then the block transform and MXFP4."""
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    p = np.ascontiguousarray(params, np.float32)
    rps = rows if rows_per_sample is None else rows_per_sample
    sh = None if shift is None else np.ascontiguousarray(shift, np.float32)
    sc = None if scale is None else np.ascontiguousarray(scale, np.float32)
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    h = np.zeros((rows, d), np.float64)
    y = np.zeros((rows, d), np.float64) if want_y else None
    rc = lib().oq_norm_quantize(_ptr(x), dt, rows, d, ldx, _ptr(sh) if sh is not None else None,
                                _ptr(sc) if sc is not None else None, max(1, rps), eps, _ptr(p), _ptr(q),
                                d // 2, _ptr(s), d // 32, _ptr(h), _ptr(y) if want_y else None, nthreads)
    _check(rc, "norm_quantize")
    return q, s, h, y


def dequantize(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """fp64 values of MXFP4 rows (q [rows, d/2], s [rows, d/32])."""
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    rows, d = q.shape[0], q.shape[1] * 2
    out = np.zeros((rows, d), np.float64)
    _check(lib().oq_dequantize(_ptr(q), q.shape[1], _ptr(s), s.shape[1], rows, d, _ptr(out)), "dequantize")
    return out


def mx_gemm(qa, sa, qb, sb, rows=None, cols=None):
    """Reference W4A4 product: Y[i][j] = sum_c deq(A)[i][c] * deq(B)[j][c] over the selected
    rows of A and rows of B (all when None), with the sum of |terms| beside it (the
    scale of the fp32 accumulation error).  Every product of two decoded MXFP4 values
    is exact in fp64; the fp64 sum's rounding is far below any fp32 tolerance."""
    ia = slice(None) if rows is None else np.asarray(rows)
    ib = slice(None) if cols is None else np.asarray(cols)
    A = dequantize(np.ascontiguousarray(qa[ia]), np.ascontiguousarray(sa[ia]))
    B = dequantize(np.ascontiguousarray(qb[ib]), np.ascontiguousarray(sb[ib]))
    return A @ B.T, np.abs(A) @ np.abs(B).T


def weight_transform(w: np.ndarray, params: np.ndarray) -> np.ndarray:
    """W' = W T^-1 (block-diagonal), fp64 [rows, d]."""
    dt, rows, ldw = _x_info(w)
    d = w.shape[1]
    p = np.ascontiguousarray(params, np.float32)
    out = np.zeros((rows, d), np.float64)
    _check(lib().oq_weight_transform(_ptr(w), dt, rows, d, ldw, _ptr(p), _ptr(out)), "weight_transform")
    return out


def quantize_weights(w: np.ndarray, params: np.ndarray, want_y: bool = False, nthreads: int = 0):
    """(q [rows, d/2], s [rows, d/32], W' fp64 or None): MXFP4 of W T^-1 along d."""
    dt, rows, ldw = _x_info(w)
    d = w.shape[1]
    p = np.ascontiguousarray(params, np.float32)
    q = np.zeros((rows, d // 2), np.uint8)
    s = np.zeros((rows, d // 32), np.uint8)
    y = np.zeros((rows, d), np.float64) if want_y else None
    rc = lib().oq_quantize_weights(_ptr(w), dt, rows, d, ldw, _ptr(p), _ptr(q), d // 2, _ptr(s), d // 32,
                                   _ptr(y) if want_y else None, nthreads)
    _check(rc, "quantize_weights")
    return q, s, y


STAT_NAMES = ("exact", "excused", "unexcused", "excused_scale_blocks", "unexcused_scale_blocks",
              "prequant_violations", "max_norm_prequant_err", "first_unexcused")


def classify(x: np.ndarray, y_o: np.ndarray, q: np.ndarray, s: np.ndarray, tol_mode: int = 0,
             tol_coef: float = 1e-5, y_c: np.ndarray | None = None) -> dict:
    """Parity accounting of candidate (q, s[, y_c]) against the oracle's y_o."""
    dt, rows, ldx = _x_info(x)
    d = x.shape[1]
    y_o = np.ascontiguousarray(y_o, np.float64)
    q = np.ascontiguousarray(q, np.uint8)
    s = np.ascontiguousarray(s, np.uint8)
    assert y_o.shape == (rows, d) and q.shape == (rows, d // 2) and s.shape == (rows, d // 32)
    if y_c is not None:
        y_c = np.ascontiguousarray(y_c, np.float32)
        assert y_c.shape == (rows, d)
    st = np.zeros(8, np.float64)
    rc = lib().oq_classify(_ptr(x), dt, rows, d, ldx, _ptr(y_o), tol_mode, tol_coef,
                           _ptr(q), d // 2, _ptr(s), d // 32,
                           _ptr(y_c) if y_c is not None else None, d, _ptr(st))
    _check(rc, "classify")
    out = dict(zip(STAT_NAMES, st.tolist()))
    out["elements"] = rows * d
    return out
