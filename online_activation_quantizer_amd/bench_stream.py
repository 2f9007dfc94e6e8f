"""ctypes binding of libkq_bench.so (include/kq_bench.h): the streaming kernel
that moves the quantizer's bytes without its arithmetic, used by the benchmark
to report the practical HBM ceiling of one call beside the quantizer's time."""
from __future__ import annotations

import ctypes
import os

from .kq import KQError

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libkq_bench.so")
EXPORTED_SYMBOLS = ("kq_bench_stream",)

_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise KQError(-7, f"libkq_bench.so not built at {LIB_PATH}; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        L.kq_bench_stream.argtypes = [P, I64, P, P, I, P]
        L.kq_bench_stream.restype = I
        _lib = L
    return _lib


def kq_bench_stream(x, q, s, grid: int, stream=None):
    """Stream x (contiguous, 64 bytes per unit) into q (16 B per unit) and s (1 B per unit)."""
    import torch
    units = x.numel() * x.element_size() // 64
    st = stream.cuda_stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = lib().kq_bench_stream(x.data_ptr(), units, q.data_ptr(), s.data_ptr(), grid, st)
    if rc != 0:
        raise KQError(rc, "kq_bench_stream")
