"""Helpers of the GPU parity tests: device copies of synthetic inputs and the
parity verdict (the oracle's classify rule) for one call of the HIP path."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import online_activation_quantizer_amd as kq

# Pre-quantization tolerance when the transform runs in fp32: 1e-5 * max|x_block|
# (tol_mode 0).  Excused code/scale mismatches must stay below 1e-4 of elements.
FP32_TOL = (0, 1e-5)
EXCUSED_FRACTION = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t) -> np.ndarray:
    import torch
    a = t.cpu()
    if a.dtype in (torch.int16, torch.bfloat16):
        return a.view(torch.int16).numpy().view(np.uint16)
    return a.numpy()


def verdict(x: np.ndarray, y_o: np.ndarray, q, s, y_c=None, tol=FP32_TOL) -> dict:
    st = oracle.classify(x, y_o, q, s, tol[0], tol[1], y_c=y_c)
    st["pass"] = (st["unexcused"] == 0 and st["excused"] < EXCUSED_FRACTION * max(1, st["elements"])
                  and (y_c is None or st["prequant_violations"] == 0))
    return st


def run_kq(x: np.ndarray, params: np.ndarray, debug: bool = True, variant: int = kq.KQ_AUTO):
    """HIP path on (x, params): returns host (q, s, y or None), from the production
    entry point, after checking the validation entry point agrees with it bit for bit."""
    import torch
    xd, pd = dev(x), dev(params)
    if variant == kq.KQ_MFMA:
        t = kq.kq_expand_factors(pd, kq.KQ_T_DENSE_BF16X3)
        tfmt = kq.KQ_T_DENSE_BF16X3
    else:
        t, tfmt = pd, kq.KQ_T_PARAMS
    q, s = kq.kq_quantize(xd, t, tfmt, variant)
    y = None
    if debug:
        q2, s2, yd = kq.kq_transform_debug(xd, t, tfmt, variant)
        torch.cuda.synchronize()
        assert torch.equal(q, q2) and torch.equal(s, s2), "debug and production kernels disagree"
        y = host(yd)
    torch.cuda.synchronize()
    return host(q), host(s), y
