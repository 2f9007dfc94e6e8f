"""Host-side helpers of bench.py checked on the CPU: the MXFP4 decode used by its
quality comparison against the oracle's pinned decode."""
import numpy as np

import bench
import oracle


def test_bench_mxfp4_decode_matches_the_oracle():
    import torch
    rng = np.random.default_rng(5)
    q = rng.integers(0, 256, size=(20, 48), dtype=np.uint8)  # every code, both nibbles
    s = rng.integers(90, 170, size=(20, 3), dtype=np.uint8)
    v = bench.mxfp4_values(torch.from_numpy(q), torch.from_numpy(s)).numpy()
    ref = oracle.dequantize(q, s)
    assert v.dtype == np.float32 and v.shape == ref.shape
    assert np.array_equal(v.astype(np.float64), ref)
