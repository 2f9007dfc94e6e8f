"""Every kernel of the HIP library keeps its working set in registers and LDS.

Each source is compiled for gfx950 to assembly (the same flags as the library)
and the compiler's per-kernel summary is read: no kernel may use scratch memory
(per-lane private memory, which lives in HBM).  Arrays of HIP's vector structs
(uint4, float4) shared between lambdas have been demoted there before, every
access then waiting for its load at once, at several times the kernel's time.
CPU only: hipcc cross-compiles without a GPU.
"""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _hipcc():
    from online_activation_quantizer_amd import build
    return build.hipcc()


pytestmark = pytest.mark.skipif(shutil.which(_hipcc()) is None and not os.path.exists(_hipcc()),
                                reason="needs hipcc")


def _kernel_scratch(src, tmpdir):
    from online_activation_quantizer_amd import build
    out = os.path.join(tmpdir, os.path.basename(src) + ".s")
    flags = [f for f in build.HIPCC_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_hipcc()] + flags + ["--cuda-device-only", "-S", "-o", out, src]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    text = open(out).read()
    # one summary per kernel: the function label, then "; ScratchSize: N" in its comment block
    names = re.findall(r"^(_Z\S+):\s", text, flags=re.M)
    sizes = [int(v) for v in re.findall(r"^; ScratchSize: (\d+)", text, flags=re.M)]
    return names, sizes


def test_no_kernel_uses_scratch(tmp_path):
    from online_activation_quantizer_amd import build
    srcs = [os.path.join(build.CSRC, s) for s in build.SOURCES + build.BENCH_SOURCES if s.endswith(".hip")]
    with ThreadPoolExecutor(4) as ex:
        results = list(ex.map(lambda s: (s, _kernel_scratch(s, str(tmp_path))), srcs))
    kernels = 0
    for src, (names, sizes) in results:
        assert sizes, f"no kernel summary in {src}"
        kernels += len(sizes)
        bad = [(n, v) for n, v in zip(names, sizes) if v]
        assert not bad and max(sizes) == 0, f"{os.path.basename(src)}: scratch in {bad or sizes}"
    assert kernels >= 20
