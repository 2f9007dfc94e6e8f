"""The host code under the address and undefined-behaviour sanitizers (CPU only).

* The C ABI's argument checks (csrc/kq_api.cpp, built with g++ for the host, the
  kernel launches replaced by stand-ins that the rejected calls never reach) run
  through tests/native/abi_checks.cpp.
* The oracle (oracle/kq_oracle.cpp) built with the same sanitizers runs the pin
  suite (without the 2^32 sweep) in a subprocess with the sanitizer runtime
  preloaded into Python; any report aborts it.
"""
import os
import shutil
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
       "-g", "-O1"]
ENV_SAN = {"ASAN_OPTIONS": "detect_leaks=0:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.skipif(not os.path.exists(os.path.join(ROCM, "include", "hip", "hip_runtime.h")),
                    reason="needs the HIP headers")
def test_abi_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_checks")
    csrc = os.path.join(ROOT, "online_activation_quantizer_amd", "csrc")
    cmd = (["g++", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
            "-I", os.path.join(ROOT, "include")] + SAN +
           ["-o", exe, os.path.join(HERE, "native", "abi_checks.cpp"), os.path.join(csrc, "kq_api.cpp"),
            os.path.join(HERE, "native", "launch_stubs.cpp"), "-L", os.path.join(ROCM, "lib"),
            "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lamdhip64"])
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=dict(os.environ, **ENV_SAN))
    assert res.returncode == 0, res.stdout + res.stderr
    assert "all passed" in res.stdout


def test_oracle_pins_under_sanitizers(tmp_path):
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("no libasan")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["g++", "-std=c++17", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"] + SAN +
                   ["-I", os.path.join(ROOT, "oracle"), "-o", lib, os.path.join(ROOT, "oracle", "kq_oracle.cpp")],
                   check=True, capture_output=True, text=True)
    env = dict(os.environ, KQ_ORACLE_LIB=lib, LD_PRELOAD=asan, **ENV_SAN)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_oracle_pins.py"), "-k", "not exhaustive"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    assert res.returncode == 0, res.stdout[-3000:] + res.stderr[-3000:]
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr, res.stderr[-3000:]
