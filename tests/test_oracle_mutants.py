"""The pins catch plausible mistakes in the oracle.

Each mutant is the oracle's source with one plausible slip planted (a transposed
operand, a reversed Kronecker order, a dropped term, an off-by-one exponent, a
wrong tie or sign rule...).  It is compiled to a temporary library and the pin
suite (tests/test_oracle_pins.py, without the 2^32 sweep) is run against it in a
subprocess: every mutant must make at least one pin fail.  Nothing here touches
the oracle that the other tests use.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "kq_oracle.cpp")

MUTANTS = {
    "factor_u_times_l": (
        "F[2 * i + j] = L[2 * i + 0] * U[0 * 2 + j] + L[2 * i + 1] * U[1 * 2 + j];",
        "F[2 * i + j] = U[2 * i + 0] * L[0 * 2 + j] + U[2 * i + 1] * L[1 * 2 + j];"),
    "dropped_inverse_u": (
        "const double U[4] = {u, v, 0.0, 1.0 / u};",
        "const double U[4] = {u, v, 0.0, u};"),
    "inverse_sign": (
        "const double Ui[4] = {1.0 / u, -v, 0.0, u};",
        "const double Ui[4] = {1.0 / u, v, 0.0, u};"),
    "reversed_kron_order": (
        "oq_kron(F[k], 2, 2, acc.data(), n, n, next.data());",
        "oq_kron(acc.data(), n, n, F[k], 2, 2, next.data());"),
    "transposed_T": (
        "acc += Tb[i * kBlk + j] * xb[j];",
        "acc += Tb[j * kBlk + i] * xb[j];"),
    "scale_off_by_one": (
        "int e = (E - 1) - 2;",
        "int e = (E - 1) - 1;"),
    "no_scale_clamp": (
        "return std::min(127, std::max(-127, e));",
        "return e;"),
    "ties_round_up": (
        "if (r <= 0.25) m = 0;",
        "if (r < 0.25) m = 0;"),
    "no_saturation": (
        "  else m = 7;",
        "  else if (r <= 7.0) m = 7;\n  else m = 0;"),
    "sign_dropped": (
        "const int sign = std::signbit(y) ? 8 : 0;",
        "const int sign = 0;"),
    "nibbles_swapped": (
        "qb[i / 2] = (uint8_t)(oq_e2m1_code(yb[i], e) | (oq_e2m1_code(yb[i + 1], e) << 4));",
        "qb[i / 2] = (uint8_t)(oq_e2m1_code(yb[i + 1], e) | (oq_e2m1_code(yb[i], e) << 4));"),
    "weight_side_transposed": (
        "for (int i = 0; i < kBlk; ++i) acc += wb[i] * Tb[i * kBlk + j];",
        "for (int i = 0; i < kBlk; ++i) acc += wb[i] * Tb[j * kBlk + i];"),
    "hadamard_wrong_sign_rule": (
        "H[i][j] = (__builtin_popcount(i & j) & 1) ? -1.0 : 1.0;",
        "H[i][j] = (__builtin_popcount(i | j) & 1) ? -1.0 : 1.0;"),
    "hadamard_scale_dropped": (
        "y[t * d + b * kBlk + i] = acc * norm;",
        "y[t * d + b * kBlk + i] = acc;"),
    "norm_unbiased_variance": (
        "      var /= (double)d;",
        "      var /= (double)(d - 1);"),
    "norm_scale_without_one": (
        "hr[c] = (hr[c] - mu) * rstd * (1.0 + sc) + sh;",
        "hr[c] = (hr[c] - mu) * rstd * sc + sh;"),
    "norm_sample_index_modulo": (
        "const int64_t g = row / rows_per_sample;",
        "const int64_t g = row % rows_per_sample;"),
    "dequant_nibbles_swapped": (
        "const int code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
        "const int code = (c % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    "dequant_scale_bias": (
        "out[t * d + c] = S == 0xFF ? std::nan(\"\") : oq_e2m1_value(code, S - 127);",
        "out[t * d + c] = S == 0xFF ? std::nan(\"\") : oq_e2m1_value(code, S - 128);"),
    "amax_without_abs": (
        "        amax = std::max(amax, std::fabs(yb[i]));\n      }\n      uint8_t* qb",
        "        amax = std::max(amax, yb[i]);\n      }\n      uint8_t* qb"),
}


def build_mutant(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site of {name} not unique"
    path = os.path.join(tmpdir, f"{name}.cpp")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = os.path.join(tmpdir, f"lib_{name}.so")
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-I", os.path.join(ROOT, "oracle"), "-o", lib, path], check=True)
    return lib


def run_pins(lib):
    env = dict(os.environ, KQ_ORACLE_LIB=lib)
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(HERE, "test_oracle_pins.py"), "-k", "not exhaustive"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return res.returncode, res.stdout[-400:]


def test_unmutated_source_passes_the_pins(tmp_path):
    src = open(SRC).read()
    path = tmp_path / "same.cpp"
    path.write_text(src)
    lib = str(tmp_path / "lib_same.so")
    subprocess.run(["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                    "-I", os.path.join(ROOT, "oracle"), "-o", lib, str(path)], check=True)
    rc, out = run_pins(lib)
    assert rc == 0, out


def test_every_mutant_is_caught(tmp_path):
    names = sorted(MUTANTS)
    libs = {n: build_mutant(n, str(tmp_path)) for n in names}
    with ThreadPoolExecutor(4) as ex:
        results = dict(zip(names, ex.map(lambda n: run_pins(libs[n]), names)))
    survivors = [n for n, (rc, _) in results.items() if rc == 0]
    assert not survivors, f"mutants not caught by any pin: {survivors}"
