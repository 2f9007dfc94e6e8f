"""The C ABI without a GPU: the library loads, exports every symbol the header
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    import online_activation_quantizer_amd as kq
    from online_activation_quantizer_amd import build
    if not os.path.exists(build.LIB_PATH):
        build.build()
    return kq.lib()


def header_functions(name="kq.h"):
    text = open(os.path.join(ROOT, "include", name)).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_header_symbols_exported(L):
    names = header_functions()
    assert {"kq_expand_factors", "kq_quantize", "sq_quantize", "kq_transform_debug",
            "sq_transform_debug", "kq_quantize_weights", "kq_weights_debug", "hq_quantize",
            "hq_transform_debug", "kq_norm_quantize", "kq_norm_debug", "kq_mx_gemm",
            "kq_mx_gemm_workspace_size", "kq_mx_gemm_ws", "kq_mx_gemm_static", "kq_mx_gemm_fused",
            "kq_mx_gemm_fused_workspace_size", "kq_mx_gemm_fused_ws", "kq_status_string",
            "kq_last_hip_error"} <= set(names)
    for n in names:
        assert hasattr(L, n), n


def test_every_header_is_covered():
    # each public header belongs to one of the two libraries checked here
    assert sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")) == \
        ["kq.h", "kq_bench.h"]


def test_bench_helper_library(L):
    from online_activation_quantizer_amd import bench_stream
    B = bench_stream.lib()
    names = header_functions("kq_bench.h")
    assert names == ["kq_bench_stream", "kq_bench_stream_design"]
    for n in names:
        assert hasattr(B, n), n
    assert B.kq_bench_stream_design(X, 4, Q, S, 8, 5, None) == SHAPE
    assert B.kq_bench_stream_design(X, 4, Q, S, 8, -1, None) == SHAPE
    assert B.kq_bench_stream_design(X, 1 << 30, Q, S, 8, 0, None) == SHAPE
    assert B.kq_bench_stream_design(None, 4, Q, S, 8, 2, None) == NULL
    assert B.kq_bench_stream_design(X, 4, Q + 8, S, 8, 1, None) == ALIGN
    assert B.kq_bench_stream(X, 4, Q, S, 0, None) == SHAPE
    assert B.kq_bench_stream(X, -1, Q, S, 8, None) == SHAPE
    assert B.kq_bench_stream(None, 4, Q, S, 8, None) == NULL
    assert B.kq_bench_stream(X + 4, 4, Q, S, 8, None) == ALIGN
    assert B.kq_bench_stream(None, 0, None, None, 8, None) == OK


def test_oracle_not_linked_into_product(L):
    # the product library must not contain the oracle's entry points
    for n in ("oq_quantize", "oq_encode", "oq_classify"):
        assert not hasattr(L, n)


# fake, suitably aligned device addresses: validation never dereferences them
X, T, Q, S, Y = 0x10000, 0x20000, 0x30000, 0x40000, 0x50000
OK, NULL, SHAPE, ALIGN, DTYPE, FORMAT, VARIANT = 0, -1, -2, -3, -4, -5, -6


def quant(L, x=X, dtype=0, rows=4, d=64, ldx=64, t=T, tfmt=0, q=Q, ldq=32, s=S, lds=2, variant=0):
    return L.kq_quantize(x, dtype, rows, d, ldx, t, tfmt, q, ldq, s, lds, variant, None)


@pytest.mark.parametrize("kw,rc", [
    (dict(dtype=7), DTYPE),
    (dict(d=48, ldx=48), SHAPE),
    (dict(d=0, ldx=0), SHAPE),
    (dict(rows=-1), SHAPE),
    (dict(ldx=32), SHAPE),
    (dict(ldq=16), SHAPE),
    (dict(lds=1), SHAPE),
    (dict(x=None), NULL),
    (dict(t=None), NULL),
    (dict(q=None), NULL),
    (dict(s=None), NULL),
    (dict(x=X + 8), ALIGN),
    (dict(q=Q + 4), ALIGN),
    (dict(ldx=68), ALIGN),
    (dict(ldq=40), ALIGN),
    (dict(t=T + 2), ALIGN),
    (dict(tfmt=9), FORMAT),
    (dict(tfmt=1), FORMAT),          # dense fp32 is not a kq_quantize input
    (dict(tfmt=0, variant=2), FORMAT),  # matrix cores need the bf16x3 split
    (dict(tfmt=2, variant=1), FORMAT),  # the butterfly needs the factors
    (dict(variant=5), VARIANT),
    (dict(tfmt=2, variant=2, dtype=1), DTYPE),  # matrix-core path takes bf16 only
    (dict(rows=0, x=None, t=None, q=None, s=None), OK),  # no-op, no HIP call
])
def test_quantize_validation(L, kw, rc):
    assert quant(L, **kw) == rc


def test_sq_and_debug_validation(L):
    assert L.sq_quantize(X, 0, 4, 64, 64, None, Q, 32, S, 2, None) == NULL
    assert L.sq_quantize(X, 0, 4, 64, 64, T + 4, Q, 32, S, 2, None) == ALIGN  # mult needs 16 B
    assert L.sq_quantize(X, 3, 4, 64, 64, T, Q, 32, S, 2, None) == DTYPE
    assert L.sq_quantize(None, 0, 0, 64, 64, None, None, 32, None, 2, None) == OK
    assert L.kq_transform_debug(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0, None, 64, None) == NULL
    assert L.kq_transform_debug(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0, Y, 32, None) == SHAPE
    assert L.kq_transform_debug(X, 0, 4, 64, 64, T, 0, Q, 32, S, 2, 0, Y + 2, 64, None) == ALIGN
    assert L.sq_transform_debug(X, 0, 4, 64, 64, T, Q, 32, S, 2, None, 64, None) == NULL


def test_weights_validation(L):
    assert L.kq_quantize_weights(X, 0, 4, 64, 64, None, Q, 32, S, 2, None) == NULL
    assert L.kq_quantize_weights(X, 0, 4, 64, 64, T + 2, Q, 32, S, 2, None) == ALIGN
    assert L.kq_quantize_weights(X, 5, 4, 64, 64, T, Q, 32, S, 2, None) == DTYPE
    assert L.kq_quantize_weights(X, 0, 4, 48, 48, T, Q, 24, S, 2, None) == SHAPE
    assert L.kq_quantize_weights(X + 8, 0, 4, 64, 64, T, Q, 32, S, 2, None) == ALIGN
    assert L.kq_quantize_weights(None, 0, 0, 64, 64, None, None, 32, None, 2, None) == OK
    assert L.kq_weights_debug(X, 0, 4, 64, 64, T, Q, 32, S, 2, None, 64, None) == NULL
    assert L.kq_weights_debug(X, 0, 4, 64, 64, T, Q, 32, S, 2, Y, 32, None) == SHAPE


def test_hadamard_validation(L):
    assert L.hq_quantize(None, 0, 4, 64, 64, Q, 32, S, 2, None) == NULL
    assert L.hq_quantize(X, 0, 4, 64, 64, None, 32, S, 2, None) == NULL
    assert L.hq_quantize(X, 0, 4, 64, 64, Q, 32, None, 2, None) == NULL
    assert L.hq_quantize(X, 2, 4, 64, 64, Q, 32, S, 2, None) == DTYPE
    assert L.hq_quantize(X, 0, 4, 40, 40, Q, 20, S, 2, None) == SHAPE
    assert L.hq_quantize(X + 4, 0, 4, 64, 64, Q, 32, S, 2, None) == ALIGN
    assert L.hq_quantize(None, 0, 0, 64, 64, None, 32, None, 2, None) == OK
    assert L.hq_transform_debug(X, 0, 4, 64, 64, Q, 32, S, 2, None, 64, None) == NULL
    assert L.hq_transform_debug(X, 0, 4, 64, 64, Q, 32, S, 2, Y, 63, None) == SHAPE


def test_norm_validation(L):
    def norm(x=X, dtype=0, rows=4, d=64, ldx=64, shift=Y, scale=Y + 256, rps=4, eps=1e-6, p=T, q=Q,
             ldq=32, s=S, lds=2):
        return L.kq_norm_quantize(x, dtype, rows, d, ldx, shift, scale, rps, eps, p, q, ldq, s, lds, None)
    assert norm(rps=0) == SHAPE
    assert norm(eps=-1.0) == -8
    assert norm(eps=float("nan")) == -8
    assert norm(eps=float("inf")) == -8
    assert norm(shift=None) == NULL          # one modulation vector alone
    assert norm(scale=None) == NULL
    assert norm(shift=Y + 4) == ALIGN
    assert norm(p=None) == NULL
    assert norm(p=T + 2) == ALIGN
    assert norm(dtype=9) == DTYPE
    assert norm(d=48, ldx=48) == SHAPE
    assert norm(d=16416, ldx=16416, q=Q, ldq=8208, lds=513) == SHAPE  # wider than one workgroup
    assert norm(x=None, rows=0, p=None, q=None, s=None) == OK
    assert L.kq_norm_debug(X, 0, 4, 64, 64, None, None, 4, 1e-6, T, Q, 32, S, 2, None, 64, None) == NULL
    assert L.kq_status_string(-8) == b"scalar argument out of range"


def test_mx_gemm_validation(L):
    def g(qa=Q, lda=64, sa=S, ldsa=4, qb=T, ldb=64, sb=Y, ldsb=4, M=8, N=8, K=128, out=X, ldo=8, dt=1):
        return L.kq_mx_gemm(qa, lda, sa, ldsa, qb, ldb, sb, ldsb, M, N, K, out, ldo, dt, None)
    assert g(dt=5) == DTYPE
    assert g(K=48, lda=32, ldb=32) == SHAPE     # K not a multiple of 32
    assert g(K=0) == SHAPE
    assert g(lda=32) == SHAPE                    # pitch below K/2
    assert g(ldsa=3) == SHAPE
    assert g(ldo=7) == SHAPE
    assert g(M=-1) == SHAPE
    assert g(qa=None) == NULL
    assert g(sb=None) == NULL
    assert g(out=None) == NULL
    assert g(qa=Q + 8) == ALIGN
    assert g(lda=72) == ALIGN
    assert g(out=X + 2) == ALIGN                 # fp32 output needs 4 bytes
    assert g(M=0, qa=None, sa=None, qb=None, sb=None, out=None) == OK
    assert g(lda=1 << 24) == SHAPE               # a tile's rows read through one 32-bit range
    assert g(ldb=1 << 24) == SHAPE


def test_mx_gemm_fused_validation(L):
    def g(x=X, dt=0, ldx=128, p=T, qb=Q, ldb=64, sb=S, ldsb=4, M=8, N=8, K=128, out=Y, ldo=8, odt=1):
        return L.kq_mx_gemm_fused(x, dt, ldx, p, qb, ldb, sb, ldsb, M, N, K, out, ldo, odt, None)
    assert g(dt=1) == DTYPE                      # fp32 activations: the prologue reads bf16
    assert g(odt=7) == DTYPE
    assert g(K=48, ldb=32) == SHAPE              # K not a multiple of 32
    assert g(K=16416, ldx=16416, ldb=8208, ldsb=513) == SHAPE  # 513 blocks: past the on-chip constants
    assert g(ldx=64) == SHAPE                    # row pitch below K
    assert g(ldsb=3) == SHAPE
    assert g(p=None) == NULL
    assert g(x=None) == NULL
    assert g(x=X + 8) == ALIGN
    assert g(ldx=132) == ALIGN                   # 264-byte rows
    assert g(M=0, x=None, p=None, qb=None, sb=None, out=None) == OK


def test_mx_gemm_fused_workspace_validation(L):
    W = 0x60000

    def g(ws=W, nbytes=1 << 20, **kw):
        a = dict(x=X, dt=0, ldx=128, p=T, qb=Q, ldb=64, sb=S, ldsb=4, M=8, N=8, K=128, out=Y, ldo=8, odt=1)
        a.update(kw)
        return L.kq_mx_gemm_fused_ws(a["x"], a["dt"], a["ldx"], a["p"], a["qb"], a["ldb"], a["sb"], a["ldsb"],
                                     a["M"], a["N"], a["K"], a["out"], a["ldo"], a["odt"], ws, nbytes, None)
    assert g(dt=1) == DTYPE                      # the fused product's own checks come first
    assert g(K=48, ldb=32) == SHAPE
    assert g(p=None) == NULL
    assert g(ws=None, nbytes=4096) == NULL       # a size without a workspace
    assert g(ws=W + 128) == ALIGN                # 256-byte alignment
    assert g(M=0, ws=None, nbytes=0, x=None, p=None, qb=None, sb=None, out=None) == OK
    n = ctypes.c_int64(-1)
    assert L.kq_mx_gemm_fused_workspace_size(8, 8, 128, None) == NULL
    assert L.kq_mx_gemm_fused_workspace_size(8, 8, 48, ctypes.byref(n)) == SHAPE
    assert L.kq_mx_gemm_fused_workspace_size(8, 8, 16416, ctypes.byref(n)) == SHAPE  # past the on-chip constants
    assert L.kq_mx_gemm_fused_workspace_size(0, 8, 128, ctypes.byref(n)) == OK and n.value == 0


def test_mx_gemm_workspace_validation(L):
    W = 0x60000

    def g(ws=W, nbytes=1 << 20, **kw):
        a = dict(qa=Q, lda=64, sa=S, ldsa=4, qb=T, ldb=64, sb=Y, ldsb=4, M=8, N=8, K=128, out=X, ldo=8, dt=1)
        a.update(kw)
        return L.kq_mx_gemm_ws(a["qa"], a["lda"], a["sa"], a["ldsa"], a["qb"], a["ldb"], a["sb"], a["ldsb"],
                               a["M"], a["N"], a["K"], a["out"], a["ldo"], a["dt"], ws, nbytes, None)
    assert g(K=48, lda=32, ldb=32) == SHAPE      # the product's own checks come first
    assert g(qa=None) == NULL
    assert g(ws=None, nbytes=4096) == NULL       # a size without a workspace
    assert g(ws=W + 128) == ALIGN                # 256-byte alignment
    assert g(M=0, ws=None, nbytes=0, qa=None, sa=None, qb=None, sb=None, out=None) == OK
    def st(**kw):
        a = dict(qa=Q, lda=64, sa=S, ldsa=4, qb=T, ldb=64, sb=Y, ldsb=4, M=8, N=8, K=128, out=X, ldo=8, dt=1)
        a.update(kw)
        return L.kq_mx_gemm_static(a["qa"], a["lda"], a["sa"], a["ldsa"], a["qb"], a["ldb"], a["sb"],
                                   a["ldsb"], a["M"], a["N"], a["K"], a["out"], a["ldo"], a["dt"], None)
    assert st(dt=5) == DTYPE                     # the static-workspace variant: the product's checks
    assert st(K=48, lda=32, ldb=32) == SHAPE
    assert st(qb=None) == NULL
    assert st(out=X + 2) == ALIGN
    assert st(M=0, qa=None, sa=None, qb=None, sb=None, out=None) == OK
    n = ctypes.c_int64(-1)
    assert L.kq_mx_gemm_workspace_size(8, 8, 128, None) == NULL
    assert L.kq_mx_gemm_workspace_size(8, 8, 48, ctypes.byref(n)) == SHAPE
    assert L.kq_mx_gemm_workspace_size(-1, 8, 128, ctypes.byref(n)) == SHAPE
    assert L.kq_mx_gemm_workspace_size(0, 8, 128, ctypes.byref(n)) == OK and n.value == 0


def test_expand_validation(L):
    assert L.kq_expand_factors(T, 4, 0, Y, None) == FORMAT  # params need no expansion
    assert L.kq_expand_factors(T, 4, 7, Y, None) == FORMAT
    assert L.kq_expand_factors(T, -1, 1, Y, None) == SHAPE
    assert L.kq_expand_factors(None, 4, 1, Y, None) == NULL
    assert L.kq_expand_factors(T, 4, 1, None, None) == NULL
    assert L.kq_expand_factors(T + 1, 4, 1, Y, None) == ALIGN
    assert L.kq_expand_factors(T, 4, 3, Y + 4, None) == ALIGN  # 2x2 factors: 16-byte rows
    assert L.kq_expand_factors(None, 4, 3, Y, None) == NULL
    assert L.kq_expand_factors(None, 0, 2, None, None) == OK


def test_status_strings(L):
    for st in range(-8, 1):
        assert L.kq_status_string(st)
    assert L.kq_status_string(-100) == b"unknown status"
    assert L.kq_last_hip_error() == 0


def test_binding_rejects_unknown_dtype():
    torch = pytest.importorskip("torch")
    import online_activation_quantizer_amd as kq
    with pytest.raises(kq.KQError):
        kq.kq_quantize(torch.zeros((2, 32), dtype=torch.float64), torch.zeros(15))


def test_mx_gemm_binding_checks_operand_shapes():
    torch = pytest.importorskip("torch")
    import online_activation_quantizer_amd as kq
    qa, sa = torch.zeros((4, 64), dtype=torch.uint8), torch.zeros((4, 4), dtype=torch.uint8)
    qb, sb = torch.zeros((3, 48), dtype=torch.uint8), torch.zeros((3, 3), dtype=torch.uint8)
    with pytest.raises(kq.KQError):
        kq.kq_mx_gemm(qa, sa, qb, sb)       # K differs between the operands
    with pytest.raises(kq.KQError):
        kq.kq_mx_gemm(qa, sa[:, :3], qa, sa)  # scales do not cover K
