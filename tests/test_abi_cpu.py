"""The C ABI without a GPU: the library loads, exports every declared symbol,
and rejects every invalid argument with its documented status before any HIP
call (so these calls never touch a device). Pointer arguments here are plain
integers that are never dereferenced.
"""
import os
import re

import pytest

from quantized_gemm_quantize_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")

OK, NULL, SHAPE, ALIGN, KOVF, BLK, DTYPE, VALUE = 0, -1, -2, -3, -4, -5, -6, -8
P = 0x10000  # an aligned, never-dereferenced stand-in for a device pointer


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libw8a8.so not built")
    return binding.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w ]+?\*?\s*\b((?:w8a8|w4a16)_\w+)\s*\(", text,
                                 re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for fn in ("w8a8_quantize_rows", "w8a8_quantize_rows_f32", "w8a8_gemm", "w8a8_gemm_addmm",
               "w8a8_fused_linear", "w8a8_bsr_gemm", "w8a8_bsr_gemm_addmm", "w8a8_compress24",
               "w8a8_sparse24_gemm", "w4a16_dequant", "w4a16_gemm", "w8a8_status_string",
               "w8a8_last_hip_error"):
        assert fn in names


def test_library_exports_every_declared_symbol(lib):
    for fn in declared_functions():
        assert hasattr(lib, fn), fn


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert f"#define W8A8_MAX_K {binding.W8A8_MAX_K}" in text
    assert f"#define W8A8_FUSED_MAX_M {binding.W8A8_FUSED_MAX_M}" in text
    assert re.search(rf"W4A16_CODES_U4\s*=\s*{binding.W4A16_CODES_U4}\b", text)
    assert re.search(rf"W4A16_CODES_S4\s*=\s*{binding.W4A16_CODES_S4}\b", text)
    assert re.search(rf"W4A16_BF16\s*=\s*{binding.W4A16_BF16}\b", text)
    assert re.search(rf"W4A16_F16\s*=\s*{binding.W4A16_F16}\b", text)
    assert 128 * 128 * binding.W8A8_MAX_K < 2 ** 31
    assert 128 * 128 * (binding.W8A8_MAX_K + 16) >= 2 ** 31
    for name in ("W8A8_ERR_NULL", "W8A8_ERR_SHAPE", "W8A8_ERR_ALIGN", "W8A8_ERR_K_OVERFLOW",
                 "W8A8_ERR_BLOCKSIZE", "W8A8_ERR_DTYPE", "W8A8_ERR_HIP", "W8A8_ERR_VALUE"):
        m = re.search(rf"{name}\s*=\s*(-?\d+)", text)
        assert int(m.group(1)) == getattr(binding, name)


def test_status_strings(lib):
    for st in (OK, NULL, SHAPE, ALIGN, KOVF, BLK, DTYPE, -7, VALUE, 99):
        assert lib.w8a8_status_string(st)
    assert lib.w8a8_last_hip_error() == 0


@pytest.mark.parametrize("fn", ["w8a8_quantize_rows", "w8a8_quantize_rows_f32"])
def test_quantize_validation(lib, fn):
    f = getattr(lib, fn)
    assert f(P, -1, 64, P, P, None) == SHAPE
    assert f(P, 4, 0, P, P, None) == SHAPE
    assert f(P, 4, 24, P, P, None) == SHAPE          # K % 16
    assert f(P, 4, 133152, P, P, None) == KOVF
    assert f(P, 2 ** 31, 64, P, P, None) == SHAPE     # more rows than workgroups can be launched
    assert f(0, 4, 64, P, P, None) == NULL
    assert f(P, 4, 64, 0, P, None) == NULL
    assert f(P, 4, 64, P, 0, None) == NULL
    assert f(P + 8, 4, 64, P, P, None) == ALIGN
    assert f(P, 4, 64, P + 4, P, None) == ALIGN
    assert f(P, 0, 64, 0, 0, None) == OK                # empty: no launch


def test_gemm_validation(lib):
    g = lib.w8a8_gemm
    args = lambda **kw: [kw.get("xq", P), kw.get("xs", P), kw.get("M", 32), kw.get("wq", P),
                         kw.get("ws", P), kw.get("N", 64), kw.get("K", 64), kw.get("out", P),
                         kw.get("od", 0), None]
    assert g(*args(M=-1)) == SHAPE
    assert g(*args(N=0)) == SHAPE
    assert g(*args(N=40)) == SHAPE                      # N % 16
    assert g(*args(K=0)) == SHAPE
    assert g(*args(K=72)) == SHAPE                      # K % 16
    assert g(*args(K=133152)) == KOVF
    assert g(*args(od=2)) == DTYPE
    assert g(*args(od=-1)) == DTYPE
    for k in ("xq", "xs", "wq", "ws", "out"):
        assert g(*args(**{k: 0})) == NULL, k
        assert g(*args(**{k: P + 4})) == ALIGN, k
    assert g(*args(M=0, xq=0, xs=0, out=0)) == OK       # empty: no launch


def test_gemm_addmm_validation(lib):
    g = lib.w8a8_gemm_addmm
    args = lambda **kw: [kw.get("xq", P), kw.get("xs", P), kw.get("M", 32), kw.get("wq", P),
                         kw.get("ws", P), kw.get("N", 64), kw.get("K", 64), kw.get("bias", P),
                         kw.get("alpha", 1.0), kw.get("beta", 1.0), kw.get("out", P), None]
    assert g(*args(M=-1)) == SHAPE
    assert g(*args(N=40)) == SHAPE
    assert g(*args(K=72)) == SHAPE
    assert g(*args(K=133152)) == KOVF
    assert g(*args(alpha=float("inf"))) == VALUE
    assert g(*args(beta=float("nan"))) == VALUE
    for k in ("xq", "xs", "wq", "ws", "out", "bias"):
        assert g(*args(**{k: 0})) == NULL, k
        assert g(*args(**{k: P + 4})) == ALIGN, k
    assert g(*args(bias=0, beta=0.0, M=0)) == OK        # no bias term, empty: no launch
    assert g(*args(M=0, xq=0, xs=0, out=0)) == OK


def test_fused_linear_validation(lib):
    f = lib.w8a8_fused_linear
    args = lambda **kw: [kw.get("x", P), kw.get("M", 16), kw.get("K", 64), kw.get("wq", P),
                         kw.get("ws", P), kw.get("N", 64), kw.get("bias", P),
                         kw.get("alpha", 1.0), kw.get("beta", 1.0), kw.get("out", P), None]
    assert f(*args(M=-1)) == SHAPE
    assert f(*args(M=65)) == SHAPE                      # above W8A8_FUSED_MAX_M
    assert f(*args(N=40)) == SHAPE
    assert f(*args(N=0)) == SHAPE
    assert f(*args(K=72)) == SHAPE
    assert f(*args(K=0)) == SHAPE
    assert f(*args(K=133152)) == KOVF
    assert f(*args(alpha=float("inf"))) == VALUE
    assert f(*args(beta=float("nan"))) == VALUE
    for k in ("x", "wq", "ws", "out", "bias"):
        assert f(*args(**{k: 0})) == NULL, k
        assert f(*args(**{k: P + 2})) == ALIGN, k
    assert f(*args(bias=0, beta=0.0, M=0)) == OK        # no bias term, empty: no launch
    assert f(*args(M=0, x=0, out=0)) == OK


def test_compress24_validation(lib):
    c = lib.w8a8_compress24
    args = lambda **kw: [kw.get("wq", P), kw.get("N", 32), kw.get("K", 128), kw.get("vals", P),
                         kw.get("meta", P), None]
    assert c(*args(N=-1)) == SHAPE
    assert c(*args(K=0)) == SHAPE
    assert c(*args(K=192)) == SHAPE                      # K % 128
    for k in ("wq", "vals", "meta"):
        assert c(*args(**{k: 0})) == NULL, k
        assert c(*args(**{k: P + 4})) == ALIGN, k
    assert c(*args(N=0, wq=0, vals=0, meta=0)) == OK


def test_sparse24_gemm_validation(lib):
    g = lib.w8a8_sparse24_gemm
    args = lambda **kw: [kw.get("xq", P), kw.get("xs", P), kw.get("M", 16), kw.get("vals", P),
                         kw.get("meta", P), kw.get("ws", P), kw.get("N", 64), kw.get("K", 128),
                         kw.get("out", P), kw.get("od", 0), None]
    assert g(*args(M=-1)) == SHAPE
    assert g(*args(K=192)) == SHAPE                      # K % 128
    assert g(*args(M=300, K=192)) == SHAPE
    assert g(*args(N=40)) == SHAPE
    assert g(*args(K=0)) == SHAPE
    assert g(*args(K=133248)) == KOVF
    assert g(*args(od=2)) == DTYPE
    for k in ("xq", "xs", "vals", "meta", "ws", "out"):
        assert g(*args(**{k: 0})) == NULL, k
        assert g(*args(**{k: P + 8})) == ALIGN, k
    assert g(*args(M=0, xq=0, xs=0, out=0)) == OK


def test_w4a16_validation(lib):
    d, g = lib.w4a16_dequant, lib.w4a16_gemm
    dargs = lambda **kw: [kw.get("wq", P), kw.get("s", P), kw.get("z", P), kw.get("N", 64),
                          kw.get("K", 256), kw.get("G", 128), kw.get("codes", 0), kw.get("dt", 0),
                          kw.get("w", P), None]
    gargs = lambda **kw: [kw.get("x", P), kw.get("M", 16), kw.get("wq", P), kw.get("s", P),
                          kw.get("z", P), kw.get("N", 64), kw.get("K", 256), kw.get("G", 128),
                          kw.get("codes", 0), kw.get("dt", 0), kw.get("out", P), None]
    for f, args in ((d, dargs), (g, gargs)):
        assert f(*args(N=40)) == SHAPE                   # N % 16
        assert f(*args(N=0)) == SHAPE
        assert f(*args(K=192)) == SHAPE                  # K % 128
        assert f(*args(G=48)) == SHAPE                   # G % 32
        assert f(*args(G=96)) == SHAPE                   # K % G
        assert f(*args(G=0)) == SHAPE
        assert f(*args(wq=0)) == NULL
        assert f(*args(wq=P + 8)) == ALIGN
        assert f(*args(s=P + 1)) == ALIGN                # scales need 2-byte alignment
        assert f(*args(z=0)) == NULL
        assert f(*args(codes=2)) == DTYPE               # neither u4 nor s4
        assert f(*args(codes=-1)) == DTYPE
        assert f(*args(dt=2)) == DTYPE                  # neither bf16 nor binary16
    assert d(*dargs(w=P + 4)) == ALIGN
    assert g(*gargs(M=-1)) == SHAPE
    assert g(*gargs(x=P + 2)) == ALIGN
    assert g(*gargs(out=0)) == NULL
    assert g(*gargs(M=0, x=0, out=0)) == OK


def test_bsr_validation(lib):
    b = lib.w8a8_bsr_gemm
    args = lambda **kw: [kw.get("xq", P), kw.get("xs", P), kw.get("M", 32), kw.get("K", 128),
                         kw.get("crow", P), kw.get("col", P), kw.get("vals", P),
                         kw.get("nnzb", 2), kw.get("bs", 64), kw.get("ws", P), kw.get("N", 128),
                         kw.get("out", P), kw.get("od", 0), None]
    assert b(*args(bs=32)) == BLK
    assert b(*args(bs=128)) == BLK
    assert b(*args(N=96)) == SHAPE                      # N % 64
    assert b(*args(K=80)) == SHAPE                      # K % 64
    assert b(*args(M=-1)) == SHAPE
    assert b(*args(nnzb=-1)) == SHAPE
    assert b(*args(nnzb=5)) == SHAPE                    # more blocks than the grid holds
    assert b(*args(K=133184)) == KOVF
    assert b(*args(od=3)) == DTYPE
    for k in ("xq", "xs", "crow", "col", "vals", "ws", "out"):
        assert b(*args(**{k: 0})) == NULL, k
        assert b(*args(**{k: P + 2})) == ALIGN, k
    assert b(*args(M=0, xq=0, xs=0, out=0)) == OK


def test_bsr_addmm_validation(lib):
    b = lib.w8a8_bsr_gemm_addmm
    args = lambda **kw: [kw.get("xq", P), kw.get("xs", P), kw.get("M", 32), kw.get("K", 128),
                         kw.get("crow", P), kw.get("col", P), kw.get("vals", P),
                         kw.get("nnzb", 2), kw.get("bs", 64), kw.get("ws", P), kw.get("N", 128),
                         kw.get("bias", P), kw.get("alpha", 1.0), kw.get("beta", 1.0),
                         kw.get("out", P), None]
    assert b(*args(bs=32)) == BLK
    assert b(*args(N=96)) == SHAPE                      # N % 64
    assert b(*args(K=80)) == SHAPE                      # K % 64
    assert b(*args(M=-1)) == SHAPE
    assert b(*args(nnzb=-1)) == SHAPE
    assert b(*args(nnzb=5)) == SHAPE
    assert b(*args(K=133184)) == KOVF
    assert b(*args(alpha=float("inf"))) == VALUE
    assert b(*args(beta=float("nan"))) == VALUE
    for k in ("xq", "xs", "crow", "col", "vals", "ws", "out", "bias"):
        assert b(*args(**{k: 0})) == NULL, k
        assert b(*args(**{k: P + 2})) == ALIGN, k
    assert b(*args(bias=0, beta=0.0, M=0)) == OK        # no bias term, empty: no launch
    assert b(*args(M=0, xq=0, xs=0, out=0)) == OK
