"""ctypes front end of the C oracle (w8a8_oracle.c) -- test infrastructure only.

Arrays are numpy: bf16 values travel as their uint16 bit patterns. Every
function here only marshals arguments; the arithmetic is in the C file, whose
header states the passages each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "w8a8_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

# IEEE semantics are part of the definition: no contraction, no fast-math.
CFLAGS = ["-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
          "-Wall", "-Wextra", "-Werror"]


def build_oracle() -> str:
    """Compile the oracle with gcc into oracle/liboracle.so (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


# A sanitizer build (AddressSanitizer + UndefinedBehaviorSanitizer) of the same
# source, for the CPU tests that run the pins under it.
SAN_CFLAGS = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
              "-fno-omit-frame-pointer", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
              "-fPIC", "-shared", "-Wall", "-Wextra", "-Werror"]


def build_oracle_sanitized(path: str) -> str:
    """Compile the oracle with AddressSanitizer and UndefinedBehaviorSanitizer into `path`
    (loaded in place of liboracle.so when W8A8_ORACLE_LIB names it, with gcc's sanitizer
    runtimes preloaded)."""
    subprocess.run(["gcc", *SAN_CFLAGS, "-o", path, _SRC, "-lm"], check=True)
    return path


def load_oracle():
    """Load liboracle.so (or the library W8A8_ORACLE_LIB names), building liboracle.so
    first only if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = os.environ.get("W8A8_ORACLE_LIB", _LIB)
    if path == _LIB and not os.path.exists(_LIB):
        build_oracle()
    lib = ctypes.CDLL(path)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_quantize_rows_bf16.argtypes = [p, i64, i64, p, p]
    lib.oracle_quantize_rows_bf16.restype = None
    lib.oracle_quantize_rows_f32.argtypes = [p, i64, i64, p, p]
    lib.oracle_quantize_rows_f32.restype = None
    lib.oracle_gemm_i32.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_gemm_i32.restype = ctypes.c_int
    lib.oracle_bf16_rne_from_f64.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne_from_f64.restype = ctypes.c_uint16
    lib.oracle_epilogue_bf16.argtypes = [p, p, p, i64, i64, p]
    lib.oracle_epilogue_bf16.restype = None
    lib.oracle_epilogue_addmm_bf16.argtypes = [p, p, p, p, ctypes.c_double, ctypes.c_double, i64,
                                                i64, p]
    lib.oracle_epilogue_addmm_bf16.restype = None
    lib.oracle_bsr_gemm_i32.argtypes = [p, i64, i64, p, p, p, i64, i64, p]
    lib.oracle_bsr_gemm_i32.restype = ctypes.c_int
    lib.oracle_compress24.argtypes = [p, i64, i64, p, p]
    lib.oracle_compress24.restype = None
    lib.oracle_decompress24.argtypes = [p, p, i64, i64, p]
    lib.oracle_decompress24.restype = ctypes.c_int
    lib.oracle_w4a16_dequant.argtypes = [p, p, p, i64, i64, i64, ctypes.c_int, ctypes.c_int, p]
    lib.oracle_w4a16_dequant.restype = None
    lib.oracle_bf16_gemm.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_f16_gemm.argtypes = [p, p, i64, i64, i64, p]
    lib.oracle_f16_gemm.restype = None
    lib.oracle_f16_rne_from_f64.argtypes = [ctypes.c_double]
    lib.oracle_f16_rne_from_f64.restype = ctypes.c_uint16
    lib.oracle_bf16_gemm.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.dtype(dtype):
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def quantize_rows_bf16(x_bits: np.ndarray):
    """X bf16 [M,K] (uint16 bit patterns) -> (q int8 [M,K], s float32 [M])."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    load_oracle().oracle_quantize_rows_bf16(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def quantize_rows_f32(x: np.ndarray):
    """W fp32 [N,K] -> (q int8 [N,K], s float32 [N]), one scale per row."""
    x = _c(x, np.float32)
    M, K = x.shape
    q = np.empty((M, K), np.int8)
    s = np.empty((M,), np.float32)
    load_oracle().oracle_quantize_rows_f32(_ptr(x), M, K, _ptr(q), _ptr(s))
    return q, s


def gemm_i32(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc int32 [M,N] = xq [M,K] . wq [N,K]^T, exact; raises if it leaves int32."""
    xq = _c(xq, np.int8)
    wq = _c(wq, np.int8)
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError("K mismatch")
    acc = np.empty((M, N), np.int32)
    rc = load_oracle().oracle_gemm_i32(_ptr(xq), _ptr(wq), M, N, K, _ptr(acc))
    if rc != 0:
        raise OverflowError("int8 dot product leaves the int32 range")
    return acc


def bf16_rne_from_f64(v: float) -> int:
    """Bit pattern of the bf16 nearest to v (ties to even)."""
    return int(load_oracle().oracle_bf16_rne_from_f64(float(v)))


def epilogue_bf16(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """out bf16 bits [M,N] = bf16_rne(acc * sx[m] * sw[n]) evaluated in float64."""
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, N = acc.shape
    if sx.shape != (M,) or sw.shape != (N,):
        raise ValueError("scale shapes")
    out = np.empty((M, N), np.uint16)
    load_oracle().oracle_epilogue_bf16(_ptr(acc), _ptr(sx), _ptr(sw), M, N, _ptr(out))
    return out


def epilogue_addmm_bf16(acc: np.ndarray, sx: np.ndarray, sw: np.ndarray, bias, alpha: float,
                        beta: float) -> np.ndarray:
    """out bf16 bits [M,N] = bf16_rne(alpha * acc * sx[m] * sw[n] + beta * bias[n]), float64;
    bias None means no bias term."""
    acc = _c(acc, np.int32)
    sx = _c(sx, np.float32)
    sw = _c(sw, np.float32)
    M, N = acc.shape
    if sx.shape != (M,) or sw.shape != (N,):
        raise ValueError("scale shapes")
    b = None if bias is None else _c(bias, np.float32)
    if b is not None and b.shape != (N,):
        raise ValueError("bias shape")
    out = np.empty((M, N), np.uint16)
    load_oracle().oracle_epilogue_addmm_bf16(_ptr(acc), _ptr(sx), _ptr(sw),
                                             None if b is None else _ptr(b), float(alpha),
                                             float(beta), M, N, _ptr(out))
    return out


def bsr_gemm_i32(xq: np.ndarray, crow: np.ndarray, col: np.ndarray, values: np.ndarray,
                 N: int) -> np.ndarray:
    """acc int32 [M,N] over the stored blocks of a BSR weight (values [nnzb,bs,bs])."""
    xq = _c(xq, np.int8)
    crow = _c(crow, np.int32)
    col = _c(col, np.int32)
    values = _c(values, np.int8)
    M, K = xq.shape
    bs = values.shape[1] if values.ndim == 3 else 64
    if values.ndim != 3 or values.shape[2] != bs or N % bs or K % bs:
        raise ValueError("BSR shapes")
    if crow.shape != (N // bs + 1,) or col.shape[0] != values.shape[0]:
        raise ValueError("BSR index shapes")
    acc = np.empty((M, N), np.int32)
    rc = load_oracle().oracle_bsr_gemm_i32(_ptr(xq), M, K, _ptr(crow), _ptr(col),
                                           _ptr(values), bs, N, _ptr(acc))
    if rc != 0:
        raise OverflowError("int8 dot product leaves the int32 range")
    return acc


def compress24(w: np.ndarray):
    """int8 [N,K] (K % 128 == 0) -> (values int8 [K/128,N,64], meta uint32 [K/128,N,4]): the
    two largest magnitudes of each group of 4 along K, in the library's storage order."""
    w = _c(w, np.int8)
    N, K = w.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    values = np.empty((K // 128, N, 64), np.int8)
    meta = np.empty((K // 128, N, 4), np.uint32)
    load_oracle().oracle_compress24(_ptr(w), N, K, _ptr(values), _ptr(meta))
    return values, meta


def decompress24(values: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """The dense int8 [N,K] weight that compressed 2:4 arrays hold."""
    values = _c(values, np.int8)
    meta = _c(meta, np.uint32)
    KB, N, width = values.shape
    K = 128 * KB
    if width != 64 or meta.shape != (KB, N, 4):
        raise ValueError("2:4 array shapes")
    w = np.empty((N, K), np.int8)
    if load_oracle().oracle_decompress24(_ptr(values), _ptr(meta), N, K, _ptr(w)) != 0:
        raise ValueError("a group's positions are not p0 < p1")
    return w


def w4a16_dequant(wq4: np.ndarray, scales: np.ndarray, zeros: np.ndarray,
                  signed: bool = False, half: bool = False) -> np.ndarray:
    """Packed 4-bit codes [N,K/2] + bf16 scales/zeros [N,K/G] (bit patterns) -> bf16 w [N,K]
    (bits): w = bf16(bf16(q - z) * s), q the nibble (u4, 0..15) or its 4-bit two's
    complement (s4, -8..7); with half, IEEE binary16 in place of bf16 throughout."""
    wq4 = _c(wq4, np.uint8)
    scales = _c(scales, np.uint16)
    zeros = _c(zeros, np.uint16)
    N, K2 = wq4.shape
    K = 2 * K2
    if scales.shape != zeros.shape or scales.shape[0] != N or K % scales.shape[1]:
        raise ValueError("W4A16 shapes")
    G = K // scales.shape[1]
    w = np.empty((N, K), np.uint16)
    load_oracle().oracle_w4a16_dequant(_ptr(wq4), _ptr(scales), _ptr(zeros), N, K, G,
                                       1 if signed else 0, 1 if half else 0, _ptr(w))
    return w


def bf16_gemm(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """bf16 x [M,K] times bf16 w [N,K]^T, summed in float64, rounded once to bf16 (bits)."""
    x_bits = _c(x_bits, np.uint16)
    w_bits = _c(w_bits, np.uint16)
    M, K = x_bits.shape
    N, K2 = w_bits.shape
    if K2 != K:
        raise ValueError("inner dimensions")
    out = np.empty((M, N), np.uint16)
    load_oracle().oracle_bf16_gemm(_ptr(x_bits), _ptr(w_bits), M, N, K, _ptr(out))
    return out


def f16_gemm(x_bits: np.ndarray, w_bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 x [M,K] times binary16 w [N,K]^T, summed in float64, rounded once to
    binary16 (bits)."""
    x_bits = _c(x_bits, np.uint16)
    w_bits = _c(w_bits, np.uint16)
    M, K = x_bits.shape
    N, K2 = w_bits.shape
    if K2 != K:
        raise ValueError("inner dimensions")
    out = np.empty((M, N), np.uint16)
    load_oracle().oracle_f16_gemm(_ptr(x_bits), _ptr(w_bits), M, N, K, _ptr(out))
    return out


def f16_rne_from_f64(v: float) -> int:
    """Bit pattern of the IEEE binary16 nearest to v (ties to even, overflow to infinity)."""
    return int(load_oracle().oracle_f16_rne_from_f64(float(v)))


def num_threads() -> int:
    return int(load_oracle().oracle_num_threads())
