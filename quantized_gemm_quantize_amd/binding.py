"""Python binding of libw8a8.so (C ABI in include/w8a8.h): marshalling only.

Each function checks tensor dtypes, shapes and devices, allocates missing
outputs with torch.empty on the input's device, and passes raw device
pointers plus the current HIP stream to the library function of the same
name. All arithmetic runs in the library's kernels; there is no fallback. If
libw8a8.so is absent, every entry point raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8a8.so")

W8A8_OK = 0
W8A8_ERR_NULL = -1
W8A8_ERR_SHAPE = -2
W8A8_ERR_ALIGN = -3
W8A8_ERR_K_OVERFLOW = -4
W8A8_ERR_BLOCKSIZE = -5
W8A8_ERR_DTYPE = -6
W8A8_ERR_HIP = -7
W8A8_ERR_VALUE = -8
W8A8_OUT_BF16 = 0
W8A8_OUT_I32 = 1
W8A8_MAX_K = 131056
W8A8_FUSED_MAX_M = 64

_lib = None


class W8A8Error(RuntimeError):
    def __init__(self, status: int, fn: str):
        lib = load()
        msg = lib.w8a8_status_string(status).decode()
        if status == W8A8_ERR_HIP:
            msg += f" (hipError_t {lib.w8a8_last_hip_error()})"
        super().__init__(f"{fn}: status {status}: {msg}")
        self.status = status


def load():
    """Load libw8a8.so and declare its C signatures (raises if not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() first")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    lib.w8a8_quantize_rows.argtypes = [p, i64, i64, p, p, p]
    lib.w8a8_quantize_rows_f32.argtypes = [p, i64, i64, p, p, p]
    lib.w8a8_gemm.argtypes = [p, p, i64, p, p, i64, i64, p, i32, p]
    lib.w8a8_bsr_gemm.argtypes = [p, p, i64, i64, p, p, p, i64, i64, p, i64, p, i32, p]
    f32 = ctypes.c_float
    lib.w8a8_gemm_addmm.argtypes = [p, p, i64, p, p, i64, i64, p, f32, f32, p, p]
    lib.w8a8_bsr_gemm_addmm.argtypes = [p, p, i64, i64, p, p, p, i64, i64, p, i64, p, f32, f32,
                                        p, p]
    lib.w8a8_fused_linear.argtypes = [p, i64, i64, p, p, i64, p, f32, f32, p, p]
    lib.w8a8_compress24.argtypes = [p, i64, i64, p, p, p]
    lib.w8a8_sparse24_gemm.argtypes = [p, p, i64, p, p, p, i64, i64, p, i32, p]
    lib.w4a16_dequant.argtypes = [p, p, p, i64, i64, i64, i32, i32, p, p]
    lib.w4a16_gemm.argtypes = [p, i64, p, p, p, i64, i64, i64, i32, i32, p, p]
    for fn in ("w8a8_quantize_rows", "w8a8_quantize_rows_f32", "w8a8_gemm", "w8a8_gemm_addmm",
               "w8a8_fused_linear", "w8a8_bsr_gemm", "w8a8_bsr_gemm_addmm", "w8a8_compress24",
               "w8a8_sparse24_gemm",
               "w4a16_dequant", "w4a16_gemm"):
        getattr(lib, fn).restype = i32
    lib.w8a8_status_string.argtypes = [i32]
    lib.w8a8_status_string.restype = ctypes.c_char_p
    lib.w8a8_last_hip_error.argtypes = []
    lib.w8a8_last_hip_error.restype = i32
    _lib = lib
    return lib


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check_tensor(t: torch.Tensor, name: str, dtype, ndim: int):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _default_beta(bias, beta):
    """beta of an addmm call: as given, else 1 with a bias and 0 without (the C ABI
    rejects a nonzero beta without a bias)."""
    if beta is None:
        return 1.0 if bias is not None else 0.0
    return beta


def _call(fn: str, *args):
    st = getattr(load(), fn)(*args)
    if st != W8A8_OK:
        raise W8A8Error(st, fn)


def _quantize(fn, x, xq, x_scale, stream, dtype):
    _check_tensor(x, "x", dtype, 2)
    M, K = x.shape
    if xq is None:
        xq = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    if tuple(xq.shape) != (M, K) or tuple(x_scale.shape) != (M,):
        raise ValueError("output shapes")
    _call(fn, x.data_ptr(), M, K, xq.data_ptr(), x_scale.data_ptr(), _stream_handle(stream))
    return xq, x_scale


def w8a8_quantize_rows(x, xq=None, x_scale=None, stream=None):
    """bf16 [M,K] -> (int8 [M,K], fp32 [M]) per-row absmax/127 quantization."""
    return _quantize("w8a8_quantize_rows", x, xq, x_scale, stream, torch.bfloat16)


def w8a8_quantize_rows_f32(x, xq=None, x_scale=None, stream=None):
    """fp32 [M,K] -> (int8 [M,K], fp32 [M]); per-output-channel weight preparation."""
    return _quantize("w8a8_quantize_rows_f32", x, xq, x_scale, stream, torch.float32)


def _out(out, M, N, out_dtype, device):
    tdtype = torch.bfloat16 if out_dtype == W8A8_OUT_BF16 else torch.int32
    if out is None:
        out = torch.empty((M, N), dtype=tdtype, device=device)
    _check_tensor(out, "out", tdtype, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape")
    return out


def _out_dtype(out_dtype) -> int:
    if out_dtype in ("bf16", torch.bfloat16, W8A8_OUT_BF16):
        return W8A8_OUT_BF16
    if out_dtype in ("i32", torch.int32, W8A8_OUT_I32):
        return W8A8_OUT_I32
    raise ValueError(f"out_dtype {out_dtype!r}")


def w8a8_gemm(xq, x_scale, wq, w_scale, out=None, out_dtype="bf16", stream=None):
    """out [M,N] = bf16(sum_k xq[m,k] wq[n,k] * x_scale[m] * w_scale[n]) (or int32 acc)."""
    od = _out_dtype(out_dtype)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    _check_tensor(wq, "wq", torch.int8, 2)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K or tuple(x_scale.shape) != (M,) or tuple(w_scale.shape) != (N,):
        raise ValueError("operand shapes")
    out = _out(out, M, N, od, xq.device)
    _call("w8a8_gemm", xq.data_ptr(), x_scale.data_ptr(), M, wq.data_ptr(), w_scale.data_ptr(),
          N, K, out.data_ptr(), od, _stream_handle(stream))
    return out


def w8a8_gemm_addmm(xq, x_scale, wq, w_scale, bias=None, alpha=1.0, beta=None, out=None,
                    stream=None):
    """out [M,N] = bf16(alpha * (sum_k xq[m,k] wq[n,k] * x_scale[m] * w_scale[n]) + beta * bias[n]);
    bias None means no bias term; beta defaults to 1 with a bias and 0 without."""
    beta = _default_beta(bias, beta)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    _check_tensor(wq, "wq", torch.int8, 2)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    N, K2 = wq.shape
    if K2 != K or tuple(x_scale.shape) != (M,) or tuple(w_scale.shape) != (N,):
        raise ValueError("operand shapes")
    if bias is not None:
        _check_tensor(bias, "bias", torch.float32, 1)
        if tuple(bias.shape) != (N,):
            raise ValueError("bias shape")
    out = _out(out, M, N, _out_dtype("bf16"), xq.device)
    _call("w8a8_gemm_addmm", xq.data_ptr(), x_scale.data_ptr(), M, wq.data_ptr(),
          w_scale.data_ptr(), N, K, None if bias is None else bias.data_ptr(), float(alpha),
          float(beta), out.data_ptr(), _stream_handle(stream))
    return out


def w8a8_compress24(wq, values=None, meta=None, stream=None):
    """int8 [N,K] weight -> (values int8 [K/128,N,64], meta int32 [K/128,N,4] holding the
    uint32 index words): the 2:4 storage of include/w8a8.h (two largest |w| per group of 4)."""
    _check_tensor(wq, "wq", torch.int8, 2)
    N, K = wq.shape
    if values is None:
        values = torch.empty((K // 128, N, 64), dtype=torch.int8, device=wq.device)
    if meta is None:
        meta = torch.empty((K // 128, N, 4), dtype=torch.int32, device=wq.device)
    _check_tensor(values, "values", torch.int8, 3)
    _check_tensor(meta, "meta", torch.int32, 3)
    if tuple(values.shape) != (K // 128, N, 64) or tuple(meta.shape) != (K // 128, N, 4):
        raise ValueError("2:4 array shapes")
    _call("w8a8_compress24", wq.data_ptr(), N, K, values.data_ptr(), meta.data_ptr(),
          _stream_handle(stream))
    return values, meta


def w8a8_sparse24_gemm(xq, x_scale, values, meta, w_scale, out=None, out_dtype="bf16",
                       stream=None):
    """W8A8 GEMM on a compressed 2:4 weight (values [K/128,N,64] int8, meta [K/128,N,4] int32)."""
    od = _out_dtype(out_dtype)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    _check_tensor(values, "values", torch.int8, 3)
    _check_tensor(meta, "meta", torch.int32, 3)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    N = w_scale.shape[0]
    if (tuple(values.shape) != (K // 128, N, 64) or tuple(meta.shape) != (K // 128, N, 4)
            or tuple(x_scale.shape) != (M,)):
        raise ValueError("operand shapes")
    out = _out(out, M, N, od, xq.device)
    _call("w8a8_sparse24_gemm", xq.data_ptr(), x_scale.data_ptr(), M, values.data_ptr(),
          meta.data_ptr(), w_scale.data_ptr(), N, K, out.data_ptr(), od, _stream_handle(stream))
    return out


def _w4a16_operands(wq4, scales, zeros):
    """Shapes and the 16-bit format (from the scales: bfloat16 or float16) of a W4A16 weight."""
    _check_tensor(wq4, "wq4", torch.uint8, 2)
    dt = scales.dtype if isinstance(scales, torch.Tensor) else None
    if dt not in (torch.bfloat16, torch.float16):
        raise TypeError("scales must be a bfloat16 or float16 tensor")
    _check_tensor(scales, "scales", dt, 2)
    _check_tensor(zeros, "zeros", dt, 2)
    N, K2 = wq4.shape
    K = 2 * K2
    if scales.shape != zeros.shape or scales.shape[0] != N or scales.shape[1] == 0 \
            or K % scales.shape[1]:
        raise ValueError("W4A16 operand shapes")
    return N, K, K // scales.shape[1], dt


W4A16_BF16, W4A16_F16 = 0, 1


def _w4a16_dtype(dt) -> int:
    return W4A16_F16 if dt == torch.float16 else W4A16_BF16


W4A16_CODES_U4, W4A16_CODES_S4 = 0, 1


def w4a16_dequant(wq4, scales, zeros, signed=False, out=None, stream=None):
    """Packed 4-bit codes [N,K/2] + scales/zeros [N,K/G] (bfloat16 or float16) -> w [N,K] of
    that type = round(round(q - z) * s); q the code (u4) or, with signed, its 4-bit two's
    complement (s4)."""
    N, K, G, dt = _w4a16_operands(wq4, scales, zeros)
    if out is None:
        out = torch.empty((N, K), dtype=dt, device=wq4.device)
    _check_tensor(out, "out", dt, 2)
    if tuple(out.shape) != (N, K):
        raise ValueError("out shape")
    _call("w4a16_dequant", wq4.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N, K, G,
          W4A16_CODES_S4 if signed else W4A16_CODES_U4, _w4a16_dtype(dt), out.data_ptr(),
          _stream_handle(stream))
    return out


def w4a16_gemm(x, wq4, scales, zeros, signed=False, out=None, stream=None):
    """out [M,N] = x [M,K] times the dequantized 4-bit weights (u4, or s4 with signed), fused;
    x, scales, zeros and out all bfloat16 or all float16."""
    N, K, G, dt = _w4a16_operands(wq4, scales, zeros)
    _check_tensor(x, "x", dt, 2)
    M = x.shape[0]
    if x.shape[1] != K:
        raise ValueError("operand shapes")
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=x.device)
    _check_tensor(out, "out", dt, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape")
    _call("w4a16_gemm", x.data_ptr(), M, wq4.data_ptr(), scales.data_ptr(), zeros.data_ptr(), N,
          K, G, W4A16_CODES_S4 if signed else W4A16_CODES_U4, _w4a16_dtype(dt), out.data_ptr(),
          _stream_handle(stream))
    return out


def w8a8_bsr_gemm(xq, x_scale, crow, col, values, w_scale, out=None, out_dtype="bf16",
                  stream=None):
    """Block-sparse W8A8 GEMM; crow [N/64+1], col [nnzb], values [nnzb,64,64] int8."""
    od = _out_dtype(out_dtype)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    _check_tensor(crow, "crow", torch.int32, 1)
    _check_tensor(col, "col", torch.int32, 1)
    _check_tensor(values, "values", torch.int8, 3)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    nnzb, bs, bs2 = values.shape
    N = w_scale.shape[0]
    if bs != bs2 or col.shape[0] != nnzb or crow.shape[0] != N // max(bs, 1) + 1:
        raise ValueError("BSR array shapes")
    out = _out(out, M, N, od, xq.device)
    _call("w8a8_bsr_gemm", xq.data_ptr(), x_scale.data_ptr(), M, K, crow.data_ptr(),
          col.data_ptr() if nnzb else 0, values.data_ptr() if nnzb else 0, nnzb, bs,
          w_scale.data_ptr(), N, out.data_ptr(), od, _stream_handle(stream))
    return out


def w8a8_bsr_gemm_addmm(xq, x_scale, crow, col, values, w_scale, bias=None, alpha=1.0, beta=None,
                        out=None, stream=None):
    """Block-sparse W8A8 GEMM with the addmm epilogue (bf16 out):
    out = bf16(alpha * (acc * x_scale[m] * w_scale[n]) + beta * bias[n]); bias None
    means no bias term; beta defaults to 1 with a bias and 0 without."""
    beta = _default_beta(bias, beta)
    _check_tensor(xq, "xq", torch.int8, 2)
    _check_tensor(x_scale, "x_scale", torch.float32, 1)
    _check_tensor(crow, "crow", torch.int32, 1)
    _check_tensor(col, "col", torch.int32, 1)
    _check_tensor(values, "values", torch.int8, 3)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = xq.shape
    nnzb, bs, bs2 = values.shape
    N = w_scale.shape[0]
    if bs != bs2 or col.shape[0] != nnzb or crow.shape[0] != N // max(bs, 1) + 1:
        raise ValueError("BSR array shapes")
    if bias is not None:
        _check_tensor(bias, "bias", torch.float32, 1)
        if tuple(bias.shape) != (N,):
            raise ValueError("bias shape")
    out = _out(out, M, N, _out_dtype("bf16"), xq.device)
    _call("w8a8_bsr_gemm_addmm", xq.data_ptr(), x_scale.data_ptr(), M, K, crow.data_ptr(),
          col.data_ptr() if nnzb else 0, values.data_ptr() if nnzb else 0, nnzb, bs,
          w_scale.data_ptr(), N, None if bias is None else bias.data_ptr(), float(alpha),
          float(beta), out.data_ptr(), _stream_handle(stream))
    return out


def w8a8_fused_linear(x, wq, w_scale, bias=None, alpha=1.0, beta=None, out=None, stream=None):
    """Single-launch quantize + GEMM for x [M,K] bf16 with M <= 64:
    out = bf16(alpha * (acc * s[m] * w_scale[n]) + beta * bias[n]), q and s as
    w8a8_quantize_rows computes them; bias None means no bias term; beta
    defaults to 1 with a bias and 0 without."""
    beta = _default_beta(bias, beta)
    _check_tensor(x, "x", torch.bfloat16, 2)
    _check_tensor(wq, "wq", torch.int8, 2)
    _check_tensor(w_scale, "w_scale", torch.float32, 1)
    M, K = x.shape
    N, K2 = wq.shape
    if K2 != K or tuple(w_scale.shape) != (N,):
        raise ValueError("operand shapes")
    if bias is not None:
        _check_tensor(bias, "bias", torch.float32, 1)
        if tuple(bias.shape) != (N,):
            raise ValueError("bias shape")
    out = _out(out, M, N, _out_dtype("bf16"), x.device)
    _call("w8a8_fused_linear", x.data_ptr(), M, K, wq.data_ptr(), w_scale.data_ptr(), N,
          None if bias is None else bias.data_ptr(), float(alpha), float(beta), out.data_ptr(),
          _stream_handle(stream))
    return out


def w8a8_linear(x, wq, w_scale, out=None, stream=None):
    """Dynamically quantized linear layer: quantize_rows(x), then the fused-dequant GEMM.
    (Two launches are faster than w8a8_fused_linear at every M it takes: each of its
    N/16 workgroups quantizes all of x.)"""
    xq, xs = w8a8_quantize_rows(x, stream=stream)
    return w8a8_gemm(xq, xs, wq, w_scale, out=out, stream=stream)
