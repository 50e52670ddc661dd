"""One small layer of every kind, run through every entry point, for the GPU tests that
compare whole runs bit for bit (streams, HIP graphs, repeated runs, the LDS-poisoned build)."""
import contextlib

import numpy as np
import torch

from quantized_gemm_quantize_amd.inputs import bsr_from_dense, make_linear, make_w4a16

DEV = "cuda:0"
M, N, K = 320, 384, 512   # tiled paths with ragged M; N, K multiples of 128
MD = 16                   # the M-small paths
KL = 4096                 # the M-small path with both operands through LDS


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def make_layer(b):
    """Inputs and preallocated outputs of one layer of every kind."""
    t = {}
    dense = make_linear(M, N, K, seed=21)
    t["x"] = _bf16(dense.x_bits)
    t["xd"] = _bf16(dense.x_bits[:MD])
    t["wq"], t["sw"] = b.w8a8_quantize_rows_f32(_dev(dense.w))
    t["bias"] = _dev((np.random.default_rng(22).standard_normal(N) * 0.5).astype(np.float32))
    long_k = make_linear(MD, N, KL, seed=26)
    t["xl"] = _bf16(long_k.x_bits)
    t["wql"], t["swl"] = b.w8a8_quantize_rows_f32(_dev(long_k.w))
    blk = make_linear(M, N, K, seed=23, bs=64, zero_frac=0.6)
    wqb, t["swb"] = b.w8a8_quantize_rows_f32(_dev(blk.w))
    crow, col, values = bsr_from_dense(wqb.cpu().numpy(), blk.block_mask, 64)
    t["crow"], t["col"], t["values"] = _dev(crow), _dev(col), _dev(values)
    sp = make_linear(M, N, K, seed=24, sparse24=True)
    wq24, t["sw24"] = b.w8a8_quantize_rows_f32(_dev(sp.w))
    t["v24"], t["m24"] = b.w8a8_compress24(wq24)
    w4 = make_w4a16(M, N, K, 128, seed=25)
    t["x4"] = _bf16(w4.x_bits)
    t["wq4"] = _dev(w4.wq4)
    t["s4"] = _bf16(w4.scales)
    t["z4"] = _bf16(w4.zeros)
    # the M-small 2:4 and W4A16 kernels that move activations through LDS (K = KL)
    spl = make_linear(MD, N, KL, seed=27, sparse24=True)
    wq24l, t["sw24l"] = b.w8a8_quantize_rows_f32(_dev(spl.w))
    t["v24l"], t["m24l"] = b.w8a8_compress24(wq24l)
    w4l = make_w4a16(MD, N, KL, 128, seed=28)
    t["x4l"] = _bf16(w4l.x_bits)
    t["wq4l"] = _dev(w4l.wq4)
    t["s4l"] = _bf16(w4l.scales)
    t["z4l"] = _bf16(w4l.zeros)
    # outputs (written by every run)
    t["xq"] = torch.empty((M, K), dtype=torch.int8, device=DEV)
    t["sx"] = torch.empty((M,), dtype=torch.float32, device=DEV)
    t["xqd"] = torch.empty((MD, K), dtype=torch.int8, device=DEV)
    t["sxd"] = torch.empty((MD,), dtype=torch.float32, device=DEV)
    t["xql"] = torch.empty((MD, KL), dtype=torch.int8, device=DEV)
    t["sxl"] = torch.empty((MD,), dtype=torch.float32, device=DEV)
    for name, rows in (("gemm", M), ("addmm", M), ("dec", MD), ("dec_addmm", MD), ("fused", MD),
                       ("decl", MD), ("decl_addmm", MD),
                       ("bsr", M), ("bsr_addmm", M), ("s24", M), ("s24d", MD), ("s24dl", MD),
                       ("w4", M), ("w4d", MD), ("w4dl", MD)):
        t["out_" + name] = torch.empty((rows, N), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    return t


OUTPUTS = ["xq", "sx", "xqd", "sxd", "xql", "sxl", "out_gemm", "out_addmm", "out_dec",
           "out_dec_addmm", "out_decl", "out_decl_addmm", "out_fused", "out_bsr", "out_bsr_addmm",
           "out_s24", "out_s24d", "out_s24dl", "out_w4", "out_w4d", "out_w4dl"]


def run_layer(b, t, stream=None):
    """Every product once, on `stream` (None: the current stream)."""
    b.w8a8_quantize_rows(t["x"], t["xq"], t["sx"], stream=stream)
    b.w8a8_quantize_rows(t["xd"], t["xqd"], t["sxd"], stream=stream)
    b.w8a8_gemm(t["xq"], t["sx"], t["wq"], t["sw"], out=t["out_gemm"], stream=stream)
    b.w8a8_gemm_addmm(t["xq"], t["sx"], t["wq"], t["sw"], bias=t["bias"], alpha=0.5, beta=2.0,
                      out=t["out_addmm"], stream=stream)
    b.w8a8_gemm(t["xqd"], t["sxd"], t["wq"], t["sw"], out=t["out_dec"], stream=stream)
    b.w8a8_gemm_addmm(t["xqd"], t["sxd"], t["wq"], t["sw"], bias=t["bias"], alpha=-1.5, beta=0.25,
                      out=t["out_dec_addmm"], stream=stream)
    b.w8a8_fused_linear(t["xd"], t["wq"], t["sw"], bias=t["bias"], alpha=1.0, beta=1.0,
                        out=t["out_fused"], stream=stream)
    b.w8a8_quantize_rows(t["xl"], t["xql"], t["sxl"], stream=stream)
    b.w8a8_gemm(t["xql"], t["sxl"], t["wql"], t["swl"], out=t["out_decl"], stream=stream)
    b.w8a8_gemm_addmm(t["xql"], t["sxl"], t["wql"], t["swl"], bias=t["bias"], alpha=0.5,
                      beta=-0.75, out=t["out_decl_addmm"], stream=stream)
    b.w8a8_bsr_gemm(t["xq"], t["sx"], t["crow"], t["col"], t["values"], t["swb"],
                    out=t["out_bsr"], stream=stream)
    b.w8a8_bsr_gemm_addmm(t["xq"], t["sx"], t["crow"], t["col"], t["values"], t["swb"],
                          bias=t["bias"], alpha=0.75, beta=-1.0, out=t["out_bsr_addmm"],
                          stream=stream)
    b.w8a8_sparse24_gemm(t["xq"], t["sx"], t["v24"], t["m24"], t["sw24"], out=t["out_s24"],
                         stream=stream)
    b.w8a8_sparse24_gemm(t["xqd"], t["sxd"], t["v24"], t["m24"], t["sw24"], out=t["out_s24d"],
                         stream=stream)
    b.w4a16_gemm(t["x4"], t["wq4"], t["s4"], t["z4"], out=t["out_w4"], stream=stream)
    b.w4a16_gemm(t["x4"][:MD], t["wq4"], t["s4"], t["z4"], out=t["out_w4d"], stream=stream)
    b.w8a8_sparse24_gemm(t["xql"], t["sxl"], t["v24l"], t["m24l"], t["sw24l"], out=t["out_s24dl"],
                         stream=stream)
    b.w4a16_gemm(t["x4l"], t["wq4l"], t["s4l"], t["z4l"], out=t["out_w4dl"], stream=stream)


def clear_outputs(t):
    for k in OUTPUTS:
        t[k].view(torch.uint8).fill_(0xA5)   # a pattern no product leaves behind


def snapshot(t):
    return {k: t[k].view(torch.uint8).cpu().numpy().copy() for k in OUTPUTS}


def assert_same(t, ref, what):
    for k in OUTPUTS:
        got = t[k].view(torch.uint8).cpu().numpy()
        assert np.array_equal(got, ref[k]), f"{what}: {k} differs from the eager result"




@contextlib.contextmanager
def library(path):
    """The binding's calls go to the library at `path` inside the block (the normal library
    is restored after it)."""
    from quantized_gemm_quantize_amd import binding
    saved = binding._lib, binding.LIB_PATH
    binding._lib, binding.LIB_PATH = None, path
    try:
        binding.load()
        yield binding
    finally:
        binding._lib, binding.LIB_PATH = saved
