"""Every entry point on a caller's stream and under HIP graph capture.

The library launches on the stream it is given and never synchronizes, so a
whole layer (quantize, the dense GEMM on both paths, the addmm epilogues, the
single-launch linear, block-sparse, 2:4 and W4A16 products) can run on a side
stream or be captured into a HIP graph and replayed. Bar: bit-identical
outputs to the eager calls on the default stream, on each of ten eager runs and
ten graph replays, with eager work (output clearing, other launches) between
the replays; the eager outputs themselves are checked against the oracle on one
product so the comparison is anchored.
"""
import numpy as np
import pytest
import torch

from quantized_gemm_quantize_amd.inputs import bsr_from_dense, make_linear, make_w4a16

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
M, N, K = 320, 384, 512   # tiled paths with ragged M; N, K multiples of 128
MD = 16                   # the M-small paths
KL = 4096                 # the M-small path with both operands through LDS
REPEATS = 10


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_gemm_quantize_amd import binding
    binding.load()
    return binding


def _bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(DEV)


def _dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


@pytest.fixture(scope="module")
def layer(b):
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
    # outputs (written by every run)
    t["xq"] = torch.empty((M, K), dtype=torch.int8, device=DEV)
    t["sx"] = torch.empty((M,), dtype=torch.float32, device=DEV)
    t["xqd"] = torch.empty((MD, K), dtype=torch.int8, device=DEV)
    t["sxd"] = torch.empty((MD,), dtype=torch.float32, device=DEV)
    t["xql"] = torch.empty((MD, KL), dtype=torch.int8, device=DEV)
    t["sxl"] = torch.empty((MD,), dtype=torch.float32, device=DEV)
    for name, rows in (("gemm", M), ("addmm", M), ("dec", MD), ("dec_addmm", MD), ("fused", MD),
                       ("decl", MD), ("decl_addmm", MD),
                       ("bsr", M), ("bsr_addmm", M), ("s24", M), ("s24d", MD), ("w4", M),
                       ("w4d", MD)):
        t["out_" + name] = torch.empty((rows, N), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    return t


OUTPUTS = ["xq", "sx", "xqd", "sxd", "xql", "sxl", "out_gemm", "out_addmm", "out_dec",
           "out_dec_addmm", "out_decl", "out_decl_addmm", "out_fused", "out_bsr", "out_bsr_addmm",
           "out_s24", "out_s24d", "out_w4", "out_w4d"]


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


def clear_outputs(t):
    for k in OUTPUTS:
        t[k].view(torch.uint8).fill_(0xA5)   # a pattern no product leaves behind


def snapshot(t):
    return {k: t[k].view(torch.uint8).cpu().numpy().copy() for k in OUTPUTS}


def assert_same(t, ref, what):
    for k in OUTPUTS:
        got = t[k].view(torch.uint8).cpu().numpy()
        assert np.array_equal(got, ref[k]), f"{what}: {k} differs from the eager result"


@pytest.fixture(scope="module")
def eager_ref(b, layer):
    clear_outputs(layer)
    run_layer(b, layer)
    torch.cuda.synchronize()
    return snapshot(layer)


def test_eager_anchor(b, oracle, layer, eager_ref):
    """The eager quantization and dense product against the oracle, so the replays below
    compare to a checked result (the parity suite covers every product on its own)."""
    x_bits = layer["x"].view(torch.int16).cpu().numpy().view(np.uint16)
    xq_ref, sx_ref = oracle.quantize_rows_bf16(x_bits)
    assert np.array_equal(eager_ref["xq"].view(np.int8), xq_ref)
    assert np.array_equal(eager_ref["sx"].view(np.uint32), sx_ref.view(np.uint32))
    acc = oracle.gemm_i32(xq_ref, layer["wq"].cpu().numpy())
    out_ref = oracle.epilogue_bf16(acc, sx_ref, layer["sw"].cpu().numpy()).astype(np.int64)
    got = eager_ref["out_gemm"].view(np.uint16).reshape(M, N).astype(np.int64)
    # bf16 patterns as ordered integers: within one unit in the last place
    order = lambda v: np.where(v & 0x8000, -(v & 0x7FFF), v)
    assert np.abs(order(got) - order(out_ref)).max() <= 1


def test_side_stream(b, layer, eager_ref):
    """The same layer on a non-default stream, passed explicitly and as the current stream."""
    side = torch.cuda.Stream()
    for explicit in (True, False):
        clear_outputs(layer)
        torch.cuda.synchronize()
        if explicit:
            run_layer(b, layer, stream=side)
        else:
            with torch.cuda.stream(side):
                run_layer(b, layer)
        side.synchronize()
        assert_same(layer, eager_ref, f"side stream ({'argument' if explicit else 'current'})")


def test_eager_repeats(b, layer, eager_ref):
    """Ten more eager runs of every entry point, each after clearing the outputs: bit-identical
    every time (no order-dependent reductions, no stale state between calls)."""
    for rep in range(REPEATS):
        clear_outputs(layer)
        run_layer(b, layer)
        torch.cuda.synchronize()
        assert_same(layer, eager_ref, f"eager run {rep}")


def test_graph_replays(b, layer, eager_ref):
    """The layer captured into one HIP graph: ten replays, each after eager clearing of the
    outputs and an unrelated eager launch, each bit-identical to the eager run."""
    warm = torch.cuda.Stream()
    warm.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(warm):
        run_layer(b, layer)
    torch.cuda.current_stream().wait_stream(warm)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_layer(b, layer)
    torch.cuda.synchronize()
    other = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    for rep in range(REPEATS):
        clear_outputs(layer)
        b.w8a8_gemm(layer["xq"], layer["sx"], layer["wq"], layer["sw"], out=other)  # eager work
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(layer, eager_ref, f"graph replay {rep}")
