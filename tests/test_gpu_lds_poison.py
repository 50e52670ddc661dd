"""The LDS-poisoned debug build against the normal build.

`libw8a8_ldspoison.so` is the library compiled with W8A8_LDS_POISON: every kernel fills its
LDS arrays with 0xA5 bytes and meets at a barrier before its first LDS access. A kernel that
read LDS its launch had not written would see that pattern instead of whatever an earlier
launch left there; left-over data can be exactly right when the same inputs run twice, which
is how such a read hides in ordinary tests. Bar: bit-identical outputs of the two builds on
every entry point (the small layer of every kind) and on the large tile configurations, with
normal-build runs in between so that each poisoned run follows launches that left
valid-looking data in LDS.
"""
import os

import pytest
import torch

from gpu_layer import DEV, assert_same, clear_outputs, library, make_layer, run_layer, snapshot
from quantized_gemm_quantize_amd.build import POISON_LIB

pytestmark = pytest.mark.gpu

# tile configurations the small layer does not reach: 256x128 tiles at one workgroup per CU
# (the prefill shape), 256x128 tiles with 64-byte K stages at two per CU (large M, short K)
# and 256x256 tiles (large M, longer K)
BIG = [(2048, 4096, 4096), (16384, 4096, 1024), (16384, 4096, 2048)]


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(POISON_LIB):
        raise RuntimeError(f"{POISON_LIB} is not built: run __graft_entry__.build() first")
    from quantized_gemm_quantize_amd import binding
    binding.load()
    return binding


def test_layer_bit_identical(b):
    layer = make_layer(b)
    clear_outputs(layer)
    run_layer(b, layer)
    torch.cuda.synchronize()
    ref = snapshot(layer)
    for rep in range(2):
        with library(POISON_LIB) as pb:
            clear_outputs(layer)
            run_layer(pb, layer)
            torch.cuda.synchronize()
            assert_same(layer, ref, f"LDS-poisoned build, run {rep}")
        clear_outputs(layer)
        run_layer(b, layer)
        torch.cuda.synchronize()
        assert_same(layer, ref, f"normal build after poisoned run {rep}")


@pytest.mark.parametrize("M,N,K", BIG)
def test_tile_configs_bit_identical(b, M, N, K):
    g = torch.Generator(device=DEV)
    g.manual_seed(M + 7 * K)
    xq = torch.randint(-128, 128, (M, K), dtype=torch.int8, device=DEV, generator=g)
    wq = torch.randint(-128, 128, (N, K), dtype=torch.int8, device=DEV, generator=g)
    sx = torch.rand(M, device=DEV, generator=g) * 1e-2 + 1e-3
    sw = torch.rand(N, device=DEV, generator=g) * 1e-3 + 1e-4
    ref_i = b.w8a8_gemm(xq, sx, wq, sw, out_dtype="i32")
    ref_b = b.w8a8_gemm(xq, sx, wq, sw)
    with library(POISON_LIB) as pb:
        got_i = pb.w8a8_gemm(xq, sx, wq, sw, out_dtype="i32")
        got_b = pb.w8a8_gemm(xq, sx, wq, sw)
        torch.cuda.synchronize()
    assert torch.equal(got_i, ref_i), f"{M}x{N}x{K}: int32 accumulators differ"
    assert torch.equal(got_b.view(torch.int16), ref_b.view(torch.int16)), f"{M}x{N}x{K}: bf16 differs"
