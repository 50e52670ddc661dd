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

from gpu_layer import DEV, M, N, assert_same, clear_outputs, make_layer, run_layer, snapshot

pytestmark = pytest.mark.gpu

REPEATS = 10


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_gemm_quantize_amd import binding
    binding.load()
    return binding


@pytest.fixture(scope="module")
def layer(b):
    return make_layer(b)


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
