"""libpeaks.so (the benchmark's on-device reference rates) on the CPU: it loads, exports its
entry points, and rejects malformed arguments before any HIP call (return -1)."""
import ctypes
import os

import pytest

from quantized_gemm_quantize_amd.build import PEAKS_LIB

ENTRY_POINTS = ["peaks_mfma_i8", "peaks_mfma_bf16", "peaks_read", "peaks_read_rows", "peaks_write",
                "peaks_operand_stream"]


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(PEAKS_LIB):
        pytest.fail(f"{PEAKS_LIB} is not built: run __graft_entry__.build() first")
    return ctypes.CDLL(PEAKS_LIB)


def test_exports(lib):
    for name in ENTRY_POINTS:
        assert hasattr(lib, name), name


def test_bad_arguments_rejected_on_the_host(lib):
    p, i32, i64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.peaks_operand_stream.argtypes = [p, p, i32, i32, i32, p, p]
    lib.peaks_read.argtypes = [p, i64, i32, p, p]
    lib.peaks_read_rows.argtypes = [p, i32, p, p]
    lib.peaks_write.argtypes = [p, i64, i32, p]
    lib.peaks_mfma_i8.argtypes = [i32, i32, p, p, p]
    lib.peaks_mfma_bf16.argtypes = [i32, i32, p, p, p]
    fake = ctypes.c_void_p(16)   # never dereferenced: every call below fails its checks first
    # operand stream: null operands, M not a multiple of 256, N not of 128, K not of 128
    assert lib.peaks_operand_stream(None, fake, 256, 128, 128, fake, None) == -1
    assert lib.peaks_operand_stream(fake, fake, 200, 128, 128, fake, None) == -1
    assert lib.peaks_operand_stream(fake, fake, 256, 100, 128, fake, None) == -1
    assert lib.peaks_operand_stream(fake, fake, 256, 128, 100, fake, None) == -1
    assert lib.peaks_operand_stream(fake, fake, 256, 128, 128, None, None) == -1
    assert lib.peaks_read(fake, 17, 1, fake, None) == -1
    assert lib.peaks_read_rows(fake, 15, fake, None) == -1
    assert lib.peaks_write(fake, 0, 1, None) == -1
    assert lib.peaks_mfma_i8(0, 1, fake, fake, None) == -1
    assert lib.peaks_mfma_bf16(1, 0, fake, fake, None) == -1
    assert lib.peaks_mfma_bf16(1, 1, None, fake, None) == -1
