"""CPU oracle for the W8A8 linear layer -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package. It shares nothing with the HIP library.
"""
from .oracle import (  # noqa: F401
    build_oracle,
    bf16_gemm,
    bf16_rne_from_f64,
    bsr_gemm_i32,
    compress24,
    decompress24,
    epilogue_addmm_bf16,
    epilogue_bf16,
    f16_gemm,
    f16_rne_from_f64,
    gemm_i32,
    load_oracle,
    num_threads,
    quantize_rows_bf16,
    quantize_rows_f32,
    w4a16_dequant,
)
