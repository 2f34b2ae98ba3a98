"""CPU reference (oracle) for dense GEMM -- test infrastructure only.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the GPU library.
"""
from .oracle import (  # noqa: F401
    build, lib_path, gemm_f32, gemm_bf16, gemm_bf16_batched, dot_bf16, dot_f32,
    round_bf16, num_threads, set_num_threads, round_bf16_value, silu, gemm_bf16_silu, swiglu_bf16,
    e4m3_decode, e4m3_encode, quantize_rows_e4m3, quantize_cols_e4m3, quantize_fixed_e4m3, swiglu_e4m3, silu_mul_bf16, gemm_fp8_nt, gemm_fp8_nt_affine,
    gemm_bf16_affine,
)
