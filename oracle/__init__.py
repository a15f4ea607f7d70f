"""CPU oracle for the quantized mat-vec path (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package; the product path never does."""
from .oracle import *  # noqa: F401,F403
from .oracle import (BLOCK_BYTES, BLOCK_WEIGHTS, QK8_0, QK_K, dequant_i8row,  # noqa: F401
                     dequant_q4_k, dequant_q6_k, dequant_q8_0, dequantize,
                     dequantize_f32, gemm_f16, gemv, gemv_packed, q4_k_codes,
                     q4_k_scales_mins, q6_k_codes, quantize_i8row, row_bytes,
                     within_tolerance)
