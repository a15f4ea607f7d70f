"""MI355X (gfx950) fused dequantize + mat-vec for block-quantized weights.

y = W x + b with W in Q8_0, Q2_K .. Q6_K (Q4_K also in the byte-minimal stream layout), per-row int8
or per-row int4 and x, y in float32,
plus small-M linear layers on binary16 X (binary16 or quantized W), all as hand-written HIP kernels behind
the C ABI of include/pesti.h.  This package is the thin Python binding
(argument marshalling only) and the seeded synthetic-input generator.
"""
from ._lib import (FORMAT_IDS, LIB_PATH, PESTI_ERR_ALIGN, PESTI_ERR_BATCH,  # noqa: F401
                   PESTI_ERR_DEVICE, PESTI_ERR_LAUNCH, PESTI_ERR_NULL, PESTI_ERR_SHAPE,
                   PESTI_OK, GemvOp, MAX_GROUP, PestiError, dequant, gemv, gemv_ops, load, pesti_abi_version,
                   pesti_dequant_i8row, pesti_dequant_q4_k, pesti_dequant_q6_k,
                   pesti_dequant_q8_0, pesti_gemm_f16_smallm, pesti_gemv_group, pesti_gemv_i8row,
                   pesti_gemv_q4_k, pesti_gemv_q6_k, pesti_gemv_q8_0, pesti_row_bytes,
                   pesti_stream_read, pesti_gemm_q8_0_smallm, pesti_gemm_q4_k_smallm,
                   pesti_gemm_q6_k_smallm, gemm_quant,
                   pesti_gemv_swiglu, pesti_gemv_q5_k, pesti_dequant_q5_k,
                   pesti_gemv_q2_k, pesti_gemv_q3_k, pesti_dequant_q2_k, pesti_dequant_q3_k,
                   pesti_gemv_i4row, pesti_dequant_i4row, pesti_gemv_q4_k_stream,
                   pesti_dequant_q4_k_stream, pesti_matrix_bytes, strerror,
                   PESTI_ERR_WORKSPACE, GEMM_FORMAT_IDS, GEMM_SCRATCH_BYTES, pesti_gemm_workspace_bytes,
                   pesti_gemm_smallm_ws, pesti_gemm_smallm_noalloc)

__all__ = [n for n in dir() if n.startswith("pesti_")] + [
    "PestiError", "GemvOp", "MAX_GROUP", "gemv", "gemv_ops", "gemm_quant", "dequant", "load", "strerror",
    "FORMAT_IDS", "GEMM_FORMAT_IDS", "LIB_PATH"]
