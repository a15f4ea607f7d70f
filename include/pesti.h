/*
 * pesti.h - C ABI of the MI355X (gfx950) quantized mat-vec library.
 *
 * What is computed
 *   The decode-step linear layer y = W x (+ b) with block-quantized W, as the
 *   row-major matrix-vector product that dominates a decode step and the
 *   fused dequantize + mat-vec that never expands W to float32 ("Project
 *   scaffold: modules, CLI, and correctness harness", file summaries of
 *   tensor.rs and quant.rs), over the GGUF K-family formats that "PESTI -
 *   Portable Execution Substrate for Transformer Inference" dequantizes
 *   byte-exactly ("What This Is").  The same boundary carries the small-M
 *   prompt-width linear layer x @ w + b ("inferno" README, "Design notes"
 *   and "Benchmarks": c_attn / c_proj / mlp_fc at 32 prompt tokens).
 *
 * Block formats (the pages name them; the byte layouts are the GGUF ones):
 *   Q8_0   34 B / 32 weights : binary16 d, int8 q[32].          w = d*q
 *   Q4_K  144 B / 256 weights: binary16 d, binary16 dmin, 12 B of packed
 *          6-bit scales sc[8] and mins m[8], 128 B of 4-bit codes.
 *                                                  w = d*sc[j]*q - dmin*m[j]
 *   Q2_K   84 B / 256 weights: 16 bytes of (4-bit scale, 4-bit min) per
 *          16-weight sub-block, 64 B of 2-bit codes, binary16 d, dmin.
 *          Weight 128h+32j+16c+l: bits 2j of code byte 32h+16c+l, sub-block
 *          8h+2j+c.                                w = d*sc[s]*q - dmin*m[s]
 *   Q3_K  110 B / 256 weights: 32 B of high bits, 64 B of 2-bit codes (as
 *          Q2_K), 12 B of sixteen 6-bit scales, binary16 d.  The code is
 *          the low bits minus 4 where its high bit (bit 4h+j of byte 16c+l)
 *          is clear.                               w = d*(scale[s]-32)*q
 *   Q5_K  176 B / 256 weights: d, dmin, the 12 scale/min bytes of Q4_K,
 *          32 B of fifth bits, 128 B of low 4-bit codes (Q4_K's runs).
 *                                                  w = d*sc[j]*q - dmin*m[j]
 *   Q6_K  210 B / 256 weights: 128 B low 4-bit parts, 64 B high 2-bit parts,
 *          int8 sc[16], binary16 d.                w = d*sc[i/16]*(q - 32)
 *   i8row int8 codes [out][in] plus one float32 scale per row. w = s[o]*q
 *   i4row 4-bit two's complement codes (-8..7), two per byte: weight 2k in
 *          the low nibble of byte k, 2k+1 in the high nibble; a row is
 *          32 B per 64 weights (padded with codes that are never read into
 *          the result), plus one float32 scale per row.      w = s[o]*q
 *
 * Layouts and conventions (every entry point)
 *   - W has out_features rows.  A packed row is ceil(in/QK) whole blocks
 *     (QK = 32 for Q8_0, 256 for the K family); rows follow each other with
 *     stride pesti_row_bytes(format, in_features) bytes.  When in_features
 *     is not a multiple of 256, the columns in_features..end of the last
 *     super-block are padding: they are never read into the result and
 *     their bytes may hold anything.
 *   - x is float32 [batch][in_features], y is float32 [batch][out_features],
 *     bias is float32 [out_features] or NULL.  y is overwritten:
 *     y[b][o] = sum_i w[o][i] * x[b][i] + bias[o].
 *   - Accumulation is float32; dequantized weights are never written out.
 *     Result bound: |y - exact| <= 1e-4 * sum_i |w_i x_i| + 1e-6 for the
 *     mat-vec (2e-3 for the f16 GEMM).
 *   - Pointers are device pointers owned by the caller, on the calling
 *     thread's current HIP device, and must be 16-byte aligned (blocks, x,
 *     y, w, codes; bias and row_scales 4-byte aligned).  x and y must not
 *     overlap.  `stream` is a hipStream_t (NULL = the legacy default
 *     stream).
 *   - Calls only enqueue work on `stream` and return; they never allocate,
 *     free or synchronize, and keep no state between calls, so they may be
 *     issued concurrently on any number of streams.
 *
 * Errors
 *   Return 0 on success or a negative PESTI_ERR_* code.  On any non-zero
 *   return nothing was enqueued and y is untouched.  An empty output
 *   (out_features == 0 or batch == 0, or rows == 0 for dequant) returns 0
 *   without touching any pointer.  in_features == 0 is a valid shape:
 *   y = bias (or 0).  Faults inside a kernel surface at the caller's next
 *   synchronization, as with any HIP kernel.  Nothing falls back to the CPU.
 */
#ifndef PESTI_H
#define PESTI_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PESTI_ABI_VERSION 3

#define PESTI_OK 0
#define PESTI_ERR_NULL (-1)   /* a required pointer is NULL                 */
#define PESTI_ERR_SHAPE (-2)  /* negative size, in_features % 32 != 0, or  */
                              /* in_features above PESTI_MAX_IN_FEATURES    */
#define PESTI_ERR_BATCH (-3)  /* batch outside [0, 8]; GEMM m outside [0,  */
                              /* PESTI_MAX_GEMM_M]                           */
#define PESTI_ERR_ALIGN (-4)  /* a pointer breaks the alignment rule above  */
#define PESTI_ERR_LAUNCH (-5) /* the HIP launch reported an error           */
#define PESTI_ERR_DEVICE (-6) /* current device is not gfx950, or no device */
#define PESTI_ERR_WORKSPACE (-7) /* GEMM workspace missing or too small     */

#define PESTI_FMT_Q8_0 0
#define PESTI_FMT_Q4_K 1
#define PESTI_FMT_Q6_K 2
#define PESTI_FMT_I8ROW 3
#define PESTI_FMT_Q5_K 4
#define PESTI_FMT_Q2_K 5
#define PESTI_FMT_Q3_K 6
#define PESTI_FMT_I4ROW 7
#define PESTI_FMT_Q4_K_STREAM 8
/* binary16 weights [out][in]: for the small-M GEMM calls that take a format */
#define PESTI_FMT_F16 16

#define PESTI_MAX_BATCH 8
#define PESTI_MAX_IN_FEATURES 32768
#define PESTI_MAX_GEMM_M 4096

/* --- quantized mat-vec, y = W x + b ------------------------------------ */

/* Q8_0 (34-byte blocks of 32 weights).  blocks: out_features rows of
 * in_features/32 blocks.  batch in [0, 8].  Matrices of at least 16384 rows
 * with rows of an even block count and at most 1024 weights, at batch 4..8,
 * run on the matrix cores with x split as described for pesti_gemv_q4_k
 * (same bound). */
int pesti_gemv_q8_0(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);

/* Q4_K (144-byte super-blocks of 256 weights, rows padded to whole
 * super-blocks).  Same arguments as pesti_gemv_q8_0.  Matrices of at least
 * 16384 rows with rows of at most 1024 weights, at batch 3..8, run on the
 * matrix cores: each 32-weight block of x is scaled by a power of two and
 * split into binary16 high and low parts (products with the exact codes
 * are exact), which adds at most 2^-22 |x_i| + 2^-39 max|x_block| per
 * element of x to the float32 error; the result meets the same
 * 1e-4 * sum|w x| + 1e-6 bound. */
int pesti_gemv_q4_k(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);

/* Q4_K in the stream layout: the byte-minimal layout of rows that are not a
 * whole number of super-blocks (the 896-weight rows of "PESTI ..." README,
 * "Conformance": hidden size 896 is 3.5 super-blocks).  The matrix's
 * weights in row-major order, weight (r, c) at position r * in + c of one
 * stream, are cut into 144-byte Q4_K super-blocks in stream order; only the
 * last super-block holds padding.  `blocks` is pesti_matrix_bytes(
 * PESTI_FMT_Q4_K_STREAM, out_features, in_features) bytes: a 896-weight row
 * takes 504 bytes instead of 576, and rows start at weight 0 or 128 of a
 * super-block.  in_features must be a multiple of 64 (rows of whole 64-weight
 * runs), else PESTI_ERR_SHAPE; for multiples of 256 the layout is the row
 * layout of pesti_gemv_q4_k byte for byte.  Same arguments and bound as
 * pesti_gemv_q4_k; every batch runs on the vector ALUs. */
int pesti_gemv_q4_k_stream(int64_t out_features, int64_t in_features, const void* blocks,
                           const float* x, float* y, const float* bias, int32_t batch,
                           void* stream);

/* Q2_K (84-byte) and Q3_K (110-byte) super-blocks of 256 weights, rows
 * padded to whole super-blocks ("PESTI ..." README, "What This Is": all
 * K-family quantizations, Q2_K to Q8_0).  Same arguments as
 * pesti_gemv_q8_0.  Matrices of at least 16384 rows with rows of at most
 * 1024 weights, at batch 3..8, run on the matrix cores with x split as
 * described for pesti_gemv_q4_k (same bound). */
int pesti_gemv_q2_k(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);
int pesti_gemv_q3_k(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);

/* Q5_K (176-byte super-blocks of 256 weights, rows padded to whole
 * super-blocks; "PESTI ..." README, "What This Is": all K-family
 * quantizations).  Same arguments as pesti_gemv_q8_0.  Matrices of at least
 * 16384 rows with rows of at most 1024 weights, at batch 3..8, run on the
 * matrix cores with x split as described for pesti_gemv_q4_k (same
 * bound). */
int pesti_gemv_q5_k(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);

/* Q6_K (210-byte super-blocks of 256 weights, rows padded to whole
 * super-blocks).  Same arguments as pesti_gemv_q8_0.  Matrices of at least
 * 16384 rows with rows of at most 1024 weights, at batch 5..8, run on the
 * matrix cores with x split as described for pesti_gemv_q4_k (same
 * bound). */
int pesti_gemv_q6_k(int64_t out_features, int64_t in_features, const void* blocks,
                    const float* x, float* y, const float* bias, int32_t batch,
                    void* stream);

/* Per-row symmetric int8 ("Project scaffold ...", quant.rs): codes int8
 * [out][in] row-major, row_scales float32 [out]. */
int pesti_gemv_i8row(int64_t out_features, int64_t in_features, const int8_t* codes,
                     const float* row_scales, const float* x, float* y,
                     const float* bias, int32_t batch, void* stream);

/* Per-row symmetric int4 ("Project scaffold ...", quant.rs lists INT4 beside
 * INT8): packed int4 rows of pesti_row_bytes(PESTI_FMT_I4ROW, in) bytes,
 * row_scales float32 [out].  Matrices of at least 16384 rows with rows of at
 * most 1024 weights, at batch 2..8, run on the matrix cores with x split as
 * described for pesti_gemv_q4_k.  Both kernels take every code exactly
 * (the vector-ALU kernel as the signed byte 16 q, the sum then scaled by
 * 2^-4 exactly), so the mat-vec bound above holds unchanged. */
int pesti_gemv_i4row(int64_t out_features, int64_t in_features, const void* packed,
                     const float* row_scales, const float* x, float* y,
                     const float* bias, int32_t batch, void* stream);

/* --- grouped mat-vec: several independent products in one launch ---------
 * One mat-vec of a group: y = W x + b with the layouts above (w is the
 * packed rows, or the int8 codes for i8row; row_scales only for i8row and
 * i4row). */
typedef struct pesti_gemv_op {
  int64_t out_features;
  int64_t in_features;
  const void* w;
  const float* row_scales;
  const float* x;
  float* y;
  const float* bias;
} pesti_gemv_op;

#define PESTI_MAX_GROUP 8

/* Up to PESTI_MAX_GROUP independent mat-vecs of one PESTI_FMT_* format and
 * one batch size, computed by one kernel launch (two or three when the ops
 * need different kernels: each op takes the kernel its own single call
 * would take - Q8_0 rows of an odd or even block count, tall K-quant, Q8_0
 * and int4 matrices on the matrix cores - so every op's y has the bits of its single
 * call).  This is the decode-step
 * case of projections that read the same activations (Q, K and V; gate and
 * up: "PESTI ..." README, "Conformance", per-head GQA and SwiGLU), where
 * one launch replaces several dependent ones.  ops is a host array read
 * during the call; each op follows the conventions and checks of the
 * single-matrix entry points (an op with out_features == 0 is skipped);
 * the y buffers of different ops must not overlap.  Returns the first
 * failing op's error, before anything is enqueued. */
int pesti_gemv_group(int32_t format, int32_t n_ops, const pesti_gemv_op* ops, int32_t batch,
                     void* stream);

/* --- fused SwiGLU feed-forward input, h = silu(W_gate x) * (W_up x) ------
 * The gate and up projections of a decode step's feed-forward block and
 * the SwiGLU that joins them ("PESTI ..." README, "Conformance": SwiGLU =
 * silu(gate) * up with the sigmoid-based SiLU, silu(g) = g / (1 + e^-g)),
 * in one launch: each lane group computes row o of both matrices and writes
 * only h[b][o].  w_gate and w_up are two matrices of one PESTI_FMT_* format
 * and the same shape, laid out as for the single mat-vecs (no bias);
 * gate_scales / up_scales are their row scales for PESTI_FMT_I8ROW and
 * PESTI_FMT_I4ROW and are ignored otherwise.  x float32 [batch][in], h float32 [batch][out].  Rows
 * must fit one load round: in_features up to 4096 (K family, i8row, i4row, Q8_0
 * with in % 64 == 0) or 2048 (other Q8_0), else PESTI_ERR_SHAPE.
 * Bound: |h - exact| <= 1.1 * eg * |u| + |silu(g)| * eu + 2 * eg * eu
 * + 1e-6 * |h| + 1e-6, with eg, eu the mat-vec bounds of g and u. */
int pesti_gemv_swiglu(int32_t format, int64_t out_features, int64_t in_features,
                      const void* w_gate, const void* w_up, const float* gate_scales,
                      const float* up_scales, const float* x, float* h, int32_t batch,
                      void* stream);

/* --- small-M binary16 linear layer, Y = X W^T + b ------------------------
 * X binary16 [m][in], W binary16 [out][in] (the same row orientation as the
 * mat-vec; a GPT-2 c_attn "768x2304" has in = 768, out = 2304), Y float32
 * [m][out], bias float32 [out] or NULL.  m in [0, PESTI_MAX_GEMM_M]; float32
 * accumulation; matrix cores for m >= 16, vector ALUs below. */
int pesti_gemm_f16_smallm(int64_t m, int64_t out_features, int64_t in_features,
                          const uint16_t* w, const uint16_t* x, float* y,
                          const float* bias, void* stream);

/* --- small-M linear layer on quantized weights, Y = X W^T + b -------------
 * The prompt-width product of the same layer ("inferno" README,
 * "Benchmarks": x @ w + b at prompt width) with W kept in the block format
 * of the mat-vec ("Project scaffold ...", quant.rs: dequantize fused into
 * the product, W never expanded).  blocks: out_features packed rows exactly
 * as for pesti_gemv_q8_0 / pesti_gemv_q4_k / pesti_gemv_q6_k; X binary16 [m][in] (16-byte
 * aligned), Y float32 [m][out], bias float32 [out] or NULL; m in [0,
 * PESTI_MAX_GEMM_M].  The matrix cores multiply the exact integer codes by
 * X (every product exact in float32) one 32-weight block or sub-block at a
 * time, and the block scales are applied to each partial sum in float32.
 * Any m >= 1 works; for m <= 8 the batched mat-vec on float32 X is the
 * faster call.  Errors as for pesti_gemm_f16_smallm. */
int pesti_gemm_q8_0_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);
int pesti_gemm_q4_k_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);
/* Q2_K, Q3_K and Q5_K rows as for their mat-vecs.  Their codes times the
 * code's own sub-block scale are small binary16 integers (q * sc <= 45,
 * |q * (sc - 32)| <= 128, q * sc <= 1953), so the operand carries the scale
 * and each lane its own sub-block's; mins (Q2_K, Q5_K) are products of X
 * sums or of X against the mins. */
int pesti_gemm_q2_k_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);
int pesti_gemm_q3_k_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);
int pesti_gemm_q5_k_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);
/* Q6_K rows as for pesti_gemv_q6_k.  Its codes are exact too (q - 32), but
 * each 32-weight k-step spans two 16-weight sub-blocks, so a step is two
 * products (each on half the operand) scaled apart. */
int pesti_gemm_q6_k_smallm(int64_t m, int64_t out_features, int64_t in_features,
                           const void* blocks, const uint16_t* x, float* y,
                           const float* bias, void* stream);

/* --- the same GEMMs with a caller's workspace (split K) -------------------
 * Narrow layers (fewer than 96 16-column tiles, e.g. the 896-wide down
 * projection) with long rows (in_features over 4096) run one workgroup per
 * output tile and leave most compute units idle.  With a workspace, K is
 * split over 2..4 workgroups per tile (more workgroups for fewer row tiles
 * of X; binary16 only at m 16; Q8_0, Q3_K and Q6_K take two row tiles of X
 * per workgroup), each writing its partial tile to the
 * workspace, and a second launch on the same stream sums the partials in a
 * fixed order and adds the bias: results do not depend on timing, but the
 * summation order differs from the call without workspace (same bound).
 *
 * pesti_gemm_workspace_bytes returns the bytes the split needs for this
 * format (PESTI_FMT_F16 or one of the six block formats) and shape: 0 when
 * the shape does not split, at most PESTI_GEMM_SCRATCH_BYTES (512 KiB);
 * negative PESTI_ERR_* for an unknown format or a bad shape.  Host-only,
 * no device needed.
 *
 * pesti_gemm_smallm_ws: arguments as for pesti_gemm_<format>_smallm (w is
 * the binary16 W or the packed blocks), plus `workspace`, device memory of
 * at least that many bytes, 16-byte aligned, owned by the caller and used
 * only by the work this call enqueues (calls that run concurrently need
 * their own); ignored when the shape needs none.  Errors as for the
 * format's call, PESTI_ERR_SHAPE for an unknown format, and
 * PESTI_ERR_WORKSPACE if a needed workspace is NULL or smaller. */
int64_t pesti_gemm_workspace_bytes(int32_t format, int64_t m, int64_t out_features, int64_t in_features);
int pesti_gemm_smallm_ws(int32_t format, int64_t m, int64_t out_features, int64_t in_features,
                         const void* w, const uint16_t* x, float* y, const float* bias,
                         void* workspace, int64_t workspace_bytes, void* stream);

/* --- allocation-free form of pesti_gemm_smallm_ws --------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * GEMM with the split partials in the library's own scratch, a static device
 * array of PESTI_GEMM_SCRATCH_BYTES on each GPU the library runs on, held
 * until the process ends.  Nothing is allocated; every shape's workspace
 * fits.  All calls on one GPU share that GPU's array: calls that overlap in
 * time on one GPU (on different streams, or graphs replayed concurrently)
 * race and may return wrong results; calls ordered on one stream are safe.
 * Nothing in the array needs to start at zero.  Results equal
 * pesti_gemm_smallm_ws bit for bit.  Errors as for pesti_gemm_smallm_ws;
 * PESTI_ERR_WORKSPACE if a shape ever needed more than the array. */
#define PESTI_GEMM_SCRATCH_BYTES (512 * 1024)
int pesti_gemm_smallm_noalloc(int32_t format, int64_t m, int64_t out_features, int64_t in_features,
                              const void* w, const uint16_t* x, float* y, const float* bias,
                              void* stream);

/* --- dequantization to float32 (bit-exact; checks the unpacking) --------
 * w_out float32 [rows][in_features]: each weight rounded once from its
 * exact value (all formats here dequantize exactly in float32 except the
 * final subtraction of Q2_K / Q4_K / Q5_K and the scale product of
 * i8row and i4row). */
int pesti_dequant_q8_0(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_q4_k(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_q4_k_stream(int64_t rows, int64_t in_features, const void* blocks,
                              float* w_out, void* stream);
int pesti_dequant_q2_k(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_q3_k(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_q5_k(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_q6_k(int64_t rows, int64_t in_features, const void* blocks,
                       float* w_out, void* stream);
int pesti_dequant_i8row(int64_t rows, int64_t in_features, const int8_t* codes,
                        const float* row_scales, float* w_out, void* stream);
int pesti_dequant_i4row(int64_t rows, int64_t in_features, const void* packed,
                        const float* row_scales, float* w_out, void* stream);

/* --- measurement hook ----------------------------------------------------
 * A plain streaming read of `bytes` bytes (a multiple of 16) at `buf`
 * (16-byte aligned): the streaming-read ceiling that a mat-vec reading the
 * same number of bytes is measured against.  PESTI_READ_GROUPS workgroups
 * each write the XOR of the dwords they read to partial[group] (the XOR of
 * all entries is the XOR of the whole buffer); `partial` is a device array
 * of PESTI_READ_GROUPS uint32 owned by the caller. */
#define PESTI_READ_GROUPS 4096
int pesti_stream_read(const void* buf, int64_t bytes, uint32_t* partial, void* stream);

/* --- host-only helpers (no device work) --------------------------------- */

/* Packed bytes per row for a PESTI_FMT_* format (code bytes only for
 * i8row); -1 for an unknown format, a negative / non-multiple-of-32
 * in_features, or PESTI_FMT_Q4_K_STREAM (whose rows have no fixed size:
 * see pesti_matrix_bytes). */
int64_t pesti_row_bytes(int32_t format, int64_t in_features);

/* Packed bytes of a whole matrix of `rows` rows: rows * pesti_row_bytes for
 * the row layouts, the super-blocks holding rows * in_features weights for
 * PESTI_FMT_Q4_K_STREAM (in_features a multiple of 64); -1 for an unknown
 * format or an invalid size. */
int64_t pesti_matrix_bytes(int32_t format, int64_t rows, int64_t in_features);

/* Static text for a status code. */
const char* pesti_strerror(int status);

/* PESTI_ABI_VERSION of the built library. */
int32_t pesti_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PESTI_H */
