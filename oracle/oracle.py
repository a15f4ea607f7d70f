"""Plain, slow, obviously-correct CPU oracle for the quantized mat-vec path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the package
entry script and the CPU-baseline leg of the benchmark use it.  It shares no
code with the HIP library and imports nothing from it.

What it computes, and the passages it follows
---------------------------------------------
* "PESTI - Portable Execution Substrate for Transformer Inference", section
  "What This Is": GGUF K-family block formats are dequantized byte-exactly,
  and every fast path is checked against an independent numpy oracle.
* The same page, section "Conformance": the forward pass is diffed against
  that oracle to a stated tolerance; the Q4_K dequant/accumulation order is
  the only expected difference.
* "Project scaffold: modules, CLI, and correctness harness" (ember PR #1),
  file summary for tensor.rs and quant.rs: the row-major matrix-vector
  product dominates a decode step; per-row symmetric int8 quantization comes
  with a fused dequantize + mat-vec that never expands weights to f32.
* "inferno" README, section "Design notes": kernels take contiguous
  row-major tensors in and out; a linear layer is x @ w + b.

The pages name the formats (Q8_0, Q4_K, Q6_K, per-row int8) but print no byte
layout.  The layouts below are the GGUF block arrangements, the plainest
reading of that page's claim to parse GGUF files and dequantize them
byte-exactly:

* Q8_0, 34 bytes per 32 weights: binary16 d, then 32 int8 codes q.
  w[i] = d * q[i].
* Q4_K, 144 bytes per 256 weights: binary16 d, binary16 dmin, 12 bytes that
  pack eight 6-bit sub-block scales sc[j] and eight 6-bit mins m[j], then 128
  bytes of 4-bit codes.  Sub-block j holds weights 32j .. 32j+31.
  w[i] = d * sc[j] * q[i] - dmin * m[j].
* Q5_K, 176 bytes per 256 weights: binary16 d, binary16 dmin, the same 12
  bytes of 6-bit scales and mins as Q4_K, 32 bytes of high bits qh, then
  128 bytes of low 4-bit codes in Q4_K's arrangement.  Weight 64r + l
  (l < 32) has high bit r*2 of qh[l], weight 64r + 32 + l bit 2r+1.
  w[i] = d * sc[j] * q[i] - dmin * m[j], q in 0..31.  (The pages list the
  whole K family by name only; this is the GGUF arrangement.)
* Q2_K, 84 bytes per 256 weights: 16 bytes, one per 16-weight sub-block,
  holding a 4-bit scale (low nibble) and a 4-bit min (high nibble); 64
  bytes of 2-bit codes; binary16 d; binary16 dmin.  Weight 128h + 32j +
  16c + l (h < 2, j < 4, c < 2, l < 16) is bits 2j, 2j+1 of code byte
  32h + 16c + l, in sub-block 8h + 2j + c.  w = d*sc*q - dmin*m, q in 0..3.
* Q3_K, 110 bytes per 256 weights: 32 bytes of high bits, 64 bytes of
  2-bit codes (arranged as in Q2_K), 12 bytes packing sixteen 6-bit scales,
  binary16 d.  Weight 128h + 32j + 16c + l has its low two bits as in Q2_K
  and its high bit at bit 4h + j of high-bit byte 16c + l; its code is the
  low two bits, minus 4 when the high bit is clear (q in -4..3).  Scale k:
  bits 0-3 are bits 4(k // 8) .. +3 of byte k % 8, bits 4-5 are bits
  2(k // 4) .. +1 of byte 8 + k % 4; w = d * (scale - 32) * q.
* Q6_K, 210 bytes per 256 weights: 128 bytes of low 4-bit code parts, 64
  bytes of high 2-bit code parts, 16 int8 sub-block scales (16 weights
  each), binary16 d.   w[i] = d * sc[i // 16] * (q[i] - 32), q in 0..63.
* per-row int8 ("i8row"): int8 codes [rows][in] and one f32 scale per row.
  w[o][i] = scale[o] * q[o][i].
* per-row int4 ("i4row"; the scaffold's quant.rs lists INT4 beside INT8):
  4-bit two's complement codes, two per byte (weight 2k in the low nibble
  of byte k, 2k + 1 in the high nibble), rows padded to 64 weights (32
  bytes), one f32 scale per row.  w[o][i] = scale[o] * q[o][i], q in -8..7.

Rows whose length is not a multiple of the 256-weight super-block are padded
to whole super-blocks; the padding columns are never part of the matrix and
the oracle drops them after decoding (their bytes may hold anything).

* Q4_K stream ("q4_k_stream"; the byte-minimal layout of rows that are not a
  whole number of super-blocks): the matrix's weights in row-major order,
  weight (r, c) at position r * in + c of one stream, cut into 256-weight
  Q4_K super-blocks in stream order; only the last super-block is padded.
  A 896-weight row is 3.5 super-blocks (504 bytes) and starts at weight 0
  or 128 of one.  Each super-block decodes as a Q4_K block; the stream is
  then cut back into rows.

All dequantized values are exact in float64 (binary16 d times a small
integer, minus binary16 dmin times a 6-bit integer, needs at most 50
significant bits; Q5_K's 5-bit codes one more; Q2_K and Q3_K fewer), so
float64 is the exact reference; the float32 value of a weight is the float64 value rounded once to nearest-even.
"""
from __future__ import annotations

import math

import numpy as np

QK8_0 = 32          # weights per Q8_0 block
QK_K = 256          # weights per K-family super-block

BLOCK_WEIGHTS = {"q8_0": QK8_0, "q2_k": QK_K, "q3_k": QK_K, "q4_k": QK_K, "q5_k": QK_K, "q6_k": QK_K}
BLOCK_BYTES = {"q8_0": 34, "q2_k": 84, "q3_k": 110, "q4_k": 144, "q5_k": 176, "q6_k": 210}


# ---------------------------------------------------------------------------
# layout helpers
# ---------------------------------------------------------------------------
def matrix_bytes(fmt: str, rows: int, in_features: int) -> int:
    """Bytes of a packed matrix: rows * row_bytes, or for the Q4_K stream
    layout the whole super-blocks that hold rows * in_features weights."""
    if fmt == "q4_k_stream":
        return -(-(rows * in_features) // QK_K) * BLOCK_BYTES["q4_k"]
    return rows * row_bytes(fmt, in_features)


def row_bytes(fmt: str, in_features: int) -> int:
    """Bytes of one packed row of `in_features` weights (row padded to whole
    blocks).  For i8row this is the code bytes only; the scale is separate."""
    if fmt == "i8row":
        return in_features
    if fmt == "i4row":
        return -(-in_features // 64) * 32
    qk = BLOCK_WEIGHTS[fmt]
    nblk = -(-in_features // qk)
    return nblk * BLOCK_BYTES[fmt]


def _blocks(packed: np.ndarray, rows: int, in_features: int, fmt: str) -> np.ndarray:
    """View the packed buffer as [rows, blocks_per_row, block_bytes] uint8."""
    packed = np.ascontiguousarray(np.asarray(packed, dtype=np.uint8))
    rb = row_bytes(fmt, in_features)
    if packed.size != rows * rb:
        raise ValueError(f"{fmt}: expected {rows * rb} bytes, got {packed.size}")
    nblk = rb // BLOCK_BYTES[fmt]
    return packed.reshape(rows, nblk, BLOCK_BYTES[fmt])


def _binary16(two_bytes: np.ndarray) -> np.ndarray:
    """Decode little-endian IEEE binary16 (last axis = 2 bytes) to float64.
    numpy's float16 decodes subnormals exactly."""
    b = np.ascontiguousarray(two_bytes, dtype=np.uint8)
    return b.view("<f2")[..., 0].astype(np.float64)


# ---------------------------------------------------------------------------
# dequantization (exact, float64)
# ---------------------------------------------------------------------------
def dequant_q8_0(packed, rows: int, in_features: int) -> np.ndarray:
    """Q8_0: w = d * q for each 32-weight block.  Returns float64 [rows, in]."""
    if in_features % QK8_0:
        raise ValueError("Q8_0 needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q8_0")
    d = _binary16(blk[:, :, 0:2])                       # [rows, nblk]
    q = blk[:, :, 2:34].view(np.int8).astype(np.float64)  # [rows, nblk, 32]
    w = d[:, :, None] * q
    return w.reshape(rows, -1)[:, :in_features]


def q2_k_codes(qs: np.ndarray) -> np.ndarray:
    """The 256 2-bit codes (0..3) of a Q2_K or the low bits of a Q3_K
    super-block from its 64 code bytes: weight i = 128h + 32j + 16c + l
    takes bits 2j, 2j+1 of byte 32h + 16c + l."""
    qs = qs.astype(np.int64)
    q = np.zeros(qs.shape[:-1] + (QK_K,), dtype=np.int64)
    for i in range(QK_K):
        h, rest = divmod(i, 128)
        j, rest = divmod(rest, 32)
        c, l = divmod(rest, 16)
        q[..., i] = (qs[..., 32 * h + 16 * c + l] >> (2 * j)) & 3
    return q


def dequant_q2_k(packed, rows: int, in_features: int) -> np.ndarray:
    """Q2_K: w = d * sc[s] * q - dmin * m[s] over 16-weight sub-blocks s
    (sc, m the nibbles of scale byte s).  float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q2_K needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q2_k")
    S = blk[:, :, 0:16].astype(np.int64)
    sc, m = S & 15, S >> 4
    q = q2_k_codes(blk[:, :, 16:80])
    d = _binary16(blk[:, :, 80:82])
    dmin = _binary16(blk[:, :, 82:84])
    sub = np.arange(QK_K) // 16
    w = d[:, :, None] * sc[:, :, sub] * q - dmin[:, :, None] * m[:, :, sub]
    return w.reshape(rows, -1)[:, :in_features]


def q3_k_scales(S: np.ndarray) -> np.ndarray:
    """The sixteen 6-bit scales (0..63, before the -32 offset) of a Q3_K
    super-block from its 12 scale bytes: scale k has bits 0-3 from bits
    4(k // 8) .. +3 of byte k % 8 and bits 4-5 from bits 2(k // 4) .. +1 of
    byte 8 + k % 4."""
    S = S.astype(np.int64)
    out = np.zeros(S.shape[:-1] + (16,), dtype=np.int64)
    for k in range(16):
        low = (S[..., k % 8] >> (4 * (k // 8))) & 15
        high = (S[..., 8 + k % 4] >> (2 * (k // 4))) & 3
        out[..., k] = low | (high << 4)
    return out


def q3_k_codes(hm: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """The 256 signed 3-bit codes (-4..3) of a Q3_K super-block: the Q2_K
    arrangement's low two bits, minus 4 where the high bit (bit 4h + j of
    high-bit byte 16c + l) is clear."""
    low = q2_k_codes(qs)
    hm = hm.astype(np.int64)
    q = np.zeros_like(low)
    for i in range(QK_K):
        h, rest = divmod(i, 128)
        j, rest = divmod(rest, 32)
        c, l = divmod(rest, 16)
        hbit = (hm[..., 16 * c + l] >> (4 * h + j)) & 1
        q[..., i] = low[..., i] - 4 * (1 - hbit)
    return q


def dequant_q3_k(packed, rows: int, in_features: int) -> np.ndarray:
    """Q3_K: w = d * (scale[s] - 32) * q over 16-weight sub-blocks s.
    float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q3_K needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q3_k")
    q = q3_k_codes(blk[:, :, 0:32], blk[:, :, 32:96])
    sc = q3_k_scales(blk[:, :, 96:108]) - 32
    d = _binary16(blk[:, :, 108:110])
    sub = np.arange(QK_K) // 16
    w = d[:, :, None] * sc[:, :, sub] * q
    return w.reshape(rows, -1)[:, :in_features]


def q4_k_scales_mins(S: np.ndarray):
    """Unpack the 12 scale bytes S[0..11] of a Q4_K super-block into eight
    6-bit scales sc[j] and eight 6-bit mins m[j] (GGUF arrangement):
      j < 4 : sc[j] = S[j] & 63,                 m[j] = S[j+4] & 63
      j >= 4: sc[j] = (S[j+4] & 15) | (S[j-4] >> 6) << 4,
              m[j]  = (S[j+4] >> 4) | (S[j]   >> 6) << 4
    S is an integer array whose last axis has 12 entries."""
    S = S.astype(np.int64)
    sc = np.zeros(S.shape[:-1] + (8,), dtype=np.int64)
    m = np.zeros_like(sc)
    for j in range(4):
        sc[..., j] = S[..., j] & 63
        m[..., j] = S[..., j + 4] & 63
    for j in range(4, 8):
        sc[..., j] = (S[..., j + 4] & 15) | ((S[..., j - 4] >> 6) << 4)
        m[..., j] = (S[..., j + 4] >> 4) | ((S[..., j] >> 6) << 4)
    return sc, m


def q4_k_codes(qs: np.ndarray) -> np.ndarray:
    """The 256 4-bit codes of a Q4_K super-block from its 128 code bytes.
    Weights come in four runs of 64: run r uses bytes 32r .. 32r+31; its
    first 32 weights are the low nibbles of those bytes, its last 32 the
    high nibbles."""
    qs = qs.astype(np.int64)
    q = np.zeros(qs.shape[:-1] + (QK_K,), dtype=np.int64)
    for i in range(QK_K):
        byte = qs[..., 32 * (i // 64) + (i % 32)]
        q[..., i] = (byte & 15) if (i % 64) < 32 else (byte >> 4)
    return q


def dequant_q4_k(packed, rows: int, in_features: int) -> np.ndarray:
    """Q4_K: w = d * sc[j] * q - dmin * m[j] in sub-block j.  float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q4_K needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q4_k")
    d = _binary16(blk[:, :, 0:2])
    dmin = _binary16(blk[:, :, 2:4])
    sc, m = q4_k_scales_mins(blk[:, :, 4:16])           # [rows, nblk, 8]
    q = q4_k_codes(blk[:, :, 16:144])                   # [rows, nblk, 256]
    sub = np.arange(QK_K) // 32                         # sub-block of each weight
    w = (d[:, :, None] * sc[:, :, sub] * q
         - dmin[:, :, None] * m[:, :, sub])
    return w.reshape(rows, -1)[:, :in_features]


def dequant_q4_k_stream(packed, rows: int, in_features: int) -> np.ndarray:
    """Q4_K stream layout: the super-blocks hold the row-major weight stream
    (see the module notes); decode them as one long Q4_K row, drop the
    padding at the end of the stream, cut into rows.  float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q4_K needs in_features % 32 == 0")
    n = rows * in_features
    nsb = -(-n // QK_K)
    flat = dequant_q4_k(np.asarray(packed).reshape(-1), 1, nsb * QK_K)[0]
    return flat[:n].reshape(rows, in_features)


def q5_k_codes(qh: np.ndarray, qs: np.ndarray) -> np.ndarray:
    """The 256 5-bit codes (0..31) of a Q5_K super-block: the low four bits
    are the Q4_K codes of the 128 bytes qs; weight i = 64r + 32c + l (run r,
    half c, l < 32) takes bit 2r + c of qh[l] as its fifth bit."""
    low = q4_k_codes(qs)
    qh = qh.astype(np.int64)
    q = np.zeros_like(low)
    for i in range(QK_K):
        r, rest = divmod(i, 64)
        c, l = divmod(rest, 32)
        q[..., i] = low[..., i] | (((qh[..., l] >> (2 * r + c)) & 1) << 4)
    return q


def dequant_q5_k(packed, rows: int, in_features: int) -> np.ndarray:
    """Q5_K: w = d * sc[j] * q - dmin * m[j] in sub-block j, q in 0..31.
    float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q5_K needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q5_k")
    d = _binary16(blk[:, :, 0:2])
    dmin = _binary16(blk[:, :, 2:4])
    sc, m = q4_k_scales_mins(blk[:, :, 4:16])
    q = q5_k_codes(blk[:, :, 16:48], blk[:, :, 48:176])
    sub = np.arange(QK_K) // 32
    w = (d[:, :, None] * sc[:, :, sub] * q
         - dmin[:, :, None] * m[:, :, sub])
    return w.reshape(rows, -1)[:, :in_features]


def q6_k_codes(ql: np.ndarray, qh: np.ndarray) -> np.ndarray:
    """The 256 6-bit codes (0..63) of a Q6_K super-block.
    Write i = 128*h + 32*g + l (h in 0..1, g in 0..3, l in 0..31).  The low
    four bits are the low nibble (g < 2) or high nibble (g >= 2) of
    ql[64h + 32*(g % 2) + l]; the high two bits are bits 2g, 2g+1 of
    qh[32h + l]."""
    ql = ql.astype(np.int64)
    qh = qh.astype(np.int64)
    q = np.zeros(ql.shape[:-1] + (QK_K,), dtype=np.int64)
    for i in range(QK_K):
        h, rest = divmod(i, 128)
        g, l = divmod(rest, 32)
        lbyte = ql[..., 64 * h + 32 * (g % 2) + l]
        low = (lbyte & 15) if g < 2 else (lbyte >> 4)
        high = (qh[..., 32 * h + l] >> (2 * g)) & 3
        q[..., i] = low | (high << 4)
    return q


def dequant_q6_k(packed, rows: int, in_features: int) -> np.ndarray:
    """Q6_K: w = d * sc[i // 16] * (q - 32).  float64 [rows, in]."""
    if in_features % 32:
        raise ValueError("Q6_K needs in_features % 32 == 0")
    blk = _blocks(packed, rows, in_features, "q6_k")
    ql = blk[:, :, 0:128]
    qh = blk[:, :, 128:192]
    sc = blk[:, :, 192:208].view(np.int8).astype(np.int64)   # [rows, nblk, 16]
    d = _binary16(blk[:, :, 208:210])
    q = q6_k_codes(ql, qh)
    sub = np.arange(QK_K) // 16
    w = d[:, :, None] * sc[:, :, sub] * (q - 32)
    return w.reshape(rows, -1)[:, :in_features]


def dequant_i8row(codes, scales) -> np.ndarray:
    """Per-row symmetric int8: w[o][i] = scale[o] * q[o][i].  float64."""
    q = np.asarray(codes, dtype=np.int8).astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    if q.ndim != 2 or s.shape != (q.shape[0],):
        raise ValueError("i8row: codes [rows, in] and scales [rows]")
    return s[:, None] * q


def i4_codes(packed: np.ndarray) -> np.ndarray:
    """Signed 4-bit codes of packed bytes (last axis): weight 2k is the low
    nibble of byte k, 2k + 1 the high nibble; nibbles 8..15 are -8..-1."""
    b = np.asarray(packed, dtype=np.uint8).astype(np.int64)
    lo, hi = b & 15, b >> 4
    q = np.stack([lo, hi], axis=-1).reshape(b.shape[:-1] + (2 * b.shape[-1],))
    return np.where(q >= 8, q - 16, q)


def dequant_i4row(packed, rows: int, in_features: int, scales) -> np.ndarray:
    """Per-row symmetric int4: w[o][i] = scale[o] * q[o][i].  float64."""
    if in_features % 32:
        raise ValueError("i4row needs in_features % 32 == 0")
    rb = row_bytes("i4row", in_features)
    b = np.asarray(packed, dtype=np.uint8).reshape(-1)
    if b.size != rows * rb:
        raise ValueError(f"i4row: expected {rows * rb} bytes, got {b.size}")
    q = i4_codes(b.reshape(rows, rb))[:, :in_features].astype(np.float64)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64)
    if s.shape != (rows,):
        raise ValueError("i4row: scales [rows]")
    return s[:, None] * q


def dequantize(fmt: str, packed, rows: int, in_features: int, scales=None) -> np.ndarray:
    """Exact float64 weights [rows, in_features] of a packed matrix."""
    if fmt == "q8_0":
        return dequant_q8_0(packed, rows, in_features)
    if fmt == "q2_k":
        return dequant_q2_k(packed, rows, in_features)
    if fmt == "q3_k":
        return dequant_q3_k(packed, rows, in_features)
    if fmt == "q4_k":
        return dequant_q4_k(packed, rows, in_features)
    if fmt == "q4_k_stream":
        return dequant_q4_k_stream(packed, rows, in_features)
    if fmt == "q5_k":
        return dequant_q5_k(packed, rows, in_features)
    if fmt == "q6_k":
        return dequant_q6_k(packed, rows, in_features)
    if fmt == "i8row":
        return dequant_i8row(np.asarray(packed).reshape(rows, in_features), scales)
    if fmt == "i4row":
        return dequant_i4row(packed, rows, in_features, scales)
    raise ValueError(f"unknown format {fmt!r}")


def dequantize_f32(fmt: str, packed, rows: int, in_features: int, scales=None) -> np.ndarray:
    """The float32 weights: the exact value rounded once to nearest-even."""
    return dequantize(fmt, packed, rows, in_features, scales).astype(np.float32)


# ---------------------------------------------------------------------------
# mat-vec / small-M matmul (float64)
# ---------------------------------------------------------------------------
def gemv(w64: np.ndarray, x, bias=None):
    """y[b, o] = sum_i w[o, i] * x[b, i] + bias[o], and the error scale
    s[b, o] = sum_i |w[o, i] * x[b, i]| + |bias[o]|.  x is [batch, in] (a 1-D
    x is one batch row).  Both results are float64 [batch, out]."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    y = x64 @ w64.T
    s = np.abs(x64) @ np.abs(w64).T
    if bias is not None:
        b64 = np.asarray(bias, dtype=np.float64)
        y = y + b64[None, :]
        s = s + np.abs(b64)[None, :]
    return y, s


def gemv_packed(fmt: str, packed, rows: int, in_features: int, x, bias=None,
                scales=None, row_chunk: int = 8192):
    """The quantized mat-vec y = W x + b from packed bytes: dequantize to
    float64, then a plain dot product, a chunk of rows at a time so that a
    large matrix never has to be expanded whole."""
    x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
    flat = np.asarray(packed).reshape(-1)
    ys, ss = [], []
    if fmt == "q4_k_stream":
        # chunks of whole super-blocks: a multiple of the rows that span one
        step = QK_K // math.gcd(in_features, QK_K)
        row_chunk = max(step, row_chunk // step * step)
    else:
        rb = row_bytes(fmt, in_features)
    for r0 in range(0, rows, row_chunk):
        r1 = min(rows, r0 + row_chunk)
        if fmt == "q4_k_stream":
            b0 = r0 * in_features // QK_K * BLOCK_BYTES["q4_k"]
            b1 = b0 + matrix_bytes(fmt, r1 - r0, in_features)
            w = dequant_q4_k_stream(flat[b0:b1], r1 - r0, in_features)
        elif fmt == "i8row":
            part = flat[r0 * in_features:r1 * in_features]
            w = dequant_i8row(part.view(np.int8).reshape(r1 - r0, in_features),
                              np.asarray(scales)[r0:r1])
        elif fmt == "i4row":
            w = dequant_i4row(flat[r0 * rb:r1 * rb], r1 - r0, in_features, np.asarray(scales)[r0:r1])
        else:
            w = dequantize(fmt, flat[r0 * rb:r1 * rb], r1 - r0, in_features)
        b = None if bias is None else np.asarray(bias)[r0:r1]
        y, s = gemv(w, x64, b)
        ys.append(y)
        ss.append(s)
    return np.concatenate(ys, axis=1), np.concatenate(ss, axis=1)


def gemm_f16(x16, w16, bias=None):
    """Small-M linear layer Y = X W^T + b with binary16 X [M, K] and W [N, K]
    (the same [out][in] orientation as the mat-vec rows), f32 bias [N].
    binary16 values are exact in float64, so are their products."""
    x64 = np.asarray(x16, dtype=np.float16).astype(np.float64)
    w64 = np.asarray(w16, dtype=np.float16).astype(np.float64)
    return gemv(w64, x64, bias)


def gemm_packed(fmt: str, packed, rows: int, in_features: int, x16, bias=None):
    """Small-M linear layer Y = X W^T + b at prompt width ("inferno" README,
    "Benchmarks") with W in a block format ("Project scaffold ...", quant.rs:
    the weights stay quantized): binary16 X [M, K], packed W [N rows].  The
    exact float64 weights times the exact float64 X - the same product as
    the mat-vec, with every row of X one batch row."""
    x64 = np.atleast_2d(np.asarray(x16, dtype=np.float16)).astype(np.float64)
    return gemv_packed(fmt, packed, rows, in_features, x64, bias)


def silu(g):
    """SiLU with the sigmoid: silu(g) = g * sigmoid(g) = g / (1 + e^-g)
    ("PESTI ..." README, "Conformance": SwiGLU = silu(gate) * up, the
    sigmoid-based SiLU, not silu squared).  float64."""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_packed(fmt: str, w_gate, w_up, rows: int, in_features: int, x,
                  gate_scales=None, up_scales=None):
    """The decode step's feed-forward input h = silu(W_gate x) * (W_up x)
    (same passage): the two quantized mat-vecs, then SiLU and the product,
    all in float64.  Returns h and the two mat-vecs' (value, error scale)
    pairs, from which a tolerance is derived."""
    g, sg = gemv_packed(fmt, w_gate, rows, in_features, x, None, gate_scales)
    u, su = gemv_packed(fmt, w_up, rows, in_features, x, None, up_scales)
    return silu(g) * u, (g, sg), (u, su)


def swiglu_tolerance(g, sg, u, su, h, rel: float = 1e-4, abs_: float = 1e-6):
    """Bound on |h_test - h| when g and u are each within rel * s + abs_:
    |silu'| <= 1.1 everywhere, so |dh| <= 1.1 eg |u| + |silu(g)| eu +
    2 eg eu, plus float32 rounding of the SiLU and the product."""
    eg = rel * np.asarray(sg) + abs_
    eu = rel * np.asarray(su) + abs_
    return 1.1 * eg * np.abs(u) + np.abs(silu(g)) * eu + 2.0 * eg * eu + 1e-6 * np.abs(h) + 1e-6


def within_tolerance(y_test, y_ref, s_ref, rel: float, abs_: float = 1e-6) -> np.ndarray:
    """Elementwise |y_test - y_ref| <= rel * s_ref + abs_ (s_ref from gemv)."""
    return np.abs(np.asarray(y_test, dtype=np.float64) - y_ref) <= rel * s_ref + abs_


# ---------------------------------------------------------------------------
# per-row symmetric int8 quantizer ("quant.rs" in ember PR #1)
# ---------------------------------------------------------------------------
def quantize_i4row(w):
    """Per-row symmetric int4 quantization of float32 weights [rows, in]
    (in % 32 == 0): scale = max|w| / 7 (as float32), q = round-half-away-
    from-zero(w / scale) clamped to [-7, 7]; a row of zeros gets scale 0 and
    codes 0.  Returns (packed uint8 [rows, row_bytes], float32 scales)."""
    w = np.asarray(w, dtype=np.float32)
    rows, n = w.shape
    amax = np.max(np.abs(w), axis=1) if n else np.zeros(rows, np.float32)
    scales = (amax.astype(np.float64) / 7.0).astype(np.float32)
    q = np.zeros((rows, -(-n // 64) * 64), dtype=np.int64)
    nz = scales > 0
    v = w[nz].astype(np.float64) / scales[nz, None].astype(np.float64)
    q[nz, :n] = np.clip(np.sign(v) * np.floor(np.abs(v) + 0.5), -7, 7)
    nib = q & 15
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    return packed, scales


def quantize_i8row(w):
    """Per-row symmetric int8 quantization of float32 weights [rows, in]:
    scale = max|w| / 127 (as float32), q = round-half-away-from-zero(w / scale)
    clamped to [-127, 127]; a row of zeros gets scale 0 and codes 0.
    Returns (int8 codes [rows, in], float32 scales [rows])."""
    w = np.asarray(w, dtype=np.float32)
    amax = np.max(np.abs(w), axis=1) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    scales = (amax.astype(np.float64) / 127.0).astype(np.float32)
    codes = np.zeros(w.shape, dtype=np.int8)
    nz = scales > 0
    v = w[nz].astype(np.float64) / scales[nz, None].astype(np.float64)
    q = np.sign(v) * np.floor(np.abs(v) + 0.5)
    codes[nz] = np.clip(q, -127, 127).astype(np.int8)
    return codes, scales
