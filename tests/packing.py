"""Field-level packers used only by the tests.

They build block bytes from explicit fields (d, dmin, scales, mins, codes),
in the forward direction, so that the oracle's unpacking can be checked
against fields that were never derived from the oracle itself.  The
arrangement is the GGUF block layout the pages name ("PESTI - Portable
Execution Substrate for Transformer Inference", section "What This Is").
"""
from __future__ import annotations

import numpy as np


def f16_bits(value: float) -> int:
    """binary16 bit pattern of a value (round to nearest-even)."""
    return int(np.array([value], dtype=np.float16).view(np.uint16)[0])


def _put_u16(buf: bytearray, off: int, bits: int) -> None:
    buf[off] = bits & 0xFF
    buf[off + 1] = (bits >> 8) & 0xFF


def pack_q8_0_block(d_bits: int, q) -> bytes:
    """34 bytes: binary16 d then 32 int8 codes."""
    q = [int(v) for v in q]
    assert len(q) == 32 and all(-128 <= v <= 127 for v in q)
    buf = bytearray(34)
    _put_u16(buf, 0, d_bits)
    for i, v in enumerate(q):
        buf[2 + i] = v & 0xFF
    return bytes(buf)


def pack_q4_k_scales(sc, m) -> bytes:
    """Twelve bytes holding eight 6-bit scales and eight 6-bit mins.
    Bytes 0-3: scale j (j < 4) in bits 0-5, and bits 4-5 of scale j+4 in
    bits 6-7.  Bytes 4-7: the same for the mins.  Bytes 8-11: bits 0-3 of
    scale j+4 in the low nibble, bits 0-3 of min j+4 in the high nibble."""
    assert len(sc) == 8 and len(m) == 8
    assert all(0 <= v < 64 for v in list(sc) + list(m))
    out = bytearray(12)
    for j in range(4):
        hi_sc = (sc[j + 4] >> 4) & 3
        hi_m = (m[j + 4] >> 4) & 3
        out[j] = sc[j] | (hi_sc << 6)
        out[4 + j] = m[j] | (hi_m << 6)
        out[8 + j] = (sc[j + 4] & 0xF) | ((m[j + 4] & 0xF) << 4)
    return bytes(out)


def pack_q4_k_block(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """144 bytes: d, dmin, packed scales/mins, 128 code bytes.  Codes come in
    runs of 64 weights; run r lives in bytes 32r..32r+31, its first half in
    the low nibbles and its second half in the high nibbles."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 16 for v in q)
    buf = bytearray(144)
    _put_u16(buf, 0, d_bits)
    _put_u16(buf, 2, dmin_bits)
    buf[4:16] = pack_q4_k_scales(sc, m)
    for r in range(4):
        for l in range(32):
            buf[16 + 32 * r + l] = q[64 * r + l] | (q[64 * r + 32 + l] << 4)
    return bytes(buf)


def pack_q5_k_block(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """176 bytes: d, dmin, packed scales/mins (as Q4_K), 32 high-bit bytes,
    128 low-nibble bytes.  Weight 64r + 32c + l (l < 32) keeps its low four
    bits in the low (c = 0) or high (c = 1) nibble of low byte 32r + l, and
    its fifth bit at bit 2r + c of high-bit byte l."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 32 for v in q)
    buf = bytearray(176)
    _put_u16(buf, 0, d_bits)
    _put_u16(buf, 2, dmin_bits)
    buf[4:16] = pack_q4_k_scales(sc, m)
    for r in range(4):
        for c in range(2):
            for l in range(32):
                v = q[64 * r + 32 * c + l]
                buf[48 + 32 * r + l] |= (v & 0xF) << (4 * c)
                buf[16 + l] |= (v >> 4) << (2 * r + c)
    return bytes(buf)


def pack_q2_k_block(d_bits: int, dmin_bits: int, sc, m, q) -> bytes:
    """84 bytes: 16 scale bytes (scale | min << 4, one per 16-weight
    sub-block), 64 code bytes, d, dmin.  Weight 128h + 32j + 16c + l keeps
    its 2-bit code at bit 2j of code byte 32h + 16c + l."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 4 for v in q)
    assert len(sc) == 16 and len(m) == 16 and all(0 <= v < 16 for v in list(sc) + list(m))
    buf = bytearray(84)
    for s in range(16):
        buf[s] = sc[s] | (m[s] << 4)
    for h in range(2):
        for j in range(4):
            for c in range(2):
                for l in range(16):
                    buf[16 + 32 * h + 16 * c + l] |= q[128 * h + 32 * j + 16 * c + l] << (2 * j)
    _put_u16(buf, 80, d_bits)
    _put_u16(buf, 82, dmin_bits)
    return bytes(buf)


def pack_q3_k_block(d_bits: int, scales, q) -> bytes:
    """110 bytes: 32 high-bit bytes, 64 low-bit bytes, 12 scale bytes, d.
    A code q in -4..3 is stored as its low two bits (q, or q + 4 when
    negative) at bit 2j of byte 32h + 16c + l and a high bit (set when
    q >= 0) at bit 4h + j of high-bit byte 16c + l.  Scale k (0..63) keeps
    bits 0-3 at bit 4(k // 8) of byte k % 8 and bits 4-5 at bit 2(k // 4) of
    byte 8 + k % 4."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(-4 <= v <= 3 for v in q)
    assert len(scales) == 16 and all(0 <= v < 64 for v in scales)
    buf = bytearray(110)
    for h in range(2):
        for j in range(4):
            for c in range(2):
                for l in range(16):
                    v = q[128 * h + 32 * j + 16 * c + l]
                    buf[32 + 32 * h + 16 * c + l] |= (v if v >= 0 else v + 4) << (2 * j)
                    if v >= 0:
                        buf[16 * c + l] |= 1 << (4 * h + j)
    for k in range(16):
        buf[96 + k % 8] |= (scales[k] & 15) << (4 * (k // 8))
        buf[96 + 8 + k % 4] |= (scales[k] >> 4) << (2 * (k // 4))
    _put_u16(buf, 108, d_bits)
    return bytes(buf)


def pack_q6_k_block(d_bits: int, sc, q) -> bytes:
    """210 bytes: 128 low-part bytes, 64 high-part bytes, 16 int8 scales, d.
    Weight i = 128h + 32g + l keeps its low four bits in the low (g < 2) or
    high (g >= 2) nibble of low-part byte 64h + 32(g % 2) + l, and its top two
    bits at bit 2g of high-part byte 32h + l."""
    q = [int(v) for v in q]
    assert len(q) == 256 and all(0 <= v < 64 for v in q)
    assert len(sc) == 16 and all(-128 <= v <= 127 for v in sc)
    ql = [0] * 128
    qh = [0] * 64
    for h in range(2):
        for g in range(4):
            for l in range(32):
                v = q[128 * h + 32 * g + l]
                shift = 4 if g >= 2 else 0
                ql[64 * h + 32 * (g % 2) + l] |= (v & 0xF) << shift
                qh[32 * h + l] |= (v >> 4) << (2 * g)
    buf = bytearray(210)
    buf[0:128] = bytes(ql)
    buf[128:192] = bytes(qh)
    buf[192:208] = bytes(int(v) & 0xFF for v in sc)
    _put_u16(buf, 208, d_bits)
    return bytes(buf)


def rows_to_array(rows_of_blocks) -> np.ndarray:
    """[[block bytes, ...] per row] -> uint8 [rows, row_bytes]."""
    return np.array([np.frombuffer(b"".join(r), dtype=np.uint8) for r in rows_of_blocks])


def pack_i4_row(q) -> bytes:
    """Bytes of one int4 row: codes -8..7 as 4-bit two's complement, weight
    2k in the low nibble of byte k, 2k + 1 in the high nibble, the row
    padded with zero codes to a multiple of 64 weights."""
    q = [int(v) for v in q]
    assert all(-8 <= v <= 7 for v in q)
    q = q + [0] * (-len(q) % 64)
    return bytes(((q[2 * k] & 15) | ((q[2 * k + 1] & 15) << 4)) for k in range(len(q) // 2))
