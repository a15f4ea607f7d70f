"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself:
* hand-worked fixtures under tests/golden/ (values derived by hand from the
  block definitions, with the derivation in each file);
* fields packed by an independent forward packer (tests/packing.py) and the
  closed forms w = d*sc*q - dmin*m (Q4_K, Q5_K), d*sc*(q-32) (Q6_K), d*q (Q8_0),
  scale*q (int8) evaluated in exact rationals;
* one-hot codes, which pin each weight's position;
* exact rational mat-vec (brute force) on 4x32 .. 8x256 matrices;
* special cases (zero codes, zero scales, q = 32, zero d, subnormal d);
* reductions to textbook operations (integer matrix product, identity).
A set of planted mistakes checks that the pins catch plausible bugs.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import pytest

import golden_io
import packing
import oracle

GEMV_REL = 1e-4
GEMM_REL = 2e-3


# ---------------------------------------------------------------------------
# helpers: exact values from explicit fields
# ---------------------------------------------------------------------------
def f16_value(bits: int) -> Fraction:
    return Fraction(float(np.array([bits], dtype=np.uint16).view(np.float16)[0]))


def random_f16_bits(rng, n):
    """binary16 patterns spanning zero, subnormals, normals and the maximum."""
    special = [0x0000, 0x0001, 0x03FF, 0x0400, 0x3C00, 0x7BFF, 0x1234]
    out = []
    for _ in range(n):
        if rng.random() < 0.3:
            out.append(int(rng.choice(special)))
        else:
            out.append(int(rng.integers(0, 0x7C00)))   # finite, non-negative
    return out


def q4_k_exact(d_bits, dmin_bits, sc, m, q):
    d, dmin = f16_value(d_bits), f16_value(dmin_bits)
    return [d * sc[i // 32] * q[i] - dmin * m[i // 32] for i in range(256)]


def q6_k_exact(d_bits, sc, q):
    d = f16_value(d_bits)
    return [d * sc[i // 16] * (q[i] - 32) for i in range(256)]


def q8_0_exact(d_bits, q):
    d = f16_value(d_bits)
    return [d * v for v in q]


def random_q4_k_fields(rng):
    return (random_f16_bits(rng, 1)[0], random_f16_bits(rng, 1)[0],
            [int(v) for v in rng.integers(0, 64, 8)], [int(v) for v in rng.integers(0, 64, 8)],
            [int(v) for v in rng.integers(0, 16, 256)])


def random_q5_k_fields(rng):
    return (random_f16_bits(rng, 1)[0], random_f16_bits(rng, 1)[0],
            [int(v) for v in rng.integers(0, 64, 8)], [int(v) for v in rng.integers(0, 64, 8)],
            [int(v) for v in rng.integers(0, 32, 256)])


def q2_k_exact(d_bits, dmin_bits, sc, m, q):
    d, dmin = f16_value(d_bits), f16_value(dmin_bits)
    return [d * sc[i // 16] * q[i] - dmin * m[i // 16] for i in range(256)]


def q3_k_exact(d_bits, scales, q):
    d = f16_value(d_bits)
    return [d * (scales[i // 16] - 32) * q[i] for i in range(256)]


def random_q2_k_fields(rng):
    return (random_f16_bits(rng, 1)[0], random_f16_bits(rng, 1)[0],
            [int(v) for v in rng.integers(0, 16, 16)], [int(v) for v in rng.integers(0, 16, 16)],
            [int(v) for v in rng.integers(0, 4, 256)])


def random_q3_k_fields(rng):
    return (random_f16_bits(rng, 1)[0], [int(v) for v in rng.integers(0, 64, 16)],
            [int(v) for v in rng.integers(-4, 4, 256)])


def random_q6_k_fields(rng):
    return (random_f16_bits(rng, 1)[0], [int(v) for v in rng.integers(-128, 128, 16)],
            [int(v) for v in rng.integers(0, 64, 256)])


def random_q8_0_fields(rng):
    return random_f16_bits(rng, 1)[0], [int(v) for v in rng.integers(-128, 128, 32)]


def as_fraction_array(w):
    return [Fraction(float(v)) for v in np.asarray(w).reshape(-1)]


# ---------------------------------------------------------------------------
# 1. hand-worked fixtures
# ---------------------------------------------------------------------------
def check_dequant_fixture(name: str) -> bool:
    fx = golden_io.load(name)
    if "f64" not in fx:
        return True
    data, scales = golden_io.packed(fx)
    w = oracle.dequantize(fx["format"], data, fx["rows"], fx["in_features"], scales)
    ok = w.shape == (fx["rows"], fx["in_features"])
    ok = ok and np.array_equal(w.reshape(-1), fx["f64"])
    f32_expect = fx.get("f32", fx["f64"]).astype(np.float32)
    w32 = oracle.dequantize_f32(fx["format"], data, fx["rows"], fx["in_features"], scales)
    return bool(ok and np.array_equal(w32.reshape(-1), f32_expect))


def check_gemv_fixture(name: str) -> bool:
    fx = golden_io.load(name)
    if "y" not in fx:
        return True
    data, scales = golden_io.packed(fx)
    y, s = oracle.gemv_packed(fx["format"], data, fx["rows"], fx["in_features"],
                              fx["x"].astype(np.float32), fx["bias"].astype(np.float32), scales)
    return bool(np.array_equal(y.reshape(-1), fx["y"]))


@pytest.mark.parametrize("name", golden_io.all_fixtures())
def test_golden_fixture(name):
    assert check_dequant_fixture(name), name
    assert check_gemv_fixture(name), name


def test_fixture_set_covers_every_format():
    fmts = {golden_io.load(n)["format"] for n in golden_io.all_fixtures()}
    assert fmts == {"q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k", "q4_k_stream", "i8row", "i4row"}


# ---------------------------------------------------------------------------
# 2. independent packer -> oracle unpack == fields; closed forms, exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(6))
def test_q4_k_fields_and_closed_form(seed):
    rng = np.random.default_rng([1, seed])
    blocks, exact = [], []
    for _ in range(8):
        d, dmin, sc, m, q = random_q4_k_fields(rng)
        blocks.append(packing.pack_q4_k_block(d, dmin, sc, m, q))
        exact.extend(q4_k_exact(d, dmin, sc, m, q))
        # field-level round trip through the oracle's unpackers
        raw = np.frombuffer(blocks[-1], dtype=np.uint8)
        sc_o, m_o = oracle.q4_k_scales_mins(raw[4:16])
        assert list(sc_o) == sc and list(m_o) == m
        assert list(oracle.q4_k_codes(raw[16:144])) == q
    data = packing.rows_to_array([blocks[:4], blocks[4:]])
    w = oracle.dequant_q4_k(data, 2, 1024)
    assert as_fraction_array(w) == exact


@pytest.mark.parametrize("seed", range(6))
def test_q2_k_fields_and_closed_form(seed):
    rng = np.random.default_rng([23, seed])
    blocks, exact = [], []
    for _ in range(6):
        d, dmin, sc, m, q = random_q2_k_fields(rng)
        blocks.append(packing.pack_q2_k_block(d, dmin, sc, m, q))
        exact.extend(q2_k_exact(d, dmin, sc, m, q))
        raw = np.frombuffer(blocks[-1], dtype=np.uint8)
        assert list(oracle.q2_k_codes(raw[16:80])) == q
    data = packing.rows_to_array([blocks[:3], blocks[3:]])
    assert as_fraction_array(oracle.dequant_q2_k(data, 2, 768)) == exact


@pytest.mark.parametrize("seed", range(6))
def test_q3_k_fields_and_closed_form(seed):
    rng = np.random.default_rng([24, seed])
    blocks, exact = [], []
    for _ in range(6):
        d, scales, q = random_q3_k_fields(rng)
        blocks.append(packing.pack_q3_k_block(d, scales, q))
        exact.extend(q3_k_exact(d, scales, q))
        raw = np.frombuffer(blocks[-1], dtype=np.uint8)
        assert list(oracle.q3_k_scales(raw[96:108])) == scales
        assert list(oracle.q3_k_codes(raw[0:32], raw[32:96])) == q
    data = packing.rows_to_array([blocks[:3], blocks[3:]])
    assert as_fraction_array(oracle.dequant_q3_k(data, 2, 768)) == exact


def test_q3_k_scale_extremes_round_trip():
    for k in range(16):
        sc_in = [63 if i == k else 0 for i in range(16)]
        raw = np.frombuffer(packing.pack_q3_k_block(0x3C00, sc_in, [0] * 256), dtype=np.uint8)
        assert list(oracle.q3_k_scales(raw[96:108])) == sc_in


@pytest.mark.parametrize("seed", range(6))
def test_q5_k_fields_and_closed_form(seed):
    rng = np.random.default_rng([21, seed])
    blocks, exact = [], []
    for _ in range(6):
        d, dmin, sc, m, q = random_q5_k_fields(rng)
        blocks.append(packing.pack_q5_k_block(d, dmin, sc, m, q))
        exact.extend(q4_k_exact(d, dmin, sc, m, q))   # same closed form, q in 0..31
        raw = np.frombuffer(blocks[-1], dtype=np.uint8)
        sc_o, m_o = oracle.q4_k_scales_mins(raw[4:16])
        assert list(sc_o) == sc and list(m_o) == m
        assert list(oracle.q5_k_codes(raw[16:48], raw[48:176])) == q
    data = packing.rows_to_array([blocks[:3], blocks[3:]])
    w = oracle.dequant_q5_k(data, 2, 768)
    assert as_fraction_array(w) == exact


@pytest.mark.parametrize("seed", range(6))
def test_q6_k_fields_and_closed_form(seed):
    rng = np.random.default_rng([2, seed])
    blocks, exact = [], []
    for _ in range(6):
        d, sc, q = random_q6_k_fields(rng)
        blocks.append(packing.pack_q6_k_block(d, sc, q))
        exact.extend(q6_k_exact(d, sc, q))
        raw = np.frombuffer(blocks[-1], dtype=np.uint8)
        assert list(oracle.q6_k_codes(raw[0:128], raw[128:192])) == q
    data = packing.rows_to_array([blocks[:3], blocks[3:]])
    w = oracle.dequant_q6_k(data, 2, 768)
    assert as_fraction_array(w) == exact


@pytest.mark.parametrize("seed", range(4))
def test_q8_0_closed_form(seed):
    rng = np.random.default_rng([3, seed])
    blocks, exact = [], []
    for _ in range(12):
        d, q = random_q8_0_fields(rng)
        blocks.append(packing.pack_q8_0_block(d, q))
        exact.extend(q8_0_exact(d, q))
    data = packing.rows_to_array([blocks[:4], blocks[4:8], blocks[8:]])
    w = oracle.dequant_q8_0(data, 3, 128)
    assert as_fraction_array(w) == exact


def test_field_extremes_round_trip():
    """All-zero and all-maximal fields, and each scale/min alone at 63."""
    for val in (0, 63):
        raw = np.frombuffer(packing.pack_q4_k_scales([val] * 8, [63 - val] * 8), dtype=np.uint8)
        sc, m = oracle.q4_k_scales_mins(raw)
        assert list(sc) == [val] * 8 and list(m) == [63 - val] * 8
    for j in range(8):
        sc_in = [63 if k == j else 0 for k in range(8)]
        m_in = [0 if k == j else 63 for k in range(8)]
        raw = np.frombuffer(packing.pack_q4_k_scales(sc_in, m_in), dtype=np.uint8)
        sc, m = oracle.q4_k_scales_mins(raw)
        assert list(sc) == sc_in and list(m) == m_in


# ---------------------------------------------------------------------------
# 3. one-hot codes pin every weight's position
# ---------------------------------------------------------------------------
def test_q4_k_one_hot_positions():
    sc = [1, 2, 3, 4, 5, 6, 7, 8]
    for i in range(256):
        q = [0] * 256
        q[i] = 9
        blk = packing.pack_q4_k_block(0x3C00, 0x0000, sc, [5] * 8, q)
        w = oracle.dequant_q4_k(np.frombuffer(blk, dtype=np.uint8), 1, 256)[0]
        nz = np.flatnonzero(w)
        assert list(nz) == [i] and w[i] == 9 * sc[i // 32], i


def test_q5_k_one_hot_positions():
    """Code 25 (fifth bit set, low nibble 9) at one position, zero elsewhere."""
    sc = [1, 2, 3, 4, 5, 6, 7, 8]
    for i in range(256):
        q = [0] * 256
        q[i] = 25
        blk = packing.pack_q5_k_block(0x3C00, 0x0000, sc, [5] * 8, q)
        w = oracle.dequant_q5_k(np.frombuffer(blk, dtype=np.uint8), 1, 256)[0]
        nz = np.flatnonzero(w)
        assert list(nz) == [i] and w[i] == 25 * sc[i // 32], i


def test_q2_k_one_hot_positions():
    sc = [min(k + 1, 15) for k in range(16)]
    for i in range(256):
        q = [0] * 256
        q[i] = 3
        blk = packing.pack_q2_k_block(0x3C00, 0x3C00, sc, [0] * 16, q)
        w = oracle.dequant_q2_k(np.frombuffer(blk, dtype=np.uint8), 1, 256)[0]
        assert list(np.flatnonzero(w)) == [i] and w[i] == 3 * sc[i // 16], i


def test_q3_k_one_hot_positions():
    """Code 0 everywhere (high bit set, low bits 0) but -3 at one position."""
    scales = [33 + k for k in range(16)]     # scale - 32 = 1 .. 16
    for i in range(256):
        q = [0] * 256
        q[i] = -3
        blk = packing.pack_q3_k_block(0x3C00, scales, q)
        w = oracle.dequant_q3_k(np.frombuffer(blk, dtype=np.uint8), 1, 256)[0]
        assert list(np.flatnonzero(w)) == [i] and w[i] == -3 * (scales[i // 16] - 32), i


def test_q6_k_one_hot_positions():
    sc = list(range(1, 17))
    for i in range(256):
        q = [32] * 256          # q = 32 dequantizes to exactly 0
        q[i] = 45
        blk = packing.pack_q6_k_block(0x3C00, sc, q)
        w = oracle.dequant_q6_k(np.frombuffer(blk, dtype=np.uint8), 1, 256)[0]
        nz = np.flatnonzero(w)
        assert list(nz) == [i] and w[i] == 13 * sc[i // 16], i


def test_q8_0_one_hot_positions():
    for i in range(32):
        q = [0] * 32
        q[i] = -7
        blk = packing.pack_q8_0_block(0x4000, q)   # d = 2
        w = oracle.dequant_q8_0(np.frombuffer(blk, dtype=np.uint8), 1, 32)[0]
        assert list(np.flatnonzero(w)) == [i] and w[i] == -14


# ---------------------------------------------------------------------------
# 4. special cases
# ---------------------------------------------------------------------------
def test_q4_k_special_cases():
    rng = np.random.default_rng(7)
    _, _, sc, m, q = random_q4_k_fields(rng)
    d, dmin = 0x3555, 0x2AAA
    # q = 0 -> -dmin*m
    w = oracle.dequant_q4_k(np.frombuffer(packing.pack_q4_k_block(d, dmin, sc, m, [0] * 256), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [-f16_value(dmin) * m[i // 32] for i in range(256)]
    # sc = 0 -> constant -dmin*m per sub-block, whatever the codes
    w = oracle.dequant_q4_k(np.frombuffer(packing.pack_q4_k_block(d, dmin, [0] * 8, m, q), np.uint8), 1, 256)[0]
    for j in range(8):
        assert np.all(w[32 * j:32 * j + 32] == w[32 * j])
    # d = 0 -> -dmin*m
    w = oracle.dequant_q4_k(np.frombuffer(packing.pack_q4_k_block(0, dmin, sc, m, q), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [-f16_value(dmin) * m[i // 32] for i in range(256)]
    # subnormal d: w = 2^-24 * sc * q exactly
    w = oracle.dequant_q4_k(np.frombuffer(packing.pack_q4_k_block(0x0001, 0, sc, m, q), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [Fraction(1, 2 ** 24) * sc[i // 32] * q[i] for i in range(256)]


def test_q5_k_special_cases():
    rng = np.random.default_rng(22)
    _, _, sc, m, q = random_q5_k_fields(rng)
    d, dmin = 0x3555, 0x2AAA
    pack = packing.pack_q5_k_block
    # q = 0 -> -dmin*m; q = 16 (fifth bit alone) -> 16 d sc - dmin m
    for qv in (0, 16, 31):
        w = oracle.dequant_q5_k(np.frombuffer(pack(d, dmin, sc, m, [qv] * 256), np.uint8), 1, 256)[0]
        assert as_fraction_array(w) == [f16_value(d) * sc[i // 32] * qv - f16_value(dmin) * m[i // 32]
                                        for i in range(256)]
    # the fifth bit of code q equals 16 * (q >> 4) on top of the Q4_K decode of the low nibbles
    blk = np.frombuffer(pack(0x3C00, 0, sc, m, q), np.uint8)
    low = [v & 15 for v in q]
    blk4 = np.frombuffer(packing.pack_q4_k_block(0x3C00, 0, sc, m, low), np.uint8)
    w5 = oracle.dequant_q5_k(blk, 1, 256)[0]
    w4 = oracle.dequant_q4_k(blk4, 1, 256)[0]
    assert np.array_equal(w5 - w4, np.array([16 * sc[i // 32] * (q[i] >> 4) for i in range(256)], float))
    # subnormal d: w = 2^-24 * sc * q exactly
    w = oracle.dequant_q5_k(np.frombuffer(pack(0x0001, 0, sc, m, q), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [Fraction(1, 2 ** 24) * sc[i // 32] * q[i] for i in range(256)]


def test_q2_k_q3_k_special_cases():
    rng = np.random.default_rng(25)
    _, _, sc, m, q = random_q2_k_fields(rng)
    # Q2_K: codes 0 -> -dmin*m; scale 0 -> constant -dmin*m per sub-block
    w = oracle.dequant_q2_k(np.frombuffer(packing.pack_q2_k_block(0x3555, 0x2AAA, sc, m, [0] * 256),
                                          np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [-f16_value(0x2AAA) * m[i // 16] for i in range(256)]
    w = oracle.dequant_q2_k(np.frombuffer(packing.pack_q2_k_block(0x3555, 0x2AAA, [0] * 16, m, q),
                                          np.uint8), 1, 256)[0]
    for s in range(16):
        assert np.all(w[16 * s:16 * s + 16] == w[16 * s])
    # Q3_K: scale 32 -> 0 whatever the codes; code -4 (all bits clear) -> -4 d (scale - 32)
    _, scales, q3 = random_q3_k_fields(rng)
    w = oracle.dequant_q3_k(np.frombuffer(packing.pack_q3_k_block(0x3C00, [32] * 16, q3), np.uint8), 1, 256)[0]
    assert np.all(w == 0)
    raw = bytearray(110)
    raw[96:108] = packing.pack_q3_k_block(0x3C00, scales, [0] * 256)[96:108]
    raw[108:110] = bytes([0x00, 0x3C])
    w = oracle.dequant_q3_k(np.frombuffer(bytes(raw), np.uint8), 1, 256)[0]
    assert list(w) == [-4.0 * (scales[i // 16] - 32) for i in range(256)]
    # subnormal d
    w = oracle.dequant_q3_k(np.frombuffer(packing.pack_q3_k_block(0x0001, scales, q3), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [Fraction(1, 2 ** 24) * (scales[i // 16] - 32) * q3[i] for i in range(256)]


def test_q6_k_special_cases():
    rng = np.random.default_rng(8)
    _, sc, q = random_q6_k_fields(rng)
    w = oracle.dequant_q6_k(np.frombuffer(packing.pack_q6_k_block(0x3C00, sc, [32] * 256), np.uint8), 1, 256)[0]
    assert np.all(w == 0)
    w = oracle.dequant_q6_k(np.frombuffer(packing.pack_q6_k_block(0, sc, q), np.uint8), 1, 256)[0]
    assert np.all(w == 0)
    w = oracle.dequant_q6_k(np.frombuffer(packing.pack_q6_k_block(0x0001, sc, q), np.uint8), 1, 256)[0]
    assert as_fraction_array(w) == [Fraction(1, 2 ** 24) * sc[i // 16] * (q[i] - 32) for i in range(256)]


def test_q8_0_special_cases():
    rng = np.random.default_rng(9)
    _, q = random_q8_0_fields(rng)
    w = oracle.dequant_q8_0(np.frombuffer(packing.pack_q8_0_block(0, q), np.uint8), 1, 32)[0]
    assert np.all(w == 0)
    w = oracle.dequant_q8_0(np.frombuffer(packing.pack_q8_0_block(0x7BFF, [-128] * 32), np.uint8), 1, 32)[0]
    assert np.all(w == -65504.0 * 128)


# ---------------------------------------------------------------------------
# 5. padding columns are dropped and their bytes do not matter
# ---------------------------------------------------------------------------
def _padding_masks_in128():
    """Byte masks (bit set = may change) of what only weights 128..255 use."""
    q4 = np.zeros(144, dtype=np.uint8)
    q4[4:8] = 0xC0          # top bits of scales 4..7
    q4[8:12] = 0xC0         # top bits of mins 4..7
    q4[12:16] = 0xFF        # low bits of scales/mins 4..7
    q4[16 + 64:144] = 0xFF  # code runs 2 and 3
    q6 = np.zeros(210, dtype=np.uint8)
    q6[64:128] = 0xFF       # low parts of h = 1
    q6[128 + 32:192] = 0xFF  # high parts of h = 1
    q6[192 + 8:208] = 0xFF  # scales of sub-blocks 8..15
    q5 = np.zeros(176, dtype=np.uint8)
    q5[4:16] = q4[4:16]     # the same scale/min bits as Q4_K
    q5[16:48] = 0xF0        # fifth bits of runs 2 and 3
    q5[48 + 64:176] = 0xFF  # low-nibble runs 2 and 3
    q2 = np.zeros(84, dtype=np.uint8)
    q2[8:16] = 0xFF         # scale/min bytes of sub-blocks 8..15
    q2[16 + 32:80] = 0xFF   # code bytes of h = 1
    q3 = np.zeros(110, dtype=np.uint8)
    q3[0:32] = 0xF0         # high bits of h = 1
    q3[32 + 32:96] = 0xFF   # low-bit bytes of h = 1
    q3[96:104] = 0xF0       # low scale bits of sub-blocks 8..15
    q3[104:108] = 0xF0      # high scale bits of sub-blocks 8..15
    return {"q2_k": q2, "q3_k": q3, "q4_k": q4, "q5_k": q5, "q6_k": q6}


@pytest.mark.parametrize("fmt", ["q2_k", "q3_k", "q4_k", "q5_k", "q6_k"])
def test_padding_bytes_do_not_matter(fmt):
    rng = np.random.default_rng(11)
    mask = _padding_masks_in128()[fmt]
    nb = oracle.BLOCK_BYTES[fmt]
    base = rng.integers(0, 256, size=(3, nb), dtype=np.uint8)
    d_off = {"q6_k": 208, "q2_k": 80, "q3_k": 108}.get(fmt, 0)
    base[:, d_off:d_off + 2] = [0x00, 0x3C]           # d = 1.0
    w0 = oracle.dequantize(fmt, base, 3, 128)
    assert w0.shape == (3, 128)
    for trial in range(5):
        noise = rng.integers(0, 256, size=base.shape, dtype=np.uint8) & mask
        alt = (base & ~mask) | noise
        assert np.array_equal(oracle.dequantize(fmt, alt, 3, 128), w0)
    # and the kept columns equal the full-block decode's first 128 columns
    assert np.array_equal(w0, oracle.dequantize(fmt, base, 3, 256)[:, :128])


# ---------------------------------------------------------------------------
# 6. brute force: exact rational mat-vec from the fields
# ---------------------------------------------------------------------------
def _exact_gemv(w_exact_rows, x, bias):
    out = []
    for b in range(x.shape[0]):
        row = []
        for o, wrow in enumerate(w_exact_rows):
            acc = sum((wv * Fraction(float(xv)) for wv, xv in zip(wrow, x[b])), Fraction(0))
            if bias is not None:
                acc += Fraction(float(bias[o]))
            row.append(acc)
        out.append(row)
    return out


def _build(fmt, rng, rows, in_features):
    """Packed matrix and its exact weights from random fields."""
    qk = 32 if fmt == "q8_0" else 256
    nblk = -(-in_features // qk)
    packed_rows, exact_rows = [], []
    for _ in range(rows):
        blocks, exact = [], []
        for _ in range(nblk):
            if fmt == "q8_0":
                d, q = random_q8_0_fields(rng)
                blocks.append(packing.pack_q8_0_block(d, q))
                exact += q8_0_exact(d, q)
            elif fmt == "q4_k":
                d, dmin, sc, m, q = random_q4_k_fields(rng)
                blocks.append(packing.pack_q4_k_block(d, dmin, sc, m, q))
                exact += q4_k_exact(d, dmin, sc, m, q)
            elif fmt == "q2_k":
                d, dmin, sc, m, q = random_q2_k_fields(rng)
                blocks.append(packing.pack_q2_k_block(d, dmin, sc, m, q))
                exact += q2_k_exact(d, dmin, sc, m, q)
            elif fmt == "q3_k":
                d, scales, q = random_q3_k_fields(rng)
                blocks.append(packing.pack_q3_k_block(d, scales, q))
                exact += q3_k_exact(d, scales, q)
            elif fmt == "q5_k":
                d, dmin, sc, m, q = random_q5_k_fields(rng)
                blocks.append(packing.pack_q5_k_block(d, dmin, sc, m, q))
                exact += q4_k_exact(d, dmin, sc, m, q)
            else:
                d, sc, q = random_q6_k_fields(rng)
                blocks.append(packing.pack_q6_k_block(d, sc, q))
                exact += q6_k_exact(d, sc, q)
        packed_rows.append(blocks)
        exact_rows.append(exact[:in_features])
    return packing.rows_to_array(packed_rows), exact_rows


BRUTE_CASES = [("q8_0", 4, 32), ("q8_0", 8, 64), ("q4_k", 4, 256), ("q4_k", 8, 256),
               ("q6_k", 4, 256), ("q6_k", 8, 256), ("q4_k", 4, 128), ("q6_k", 4, 128),
               ("q4_k", 3, 384), ("q5_k", 4, 256), ("q5_k", 3, 384), ("q5_k", 4, 128),
               ("q2_k", 4, 256), ("q2_k", 3, 384), ("q3_k", 4, 256), ("q3_k", 3, 384)]


@pytest.mark.parametrize("fmt,rows,inf", BRUTE_CASES)
def test_gemv_brute_force(fmt, rows, inf):
    rng = np.random.default_rng([4, rows, inf])
    data, exact_w = _build(fmt, rng, rows, inf)
    x = rng.standard_normal((2, inf)).astype(np.float32)
    bias = rng.normal(0, 0.02, rows).astype(np.float32)
    y, s = oracle.gemv_packed(fmt, data, rows, inf, x, bias)
    ex = _exact_gemv(exact_w, x, bias)
    assert y.shape == (2, rows)
    for b in range(2):
        for o in range(rows):
            err = abs(Fraction(float(y[b, o])) - ex[b][o])
            assert err <= Fraction(2.0 ** -50) * Fraction(float(s[b, o])) + Fraction(1, 2 ** 200), (b, o)
            # the error scale is sum |w x| + |b| itself
            ref_s = sum(abs(wv * Fraction(float(xv))) for wv, xv in zip(exact_w[o], x[b])) \
                + abs(Fraction(float(bias[o])))
            assert abs(Fraction(float(s[b, o])) - ref_s) <= Fraction(2.0 ** -48) * ref_s


@pytest.mark.parametrize("rows,inf", [(4, 32), (8, 64)])
def test_i8row_brute_force(rows, inf):
    rng = np.random.default_rng([5, rows])
    codes = rng.integers(-127, 128, size=(rows, inf)).astype(np.int8)
    scales = (rng.random(rows) * 0.01).astype(np.float32)
    x = rng.standard_normal((3, inf)).astype(np.float32)
    y, s = oracle.gemv_packed("i8row", codes.view(np.uint8), rows, inf, x, None, scales)
    for b in range(3):
        for o in range(rows):
            ex = sum(Fraction(float(scales[o])) * int(codes[o, i]) * Fraction(float(x[b, i]))
                     for i in range(inf))
            assert abs(Fraction(float(y[b, o])) - ex) <= Fraction(2.0 ** -50) * Fraction(float(s[b, o]))


# ---------------------------------------------------------------------------
# 7. textbook reductions
# ---------------------------------------------------------------------------
def test_i8row_unit_scale_is_integer_matmul():
    rng = np.random.default_rng(12)
    codes = rng.integers(-127, 128, size=(16, 96)).astype(np.int8)
    xi = rng.integers(-1000, 1000, size=(2, 96))
    y, _ = oracle.gemv_packed("i8row", codes.view(np.uint8), 16, 96, xi.astype(np.float32),
                              None, np.ones(16, np.float32))
    assert np.array_equal(y, (xi @ codes.astype(np.int64).T).astype(np.float64))


def test_gemm_f16_identity_and_brute_force():
    rng = np.random.default_rng(13)
    w = rng.normal(0, 0.02, size=(5, 8)).astype(np.float16)
    bias = rng.normal(0, 0.02, 5).astype(np.float32)
    eye = np.eye(8, dtype=np.float16)[:3]
    y, _ = oracle.gemm_f16(eye, w, bias)
    for m in range(3):
        assert np.array_equal(y[m], w[:, m].astype(np.float64) + bias.astype(np.float64))
    x = rng.standard_normal((3, 8)).astype(np.float16)
    y, s = oracle.gemm_f16(x, w, bias)
    for m in range(3):
        for n in range(5):
            ex = sum(Fraction(float(x[m, k])) * Fraction(float(w[n, k])) for k in range(8)) \
                + Fraction(float(bias[n]))
            assert abs(Fraction(float(y[m, n])) - ex) <= Fraction(2.0 ** -50) * Fraction(float(s[m, n]))


def test_gemm_packed_unit_rows_pick_columns():
    """Rows of X that are unit vectors pick columns of W: Y[m] = W[:, k_m] + b,
    with W from the field-level decode (orientation and the f16 X path)."""
    rng = np.random.default_rng(14)
    for fmt, rows, inf in [("q8_0", 5, 64), ("q4_k", 3, 256), ("q4_k", 4, 128), ("q6_k", 3, 256),
                           ("q6_k", 2, 96)]:
        data, exact_w = _build(fmt, rng, rows, inf)
        ks = [0, 31, 32, inf - 1]
        x = np.zeros((len(ks), inf), np.float16)
        for m, k in enumerate(ks):
            x[m, k] = 1.0
        bias = rng.normal(0, 0.02, rows).astype(np.float32)
        y, _ = oracle.gemm_packed(fmt, data, rows, inf, x, bias)
        for m, k in enumerate(ks):
            for n in range(rows):
                # one rounding of the exact sum (weights can reach 2^23)
                assert float(y[m, n]) == float(exact_w[n][k] + Fraction(float(bias[n]))), (fmt, m, n)


def test_gemm_packed_unit_scale_q8_0_is_f16_matmul():
    """Q8_0 blocks with d = 1 hold the integer codes themselves, which
    binary16 represents exactly: the packed product reduces to the binary16
    GEMM on the code matrix."""
    rng = np.random.default_rng(15)
    rows, inf = 6, 96
    codes = rng.integers(-128, 128, size=(rows, inf))
    one = packing.f16_bits(1.0)
    data = packing.rows_to_array([[packing.pack_q8_0_block(one, codes[r, 32 * b:32 * b + 32])
                                   for b in range(inf // 32)] for r in range(rows)])
    x = rng.standard_normal((5, inf)).astype(np.float16)
    y, s = oracle.gemm_packed("q8_0", data, rows, inf, x)
    y2, s2 = oracle.gemm_f16(x, codes.astype(np.float16))
    assert np.array_equal(y, y2) and np.array_equal(s, s2)


def test_gemm_packed_brute_force():
    rng = np.random.default_rng(16)
    for fmt, rows, inf in [("q8_0", 3, 64), ("q4_k", 3, 256), ("q6_k", 2, 256)]:
        data, exact_w = _build(fmt, rng, rows, inf)
        x = rng.standard_normal((4, inf)).astype(np.float16)
        bias = rng.normal(0, 0.02, rows).astype(np.float32)
        y, s = oracle.gemm_packed(fmt, data, rows, inf, x, bias)
        ex = _exact_gemv(exact_w, x, bias)
        for m in range(4):
            for n in range(rows):
                err = abs(Fraction(float(y[m, n])) - ex[m][n])
                assert err <= Fraction(2.0 ** -50) * Fraction(float(s[m, n])) + Fraction(1, 2 ** 200)


def test_silu_closed_forms():
    """silu(0) = 0; silu(g) - silu(-g) = g (sigmoid(g) + sigmoid(-g) = 1);
    silu(g) = g * scipy's logistic sigmoid; the tails go to g and to 0."""
    from scipy.special import expit
    g = np.linspace(-30, 30, 241)
    assert oracle.silu(0.0) == 0.0
    assert np.allclose(oracle.silu(g) - oracle.silu(-g), g, rtol=0, atol=1e-12)
    assert np.allclose(oracle.silu(g), g * expit(g), rtol=1e-14, atol=1e-300)
    assert oracle.silu(800.0) == 800.0 and oracle.silu(-800.0) == 0.0
    # a known value: silu(1) = 1 / (1 + 1/e)
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16


def test_swiglu_is_silu_of_gate_times_up():
    """The fused result is the product of the two pinned mat-vecs through the
    SiLU: swapping the roles of gate and up changes it, and a zero up matrix
    (i8row codes 0) gives 0."""
    rng = np.random.default_rng(17)
    codes_g = rng.integers(-127, 128, size=(6, 64)).astype(np.int8)
    codes_u = rng.integers(-127, 128, size=(6, 64)).astype(np.int8)
    sc = np.full(6, 0.01, np.float32)
    x = rng.standard_normal((2, 64)).astype(np.float32)
    h, (g, _), (u, _) = oracle.swiglu_packed("i8row", codes_g.view(np.uint8), codes_u.view(np.uint8), 6, 64,
                                             x, sc, sc)
    g_ref, _ = oracle.gemv_packed("i8row", codes_g.view(np.uint8), 6, 64, x, None, sc)
    u_ref, _ = oracle.gemv_packed("i8row", codes_u.view(np.uint8), 6, 64, x, None, sc)
    assert np.array_equal(g, g_ref) and np.array_equal(u, u_ref)
    for b in range(2):
        for o in range(6):
            ex = Fraction(float(g[b, o])) / (1 + Fraction(float(np.exp(-g[b, o])))) * Fraction(float(u[b, o]))
            assert abs(Fraction(float(h[b, o])) - ex) <= Fraction(2.0 ** -50) * abs(ex) + Fraction(1, 2 ** 300)
    h2, _, _ = oracle.swiglu_packed("i8row", codes_u.view(np.uint8), codes_g.view(np.uint8), 6, 64, x, sc, sc)
    assert not np.allclose(h, h2)
    h0, _, _ = oracle.swiglu_packed("i8row", codes_g.view(np.uint8), np.zeros_like(codes_u).view(np.uint8),
                                    6, 64, x, sc, sc)
    assert np.all(h0 == 0)


@pytest.mark.parametrize("inf", [32, 64, 96, 896])
def test_i4row_codes_and_closed_form(inf):
    rng = np.random.default_rng([26, inf])
    rows = 5
    q = rng.integers(-8, 8, size=(rows, inf))
    scales = (rng.random(rows) * 0.01).astype(np.float32)
    data = np.array([np.frombuffer(packing.pack_i4_row(q[r]), np.uint8) for r in range(rows)])
    assert list(oracle.i4_codes(data)[0, :inf]) == list(q[0])
    w = oracle.dequant_i4row(data, rows, inf, scales)
    for r in range(rows):
        assert as_fraction_array(w[r]) == [Fraction(float(scales[r])) * int(v) for v in q[r]]


def test_i4row_one_hot_positions():
    for i in range(64):
        q = [0] * 64
        q[i] = -3
        data = np.frombuffer(packing.pack_i4_row(q), np.uint8)
        w = oracle.dequant_i4row(data, 1, 64, np.array([2.0], np.float32))[0]
        assert list(np.flatnonzero(w)) == [i] and w[i] == -6.0


@pytest.mark.parametrize("rows,inf", [(4, 32), (6, 96)])
def test_i4row_brute_force(rows, inf):
    rng = np.random.default_rng([27, rows])
    q = rng.integers(-8, 8, size=(rows, inf))
    scales = (rng.random(rows) * 0.01).astype(np.float32)
    data = np.array([np.frombuffer(packing.pack_i4_row(q[r]), np.uint8) for r in range(rows)])
    x = rng.standard_normal((2, inf)).astype(np.float32)
    y, s = oracle.gemv_packed("i4row", data, rows, inf, x, None, scales)
    for b in range(2):
        for o in range(rows):
            ex = sum(Fraction(float(scales[o])) * int(q[o, i]) * Fraction(float(x[b, i])) for i in range(inf))
            assert abs(Fraction(float(y[b, o])) - ex) <= Fraction(2.0 ** -50) * Fraction(float(s[b, o]))


def test_quantize_i4row_round_trip():
    rng = np.random.default_rng(28)
    w = rng.normal(0, 0.02, size=(16, 96)).astype(np.float32)
    w[2] = 0.0
    packed, scales = oracle.quantize_i4row(w)
    assert packed.shape == (16, 64) and scales[2] == 0
    codes = oracle.i4_codes(packed)[:, :96]
    assert np.all(codes[2] == 0) and codes.min() >= -7 and codes.max() <= 7
    for r in range(16):
        if r == 2:
            continue
        assert scales[r] == np.float32(np.max(np.abs(w[r])) / 7.0)
        assert abs(int(codes[r, int(np.argmax(np.abs(w[r])))])) == 7
        deq = scales[r].astype(np.float64) * codes[r].astype(np.float64)
        assert np.all(np.abs(deq - w[r]) <= scales[r] * 0.5 * (1 + 1e-6))
    # halves round away from zero
    p, s = oracle.quantize_i4row(np.array([[7.0, 0.5, -0.5, 1.5, -2.5] + [0.0] * 27], np.float32))
    assert s[0] == 1.0 and list(oracle.i4_codes(p)[0, :5]) == [7, 1, -1, 2, -3]


def test_quantize_i8row_round_trip():
    rng = np.random.default_rng(14)
    w = rng.normal(0, 0.02, size=(32, 200)).astype(np.float32)
    w[3] = 0.0
    codes, scales = oracle.quantize_i8row(w)
    assert scales[3] == 0 and np.all(codes[3] == 0)
    for r in range(32):
        if r == 3:
            continue
        assert scales[r] == np.float32(np.max(np.abs(w[r])) / 127.0)
        amax_at = int(np.argmax(np.abs(w[r])))
        assert abs(int(codes[r, amax_at])) == 127
        deq = scales[r].astype(np.float64) * codes[r].astype(np.float64)
        assert np.all(np.abs(deq - w[r]) <= scales[r] * 0.5 * (1 + 1e-6))
    assert codes.min() >= -127 and codes.max() <= 127
    # halves round away from zero
    c, s = oracle.quantize_i8row(np.array([[127.0, 0.5, -0.5, 1.5, -2.5]], np.float32))
    assert s[0] == 1.0 and list(c[0]) == [127, 1, -1, 2, -3]


def test_tolerance_helper():
    y_ref = np.array([[1.0, 2.0]])
    s_ref = np.array([[10.0, 0.0]])
    ok = oracle.within_tolerance(np.array([[1.0 + 9e-4, 2.0 + 2e-6]]), y_ref, s_ref, 1e-4)
    assert list(ok[0]) == [True, False]


# ---------------------------------------------------------------------------
# 8. planted mistakes are caught by the pins above
# ---------------------------------------------------------------------------
def _all_dequant_fixtures_pass():
    return all(check_dequant_fixture(n) and check_gemv_fixture(n) for n in golden_io.all_fixtures())


def test_planted_mistakes_are_caught(monkeypatch):
    mod = oracle.oracle
    good_codes4, good_codes6, good_sm = mod.q4_k_codes, mod.q6_k_codes, mod.q4_k_scales_mins
    good_gemv = mod.gemv
    assert _all_dequant_fixtures_pass()

    def codes4_swapped(qs):          # low/high nibble order exchanged
        q = good_codes4(qs)
        out = q.copy()
        for r in range(4):
            out[..., 64 * r:64 * r + 32] = q[..., 64 * r + 32:64 * r + 64]
            out[..., 64 * r + 32:64 * r + 64] = q[..., 64 * r:64 * r + 32]
        return out

    def sm_swapped(S):               # scales and mins exchanged
        sc, m = good_sm(S)
        return m, sc

    def sm_no_high_bits(S):          # top bits of scales 4..7 dropped
        sc, m = good_sm(S)
        sc = sc.copy()
        sc[..., 4:] &= 15
        return sc, m

    def codes6_offset(ql, qh):       # high 2 bits in the wrong place
        q = good_codes6(ql, qh)
        return (q & 15) | ((q >> 4) << 5) & 63

    def gemv_no_bias(w64, x, bias=None):
        return good_gemv(w64, x, None)

    good_codes5 = mod.q5_k_codes
    good_codes2, good_scales3 = mod.q2_k_codes, mod.q3_k_scales

    def codes2_halves_swapped(qs):     # the 16-weight halves c = 0, 1 exchanged
        q = good_codes2(qs)
        out = q.copy()
        for b in range(0, 256, 32):
            out[..., b:b + 16], out[..., b + 16:b + 32] = q[..., b + 16:b + 32], q[..., b:b + 16]
        return out

    good_i4 = mod.i4_codes

    def i4_nibbles_swapped(packed):     # high nibble taken as the even weight
        q = good_i4(packed)
        out = q.copy()
        out[..., 0::2], out[..., 1::2] = q[..., 1::2], q[..., 0::2]
        return out

    def scales3_halves_swapped(S):     # scales 0..7 and 8..15 exchanged
        sc = good_scales3(S)
        return np.concatenate([sc[..., 8:], sc[..., :8]], axis=-1)

    def codes5_half_swapped(qh, qs):   # fifth bits of the two halves of a run exchanged
        q = good_codes5(qh, qs)
        low = q & 15
        high = q >> 4
        out = q.copy()
        for r in range(4):
            out[..., 64 * r:64 * r + 32] = low[..., 64 * r:64 * r + 32] | (high[..., 64 * r + 32:64 * r + 64] << 4)
            out[..., 64 * r + 32:64 * r + 64] = low[..., 64 * r + 32:64 * r + 64] | (high[..., 64 * r:64 * r + 32] << 4)
        return out

    for name, bad in [("q4_k_codes", codes4_swapped), ("q4_k_scales_mins", sm_swapped),
                      ("q4_k_scales_mins", sm_no_high_bits), ("q6_k_codes", codes6_offset),
                      ("gemv", gemv_no_bias), ("q5_k_codes", codes5_half_swapped),
                      ("q2_k_codes", codes2_halves_swapped), ("q3_k_scales", scales3_halves_swapped),
                      ("i4_codes", i4_nibbles_swapped)]:
        monkeypatch.setattr(mod, name, bad)
        assert not _all_dequant_fixtures_pass(), name
        monkeypatch.undo()
    assert _all_dequant_fixtures_pass()


def test_planted_transpose_and_dropped_min_are_caught(monkeypatch):
    mod = oracle.oracle
    # a dropped min term in Q4_K
    good = mod.dequant_q4_k

    def no_min(packed, rows, in_features):
        blk = mod._blocks(packed, rows, in_features, "q4_k")
        d = mod._binary16(blk[:, :, 0:2])
        sc, _ = mod.q4_k_scales_mins(blk[:, :, 4:16])
        q = mod.q4_k_codes(blk[:, :, 16:144])
        sub = np.arange(256) // 32
        return (d[:, :, None] * sc[:, :, sub] * q).reshape(rows, -1)[:, :in_features]

    monkeypatch.setattr(mod, "dequant_q4_k", no_min)
    assert not check_dequant_fixture("q4_k_hand.txt")
    monkeypatch.setattr(mod, "dequant_q4_k", good)

    # a transposed operand in the mat-vec: caught by a non-square brute force
    def transposed(w64, x, bias=None):
        x64 = np.atleast_2d(np.asarray(x, dtype=np.float64))
        wt = w64.T.reshape(w64.shape)           # same shape, wrong element order
        y = x64 @ wt.T
        s = np.abs(x64) @ np.abs(wt).T
        if bias is not None:
            y = y + bias
            s = s + np.abs(bias)
        return y, s

    monkeypatch.setattr(mod, "gemv", transposed)
    with pytest.raises(AssertionError):
        test_gemv_brute_force("q8_0", 4, 32)


# ---------------------------------------------------------------------------
# Q4_K stream layout (the byte-minimal layout for rows that are not whole
# super-blocks): weights in row-major order cut into super-blocks in order
# ---------------------------------------------------------------------------
def _stream_from_fields(rng, rows, inf):
    """Packed stream bytes and the exact weights [rows][inf] from random
    fields of ceil(rows * inf / 256) super-blocks (independent packer)."""
    nsb = -(-rows * inf // 256)
    blocks, exact = [], []
    for _ in range(nsb):
        d, dmin, sc, m, q = random_q4_k_fields(rng)
        blocks.append(packing.pack_q4_k_block(d, dmin, sc, m, q))
        exact += q4_k_exact(d, dmin, sc, m, q)
    flat = exact[:rows * inf]
    return (np.frombuffer(b"".join(blocks), dtype=np.uint8).copy(),
            [flat[r * inf:(r + 1) * inf] for r in range(rows)])


@pytest.mark.parametrize("rows,inf", [(2, 128), (3, 384), (5, 896), (7, 64), (3, 192)])
def test_q4_k_stream_fields_and_closed_form(rows, inf):
    rng = np.random.default_rng([71, rows, inf])
    data, exact = _stream_from_fields(rng, rows, inf)
    assert data.size == oracle.matrix_bytes("q4_k_stream", rows, inf)
    w = oracle.dequantize("q4_k_stream", data, rows, inf)
    assert w.shape == (rows, inf)
    assert as_fraction_array(w) == [v for row in exact for v in row]


@pytest.mark.parametrize("rows,inf", [(3, 256), (2, 512), (2, 4864)])
def test_q4_k_stream_of_whole_super_block_rows_is_the_row_layout(rows, inf):
    """When a row is whole super-blocks the stream and the padded row layout
    are the same bytes, and so are the weights."""
    rng = np.random.default_rng([72, rows, inf])
    data, _ = _stream_from_fields(rng, rows, inf)
    assert oracle.matrix_bytes("q4_k_stream", rows, inf) == rows * oracle.row_bytes("q4_k", inf)
    assert np.array_equal(oracle.dequantize("q4_k_stream", data, rows, inf),
                          oracle.dequantize("q4_k", data, rows, inf))


def test_q4_k_stream_one_hot_positions():
    """One code 9 at stream position p lands at row p // in, column p % in
    (rows of 896 weights: 3.5 super-blocks, starting at weight 0 or 128)."""
    rows, inf = 3, 896
    nsb = -(-rows * inf // 256)
    sc = [1, 2, 3, 4, 5, 6, 7, 8]
    for p in (0, 31, 127, 128, 255, 895, 896, 1023, 1024, 1151, 1791, 1792, 2687):
        blocks = []
        for k in range(nsb):
            q = [0] * 256
            if p // 256 == k:
                q[p % 256] = 9
            blocks.append(packing.pack_q4_k_block(0x3C00, 0x0000, sc, [5] * 8, q))
        w = oracle.dequantize("q4_k_stream", np.frombuffer(b"".join(blocks), np.uint8), rows, inf)
        nz = np.argwhere(w)
        assert nz.tolist() == [[p // inf, p % inf]], p
        assert w[p // inf, p % inf] == 9 * sc[(p % 256) // 32]


def test_q4_k_stream_padding_at_the_end_does_not_matter():
    rng = np.random.default_rng(73)
    rows, inf = 3, 896          # 2688 weights: the last super-block's second half is padding
    data, _ = _stream_from_fields(rng, rows, inf)
    other = data.copy()
    last = other[-144:]
    # weights 128..255 of the last block are runs 2 and 3 (code bytes
    # 64..127) with sub-blocks 4..7, whose scale bytes 8..11 hold nothing else
    last[16 + 64:] = rng.integers(0, 256, 64, dtype=np.uint8)
    last[12:16] = rng.integers(0, 256, 4, dtype=np.uint8)
    assert np.array_equal(oracle.dequantize("q4_k_stream", data, rows, inf),
                          oracle.dequantize("q4_k_stream", other, rows, inf))


@pytest.mark.parametrize("rows,inf", [(3, 128), (5, 384), (4, 896)])
def test_q4_k_stream_gemv_brute_force(rows, inf):
    rng = np.random.default_rng([74, rows, inf])
    data, exact_w = _stream_from_fields(rng, rows, inf)
    x = rng.standard_normal((2, inf)).astype(np.float32)
    bias = rng.normal(0, 0.02, rows).astype(np.float32)
    y, s = oracle.gemv_packed("q4_k_stream", data, rows, inf, x, bias)
    ex = _exact_gemv(exact_w, x, bias)
    for b in range(2):
        for o in range(rows):
            err = abs(Fraction(float(y[b, o])) - ex[b][o])
            assert err <= Fraction(2.0 ** -50) * Fraction(float(s[b, o])) + Fraction(1, 2 ** 200), (b, o)


def test_q4_k_stream_gemv_row_chunks_start_on_super_blocks():
    """The oracle expands a large stream matrix in row chunks; each chunk
    must begin on a super-block (a multiple of 2 rows at 896 columns)."""
    rng = np.random.default_rng(75)
    rows, inf = 37, 896
    data, _ = _stream_from_fields(rng, rows, inf)
    x = rng.standard_normal((1, inf)).astype(np.float32)
    whole, s = oracle.gemv(oracle.dequantize("q4_k_stream", data, rows, inf), x)
    for chunk in (1, 2, 3, 8, 1000):
        y, _ = oracle.gemv_packed("q4_k_stream", data, rows, inf, x, row_chunk=chunk)
        # float64 sums in another blocking differ at most by rounding
        assert np.all(np.abs(y - whole) <= 2.0 ** -40 * s), chunk


def test_planted_row_layout_reading_of_the_stream_is_caught():
    """Reading a stream matrix as padded rows (896-weight rows as whole
    super-blocks) fails the stream fixtures."""
    fx = golden_io.load("q4_k_stream_rows.txt")
    data, _ = golden_io.packed(fx)
    w = oracle.dequantize("q4_k_stream", data, fx["rows"], fx["in_features"])
    assert np.array_equal(w.reshape(-1), fx["f64"])
    # padded rows of 384 weights are two whole super-blocks (288 bytes)
    wrong = oracle.dequant_q4_k(data[:2 * 288], 2, fx["in_features"])
    assert not np.array_equal(wrong.reshape(-1), fx["f64"][:2 * fx["in_features"]])
