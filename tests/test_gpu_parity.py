"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bars: dequantized weights bit-exact (value equality with the oracle's
float32 rounding); mat-vec |y - y_oracle| <= 1e-4 * sum|w x| + 1e-6; binary16
GEMM the same with 2e-3.  Inputs come from the seeded generator; shapes span
several row tiles and ragged tails; the full decode-step shapes are checked
on sampled rows in the launch configuration the benchmark times.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import dequantize_mat_vec_amd as dmv
from dequantize_mat_vec_amd import synth
from gpu_util import (announce, assert_within, run_dequant, run_gemm, run_gemm_quant, run_gemm_ws, run_gemv,
                      run_swiglu)

pytestmark = pytest.mark.gpu

GEMV_REL = 1e-4
GEMM_REL = 2e-3
FORMATS = ("q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k", "i8row", "i4row")


@pytest.fixture(autouse=True)
def _name_case(request):
    announce(request.node.nodeid)
    yield


def make(fmt, out, inf, seed, batch=1, with_bias=True):
    rng = np.random.default_rng([777, seed, out, inf, batch])
    packed, scales = synth.matrix(fmt, rng, out, inf)
    x = synth.activations(rng, batch, inf)
    bias = synth.bias(rng, out) if with_bias else None
    return packed, scales, x, bias


# ---------------------------------------------------------------------------
# dequantization: bit-exact
# ---------------------------------------------------------------------------
DEQUANT_SHAPES = [(1, 32), (7, 256), (19, 896), (33, 288), (5, 4864)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("rows,inf", DEQUANT_SHAPES)
def test_dequant_bit_exact(fmt, rows, inf):
    packed, scales, _, _ = make(fmt, rows, inf, 1)
    got = run_dequant(fmt, packed, scales, rows, inf)
    want = oracle.dequantize_f32(fmt, packed, rows, inf, scales)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k"])
@pytest.mark.parametrize("d_bits", [0x0000, 0x0001, 0x0400, 0x7BFF])
def test_dequant_forced_scales(fmt, d_bits):
    rng = np.random.default_rng([5, d_bits])
    packed = synth.quant_blocks(fmt, rng, 9, 512, force_d=d_bits)
    got = run_dequant(fmt, packed, None, 9, 512)
    assert np.array_equal(got, oracle.dequantize_f32(fmt, packed, 9, 512))


# ---------------------------------------------------------------------------
# mat-vec parity
# ---------------------------------------------------------------------------
GEMV_SHAPES = [(1, 32), (5, 64), (67, 896), (130, 288), (37, 1056), (300, 4864), (16, 768)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("out,inf", GEMV_SHAPES)
@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_parity(fmt, out, inf, batch):
    packed, scales, x, bias = make(fmt, out, inf, 2, batch)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("batch", [2, 4, 5, 6, 7])
def test_gemv_every_batch(fmt, batch):
    packed, scales, x, bias = make(fmt, 45, 896, 3, batch)
    y = run_gemv(fmt, packed, scales, 45, 896, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, 45, 896, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} b{batch}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_gemv_large_in_batch_split(fmt):
    """A staged x that cannot hold every batch row at once is split."""
    packed, scales, x, bias = make(fmt, 24, 16384, 4, 8)
    y = run_gemv(fmt, packed, scales, 24, 16384, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, 24, 16384, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} in=16384 b8")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("out,inf,batch", [(37, 4160, 1), (37, 4352, 3), (5, 4864, 1), (130, 12288, 2),
                                           (2, 16384, 8)])
def test_gemv_rows_split_across_wavefronts(fmt, out, inf, batch):
    """Long rows of short matrices: each row's units are split over 2 or 4
    wavefronts (unit counts that do not divide evenly, ragged tiles)."""
    packed, scales, x, bias = make(fmt, out, inf, 6, batch)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("inf,batch", [(20480, 1), (32768, 3), (16416, 2)])
def test_gemv_rows_longer_than_one_load_round(fmt, inf, batch):
    """Rows of more than 256 units: whole-wave lane groups walk their units
    with two register buffers (odd and even unit counts per lane)."""
    packed, scales, x, bias = make(fmt, 9, inf, 5, batch)
    y = run_gemv(fmt, packed, scales, 9, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, 9, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} in={inf} b{batch}")


# ---------------------------------------------------------------------------
# invariants and edge cases
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("fmt", FORMATS)
def test_one_hot_x_gives_dequantized_column(fmt):
    """x = e_j makes y column j of W, bit-exact: every other term is 0."""
    out, inf = 40, 896
    packed, scales, _, _ = make(fmt, out, inf, 5)
    w32 = oracle.dequantize_f32(fmt, packed, out, inf, scales)
    cols = [0, 1, 31, 32, 255, 256, 511, 767, 768, 895]
    x = np.zeros((8, inf), np.float32)
    for b, j in enumerate(cols[:8]):
        x[b, j] = 1.0
    y = run_gemv(fmt, packed, scales, out, inf, x)
    for b, j in enumerate(cols[:8]):
        assert np.array_equal(y[b], w32[:, j]), (fmt, j)


@pytest.mark.parametrize("fmt", FORMATS)
def test_power_of_two_scaling_is_exact(fmt):
    out, inf = 50, 896
    packed, scales, x, _ = make(fmt, out, inf, 6)
    y1 = run_gemv(fmt, packed, scales, out, inf, x)
    y2 = run_gemv(fmt, packed, scales, out, inf, x * np.float32(8.0))
    assert np.array_equal(y2, y1 * np.float32(8.0))


@pytest.mark.parametrize("fmt", ["q2_k", "q3_k", "q4_k", "q5_k", "q6_k"])
def test_padding_bytes_do_not_matter(fmt):
    """Rows of 896 hold 3.5 super-blocks; the padding half must be ignored."""
    out, inf = 33, 896
    packed, _, x, bias = make(fmt, out, inf, 7)
    rng = np.random.default_rng(99)
    other = packed.copy().reshape(out, -1)
    nb = {"q2_k": 84, "q3_k": 110, "q4_k": 144, "q5_k": 176, "q6_k": 210}[fmt]
    last = other[:, 3 * nb:4 * nb]

    def high_nibbles(lo, hi):   # randomize bits 4-7 of bytes lo..hi-1
        last[:, lo:hi] = (last[:, lo:hi] & 0x0F) | (rng.integers(0, 16, last[:, lo:hi].shape,
                                                                  dtype=np.uint8) << 4)
    if fmt == "q2_k":
        last[:, 8:16] = rng.integers(0, 256, last[:, 8:16].shape, dtype=np.uint8)
        last[:, 48:80] = rng.integers(0, 256, last[:, 48:80].shape, dtype=np.uint8)
    elif fmt == "q3_k":
        high_nibbles(0, 32)       # high bits of the second half (bits 4..7)
        last[:, 64:96] = rng.integers(0, 256, last[:, 64:96].shape, dtype=np.uint8)
        high_nibbles(96, 108)     # scale bits of sub-blocks 8..15
    elif fmt == "q5_k":
        last[:, 48 + 64:] = rng.integers(0, 256, last[:, 48 + 64:].shape, dtype=np.uint8)
        last[:, 16:48] = (last[:, 16:48] & 0x0F) | (rng.integers(0, 16, last[:, 16:48].shape,
                                                               dtype=np.uint8) << 4)
        last[:, 12:16] = rng.integers(0, 256, last[:, 12:16].shape, dtype=np.uint8)
        last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, last[:, 4:12].shape,
                                                             dtype=np.uint8) << 6)
    elif fmt == "q4_k":
        last[:, 16 + 64:] = rng.integers(0, 256, last[:, 16 + 64:].shape, dtype=np.uint8)
        last[:, 12:16] = rng.integers(0, 256, last[:, 12:16].shape, dtype=np.uint8)
        last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, last[:, 4:12].shape,
                                                             dtype=np.uint8) << 6)
    else:
        last[:, 64:128] = rng.integers(0, 256, last[:, 64:128].shape, dtype=np.uint8)
        last[:, 160:192] = rng.integers(0, 256, last[:, 160:192].shape, dtype=np.uint8)
        last[:, 200:208] = rng.integers(0, 256, last[:, 200:208].shape, dtype=np.uint8)
    y1 = run_gemv(fmt, packed, None, out, inf, x, bias)
    y2 = run_gemv(fmt, other, None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("fmt", FORMATS)
def test_in_features_zero_gives_bias(fmt):
    rng = np.random.default_rng(8)
    bias = synth.bias(rng, 21)
    import torch
    from gpu_util import guarded_y, guards_intact, to_dev
    import dequantize_mat_vec_amd as dmv
    fbuf, y = guarded_y(2 * 21)
    scales = to_dev(np.ones(21, np.float32)) if fmt in ("i8row", "i4row") else None
    dmv.gemv(fmt, 21, 0, None, None, y, to_dev(bias), 2, scales=scales)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, 42)
    got = y.cpu().numpy().reshape(2, 21)
    assert np.array_equal(got, np.stack([bias, bias]))


@pytest.mark.parametrize("fmt", FORMATS)
def test_empty_output_touches_nothing(fmt):
    import torch
    from gpu_util import guarded_y, guards_intact
    import dequantize_mat_vec_amd as dmv
    fbuf, y = guarded_y(0)
    dmv.gemv(fmt, 0, 64, None, None, y, None, 1)
    dmv.gemv(fmt, 16, 64, None, None, y, None, 0)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, 0)


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k"])
@pytest.mark.parametrize("d_bits", [0x0000, 0x0001, 0x0400, 0x7BFF])
def test_gemv_forced_scales(fmt, d_bits):
    rng = np.random.default_rng([9, d_bits])
    packed = synth.quant_blocks(fmt, rng, 40, 896, force_d=d_bits)
    x = synth.activations(rng, 2, 896)
    y = run_gemv(fmt, packed, None, 40, 896, x)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, 40, 896, x)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} d={d_bits:#06x}")


def test_q6_k_all_codes_32_is_zero():
    """q = 32 everywhere dequantizes to 0: y must equal the bias exactly
    (the (q - 32) factor is formed exactly, never as q*x - 32*x)."""
    rng = np.random.default_rng(10)
    out, inf = 20, 896
    packed = synth.quant_blocks("q6_k", rng, out, inf).reshape(out, -1, 210)
    packed[:, :, 0:128] = 0x00      # low parts 0
    packed[:, :, 128:192] = 0xAA    # high parts 2 -> q = 32
    packed = packed.reshape(out, -1)
    assert np.all(oracle.dequant_q6_k(packed, out, inf) == 0)
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q6_k", packed, None, out, inf, x, bias)
    assert np.array_equal(y[0], bias)


def test_i4row_padding_codes_do_not_matter():
    """Rows of 800 weights take 13 units of 64; the last 16 bytes of every
    row are padding codes and never reach the result."""
    out, inf = 45, 800
    packed, scales, x, bias = make("i4row", out, inf, 14, 2)
    other = packed.copy().reshape(out, -1)
    assert other.shape[1] == 13 * 32
    other[:, 400:] = np.random.default_rng(15).integers(0, 256, (out, 16), dtype=np.uint8)
    y1 = run_gemv("i4row", packed, scales, out, inf, x, bias)
    y2 = run_gemv("i4row", other, scales, out, inf, x, bias)
    assert np.array_equal(y1, y2)
    y_ref, s_ref = oracle.gemv_packed("i4row", packed, out, inf, x, bias, scales)
    assert_within(y1, y_ref, s_ref, GEMV_REL, "i4row in=800")


@pytest.mark.parametrize("density", [0.0, 0.02, 0.3])
@pytest.mark.parametrize("batch", [1, 2])
def test_i4row_sparse_codes(density, batch):
    """Rows of mostly zero int4 codes (an all-zero row must give exactly the
    bias) meet the plain mat-vec bound 1e-4 * sum|w x| + 1e-6 at batch 1
    (vector ALUs) and 2 (matrix cores for tall matrices, vector ALUs for
    this 96-row one)."""
    import packing
    rng = np.random.default_rng([16, int(density * 100), batch])
    out, inf = 96, 4864
    q = rng.integers(-8, 8, (out, inf)) * (rng.random((out, inf)) < density)
    packed = np.array([np.frombuffer(packing.pack_i4_row(q[r]), np.uint8) for r in range(out)])
    scales = (0.005 + 0.01 * rng.random(out)).astype(np.float32)
    x = synth.activations(rng, batch, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("i4row", packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("i4row", packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"i4row density {density} b{batch}")
    if density == 0.0:
        assert np.array_equal(y, np.broadcast_to(bias, y.shape))


def test_q8_0_zero_codes_is_exact_bias():
    rng = np.random.default_rng(11)
    out, inf = 20, 896
    packed = synth.quant_blocks("q8_0", rng, out, inf).reshape(out, -1, 34)
    packed[:, :, 2:] = 0
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q8_0", packed.reshape(out, -1), None, out, inf, x, bias)
    assert np.array_equal(y[0], bias)


def test_odd_rows_misaligned_blocks():
    """Q8_0 rows of an odd block count start 2 bytes off a dword boundary;
    Q6_K super-blocks do so every other one."""
    for fmt, inf in (("q8_0", 96), ("q8_0", 4896), ("q6_k", 4864), ("q6_k", 1280)):
        packed, scales, x, bias = make(fmt, 31, inf, 12, 2)
        y = run_gemv(fmt, packed, scales, 31, inf, x, bias)
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, 31, inf, x, bias, scales)
        assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} in={inf}")


# ---------------------------------------------------------------------------
# full decode-step shapes, sampled rows, benchmark launch configuration
# ---------------------------------------------------------------------------
FULL = [("q8_0", synth.QWEN_VOCAB, 896, 1), ("q8_0", synth.QWEN_VOCAB, 896, 8),
        ("q4_k", synth.QWEN_VOCAB, 896, 4), ("q6_k", synth.QWEN_VOCAB, 896, 2),
        ("q8_0", synth.GPT2_VOCAB, 768, 1),
        ("q4_k", 4864, 896, 1), ("q4_k", 896, 4864, 1), ("q6_k", 896, 4864, 1),
        ("q4_k", 128, 896, 1), ("i8row", 896, 896, 1),
        ("q5_k", synth.QWEN_VOCAB, 896, 1), ("q5_k", 4864, 896, 1), ("q5_k", 896, 4864, 3),
        ("q2_k", synth.QWEN_VOCAB, 896, 1), ("q2_k", 896, 4864, 2), ("q3_k", synth.QWEN_VOCAB, 896, 1),
        ("q3_k", 896, 4864, 4), ("i4row", synth.QWEN_VOCAB, 896, 1), ("i4row", 4864, 896, 2),
        ("i4row", 896, 4864, 1)]


@pytest.mark.parametrize("fmt,out,inf,batch", FULL)
def test_full_size_sampled_rows(fmt, out, inf, batch):
    rng = np.random.default_rng([13, out, inf, batch])
    packed, scales = synth.matrix(fmt, rng, out, inf)
    x = synth.activations(rng, batch, inf)
    bias = synth.bias(rng, out)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    rows = np.unique(np.concatenate([rng.integers(0, out, 384), [0, out - 1]]))
    sub = packed.reshape(out, -1)[rows]
    y_ref, s_ref = oracle.gemv_packed(fmt, sub, len(rows), inf, x, bias[rows],
                                      None if scales is None else scales[rows])
    assert_within(y[:, rows], y_ref, s_ref, GEMV_REL, f"{fmt} {out}x{inf} b{batch}")


# ---------------------------------------------------------------------------
# binary16 small-M GEMM
# ---------------------------------------------------------------------------
GEMM_CASES = [(8, 768, 2304), (32, 768, 768), (64, 768, 3072), (64, 3072, 768),
              (1, 64, 40), (15, 96, 33), (16, 32, 16), (17, 160, 70), (100, 256, 48),
              (8, 3072, 768), (32, 3072, 768), (5, 2080, 33), (15, 4096, 70),
              # no columns: y is the bias; long rows: several load rounds
              (20, 0, 37), (5, 0, 9), (8, 8192, 40), (3, 16384, 24), (48, 16384, 20),
              # a ragged K split: 3 k-steps over the workgroup's wavefronts
              (33, 96, 17),
              # K a multiple of 64 (odd rows load each pair of k-steps in
              # swapped order): odd step counts per wavefront, one step per
              # wavefront, and the 8- and 16-wavefront launch shapes
              (33, 192, 40), (16, 576, 40), (17, 64, 70), (16, 576, 1600), (40, 1344, 1540),
              # narrow layers over 128 k-steps (16 K slices): the Qwen down shape
              (16, 4864, 896), (33, 4128, 70),
              # wide layers (96+ column tiles): 1, 2 and 4 row tiles per
              # workgroup, ragged in M and N
              (16, 64, 1600), (20, 128, 2000), (40, 96, 1540),
              # 256+ workgroups at 1, 2 and 4 row tiles of X (8 K slices),
              # ragged in M and N, K a multiple of 64 or not
              (16, 896, 4100), (24, 896, 4100), (50, 256, 4864), (100, 160, 4100),
              # wide layers (1024+ column tiles): X rows staged in LDS once
              # per workgroup
              (17, 96, 16385), (65, 1024, 16400), (130, 256, 16500), (16, 4096, 16384),
              (40, 32, 33000), (64, 896, 4864),
              # the largest m the entry point takes (PESTI_MAX_GEMM_M)
              (4096, 64, 40)]


@pytest.mark.parametrize("m,k,n", GEMM_CASES)
def test_gemm_f16_parity(m, k, n):
    rng = np.random.default_rng([14, m, k, n])
    x = synth.f16_activations(rng, m, k)
    w = synth.f16_weights(rng, n, k)
    bias = synth.bias(rng, n)
    y = run_gemm(x, w, bias)
    y_ref, s_ref = oracle.gemm_f16(x, w, bias)
    assert_within(y, y_ref, s_ref, GEMM_REL, f"gemm m{m} k{k} n{n}")


# ---------------------------------------------------------------------------
# small-M GEMM on quantized weights: exact codes on the matrix cores, block
# scales in float32, so the mat-vec's bound applies
# ---------------------------------------------------------------------------
QGEMM_REL = GEMV_REL
QGEMM_CASES = [(16, 896, 4864), (32, 4864, 896), (64, 896, 128), (17, 896, 70),
               (1, 64, 40), (5, 96, 33), (16, 32, 16), (100, 1056, 48),
               # ragged K split: 3 k-steps over the workgroup's wavefronts;
               # Q8_0 rows of an odd block count (misaligned blocks); Q4_K
               # rows padded to whole super-blocks
               (33, 96, 17), (40, 320, 77), (19, 4896, 31),
               # no columns: Y is the bias; long rows
               (20, 0, 37), (8, 8192, 40), (48, 16384, 20), (3, 32768, 9),
               # wide layers: 1, 2 and 4 row tiles per workgroup
               (16, 64, 1600), (20, 256, 2000), (40, 96, 1540), (64, 128, 1536),
               # 256+ workgroups at 1, 2 and 4 row tiles of X (8 K slices)
               (16, 896, 4100), (5, 96, 4864), (24, 896, 4100), (50, 256, 4864), (100, 160, 4100),
               # the largest m the entry points take (PESTI_MAX_GEMM_M)
               (4096, 96, 40)]
# Wide layers (1024+ column tiles, 256+ for Q4_K; X rows staged in LDS):
# ragged N and M, several 64-row chunks of X, one k-step, rows of several
# wavefronts' tiles, wavefronts left without a tile.
QGEMM_WIDE = [(16, 896, 16400), (17, 96, 16385), (33, 320, 16390), (64, 1024, 16384),
              (65, 32, 16400), (130, 256, 16500), (1, 64, 16384), (8, 4096, 16384),
              (48, 896, 4864), (100, 96, 33000), (3, 32, 40000)]
QGEMM_CASES += QGEMM_WIDE


QGEMM_FORMATS = ("q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k")


@pytest.mark.parametrize("fmt", QGEMM_FORMATS)
@pytest.mark.parametrize("m,k,n", QGEMM_CASES)
def test_gemm_quant_parity(fmt, m, k, n):
    rng = np.random.default_rng([15, m, k, n])
    packed = synth.quant_blocks(fmt, rng, n, k) if k else np.zeros((n, 0), np.uint8)
    x = synth.f16_activations(rng, m, k)
    bias = synth.bias(rng, n)
    y = run_gemm_quant(fmt, packed, m, n, k, x, bias)
    y_ref, s_ref = oracle.gemm_packed(fmt, packed, n, k, x, bias)
    assert_within(y, y_ref, s_ref, QGEMM_REL, f"{fmt} gemm m{m} k{k} n{n}")


@pytest.mark.parametrize("fmt", QGEMM_FORMATS)
def test_gemm_quant_no_bias_and_one_hot(fmt):
    """Unit rows of X return dequantized columns of W (no bias)."""
    rng = np.random.default_rng([16, len(fmt)])
    n, k = 40, 512
    packed = synth.quant_blocks(fmt, rng, n, k)
    ks = [0, 1, 31, 32, 255, 256, 300, 511] * 2 + [7] * 4
    x = np.zeros((len(ks), k), np.float16)
    for m, kk in enumerate(ks):
        x[m, kk] = 1.0
    y = run_gemm_quant(fmt, packed, len(ks), n, k, x)
    w32 = oracle.dequantize_f32(fmt, packed, n, k)
    for m, kk in enumerate(ks):
        assert np.array_equal(y[m], w32[:, kk]), (fmt, m, kk)


QGEMM_FULL = [("q8_0", 16, synth.QWEN_VOCAB, 896), ("q4_k", 64, synth.QWEN_VOCAB, 896),
              ("q4_k", 64, 4864, 896), ("q4_k", 32, 896, 4864), ("q8_0", 64, 896, 4864),
              ("q6_k", 64, 896, 4864), ("q6_k", 16, 4864, 896), ("q6_k", 32, synth.QWEN_VOCAB, 896),
              ("q2_k", 64, synth.QWEN_VOCAB, 896), ("q3_k", 16, synth.QWEN_VOCAB, 896),
              ("q5_k", 32, synth.QWEN_VOCAB, 896), ("q2_k", 32, 896, 4864), ("q3_k", 64, 896, 4864),
              ("q5_k", 16, 896, 4864)]


@pytest.mark.parametrize("fmt,m,n,k", QGEMM_FULL)
def test_gemm_quant_full_size_sampled_columns(fmt, m, n, k):
    rng = np.random.default_rng([17, m, n, k])
    packed = synth.quant_blocks(fmt, rng, n, k)
    x = synth.f16_activations(rng, m, k)
    bias = synth.bias(rng, n)
    y = run_gemm_quant(fmt, packed, m, n, k, x, bias)
    cols = np.unique(np.concatenate([rng.integers(0, n, 256), [0, n - 1]]))
    sub = packed.reshape(n, -1)[cols]
    y_ref, s_ref = oracle.gemm_packed(fmt, sub, len(cols), k, x, bias[cols])
    assert_within(y[:, cols], y_ref, s_ref, QGEMM_REL, f"{fmt} gemm m{m} {n}x{k}")


# ---------------------------------------------------------------------------
# the same GEMMs with a caller's workspace: K split over workgroups on narrow
# layers with long rows, partial tiles summed by a second launch
# ---------------------------------------------------------------------------
WS_FORMATS = ("f16",) + QGEMM_FORMATS
# (m, k, n): 4 splits at m 16 on the down shape; one and eight rows of X
# (binary16 below 16 rows: vector ALUs, unsplit); ragged K (129 k-steps);
# 2 and 3 row tiles of X; 95 column tiles (2 splits); very long rows
WS_SPLIT_CASES = [(16, 4864, 896), (1, 4864, 896), (8, 4864, 896), (16, 4128, 70), (33, 8192, 40),
                  (32, 4864, 896), (16, 4160, 1520), (5, 16384, 24), (16, 32768, 20),
                  # Q3_K, Q6_K: two row tiles of X per workgroup (the
                  # second ragged at 48 and 47 rows); the others do not split
                  (48, 4864, 896), (64, 4864, 896), (47, 4128, 70)]
# shapes that do not split in any format: the workspace call equals the
# plain call
WS_PLAIN_CASES = [(80, 4864, 896), (16, 896, 4864), (16, 4096, 896)]


def _ws_inputs(fmt, m, k, n, seed):
    rng = np.random.default_rng([seed, m, k, n, len(fmt)])
    w = synth.f16_weights(rng, n, k) if fmt == "f16" else synth.quant_blocks(fmt, rng, n, k)
    return w, synth.f16_activations(rng, m, k), synth.bias(rng, n)


def _ws_oracle(fmt, w, m, n, k, x, bias):
    return oracle.gemm_f16(x, w, bias) if fmt == "f16" else oracle.gemm_packed(fmt, w, n, k, x, bias)


@pytest.mark.parametrize("fmt", WS_FORMATS)
@pytest.mark.parametrize("m,k,n", WS_SPLIT_CASES)
def test_gemm_ws_split_parity(fmt, m, k, n):
    w, x, bias = _ws_inputs(fmt, m, k, n, 31)
    need = dmv.pesti_gemm_workspace_bytes(fmt, m, n, k)
    if m <= 33 and (fmt != "f16" or (m == 16 and (n + 15) // 16 < 96)):
        assert need > 0, (fmt, m, k, n)
    if m >= 47 and fmt in ("q3_k", "q6_k"):
        assert need > 0, (fmt, m, k, n)
    y = run_gemm_ws(fmt, w, m, n, k, x, bias)
    y_ref, s_ref = _ws_oracle(fmt, w, m, n, k, x, bias)
    assert_within(y, y_ref, s_ref, QGEMM_REL if fmt != "f16" else GEMM_REL, f"{fmt} ws gemm m{m} k{k} n{n}")
    # the partials are summed in a fixed order: a second call gives the same bits
    assert np.array_equal(run_gemm_ws(fmt, w, m, n, k, x, bias), y)


@pytest.mark.parametrize("fmt", WS_FORMATS)
@pytest.mark.parametrize("m,k,n", WS_PLAIN_CASES)
def test_gemm_ws_without_split_equals_plain_call(fmt, m, k, n):
    w, x, bias = _ws_inputs(fmt, m, k, n, 32)
    assert dmv.pesti_gemm_workspace_bytes(fmt, m, n, k) == 0
    y = run_gemm_ws(fmt, w, m, n, k, x, bias)
    plain = run_gemm(x, w, bias) if fmt == "f16" else run_gemm_quant(fmt, w, m, n, k, x, bias)
    assert np.array_equal(y, plain)


@pytest.mark.parametrize("fmt", ("f16", "q6_k"))
def test_gemm_ws_rejects_missing_or_short_workspace(fmt):
    m, k, n = 16, 4864, 896
    w, x, bias = _ws_inputs(fmt, m, k, n, 33)
    need = dmv.pesti_gemm_workspace_bytes(fmt, m, n, k)
    for nbytes in (0, need - 16):
        with pytest.raises(dmv.PestiError) as ei:
            run_gemm_ws(fmt, w, m, n, k, x, bias, workspace_bytes=nbytes)
        assert ei.value.status == dmv.PESTI_ERR_WORKSPACE


# ---------------------------------------------------------------------------
# fused SwiGLU feed-forward input: h = silu(W_gate x) * (W_up x)
# ---------------------------------------------------------------------------
SWIGLU_CASES = [(4864, 896, 1), (4864, 896, 8), (37, 896, 3), (130, 288, 2), (1, 32, 1),
                (300, 1056, 5), (64, 4096, 1), (17, 2048, 4), (2049, 64, 7), (65, 1024, 6)]


def _assert_swiglu(h, h_ref, g, sg, u, su, what):
    tol = oracle.swiglu_tolerance(g, sg, u, su, h_ref)
    err = np.abs(h.astype(np.float64) - h_ref)
    bad = err > tol
    assert not np.any(bad), f"{what}: {int(bad.sum())} outside tolerance, first {np.argwhere(bad)[:3].tolist()}"
    assert np.all(np.isfinite(h)), what


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("out,inf,batch", SWIGLU_CASES)
def test_swiglu_parity(fmt, out, inf, batch):
    if fmt == "q8_0" and inf % 64 and inf > 2048:
        pytest.skip("Q8_0 rows of an odd block count fit one round up to 2048 weights")
    rng = np.random.default_rng([18, out, inf, batch, len(fmt)])
    wg, sg_ = synth.matrix(fmt, rng, out, inf)
    wu, su_ = synth.matrix(fmt, rng, out, inf)
    x = synth.activations(rng, batch, inf)
    h = run_swiglu(fmt, wg, wu, sg_, su_, out, inf, x)
    h_ref, (g, sg), (u, su) = oracle.swiglu_packed(fmt, wg, wu, out, inf, x, sg_, su_)
    _assert_swiglu(h, h_ref, g, sg, u, su, f"swiglu {fmt} {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", FORMATS)
def test_swiglu_equals_silu_of_separate_mat_vecs(fmt):
    """The fused launch against the two plain mat-vecs run on the GPU, the
    SiLU and product taken in float64 on their outputs."""
    rng = np.random.default_rng([19, len(fmt)])
    out, inf, batch = 4864, 896, 2
    wg, sg_ = synth.matrix(fmt, rng, out, inf)
    wu, su_ = synth.matrix(fmt, rng, out, inf)
    x = synth.activations(rng, batch, inf)
    h = run_swiglu(fmt, wg, wu, sg_, su_, out, inf, x)
    g_gpu = run_gemv(fmt, wg, sg_, out, inf, x).astype(np.float64)
    u_gpu = run_gemv(fmt, wu, su_, out, inf, x).astype(np.float64)
    h_sep = oracle.silu(g_gpu) * u_gpu
    assert np.allclose(h, h_sep, rtol=2e-4, atol=1e-5), fmt


def test_swiglu_without_columns_is_zero():
    import torch
    import dequantize_mat_vec_amd as dmv
    h = torch.full((3 * 40,), 7.0, dtype=torch.float32, device="cuda")
    dmv.pesti_gemv_swiglu("q4_k", 40, 0, None, None, None, h, 3)
    torch.cuda.synchronize()
    assert torch.all(h == 0)


# ---------------------------------------------------------------------------
# grouped launches
# ---------------------------------------------------------------------------
GROUP_SHAPES = [(37, 896), (130, 288), (8, 4864), (0, 896), (1, 32), (300, 896), (64, 1056)]


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("batch", [1, 3])
def test_group_matches_oracle_per_op(fmt, batch):
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import guarded_y, guards_intact, to_dev
    cases, ops, bufs = [], [], []
    for i, (out, inf) in enumerate(GROUP_SHAPES):
        packed, scales, x, bias = make(fmt, out, inf, 40 + i, batch, with_bias=(i % 2 == 0))
        fbuf, y = guarded_y(batch * out)
        w_d = to_dev(packed.reshape(-1).view(np.uint8)) if packed.size else None
        s_d = to_dev(scales) if scales is not None and scales.size else None
        x_d = to_dev(x) if x.size else None
        b_d = to_dev(bias) if bias is not None and bias.size else None
        bufs.append((w_d, s_d, x_d, b_d, fbuf))
        ops.append((out, inf, w_d, x_d, y, b_d, s_d))
        cases.append((packed, scales, x, bias, out, inf, fbuf, y))
    dmv.pesti_gemv_group(fmt, ops, batch)
    torch.cuda.synchronize()
    for packed, scales, x, bias, out, inf, fbuf, y in cases:
        assert guards_intact(fbuf, batch * out)
        if out == 0:
            continue
        got = y.cpu().numpy().reshape(batch, out)
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias, scales)
        assert_within(got, y_ref, s_ref, GEMV_REL, f"group {fmt} {out}x{inf}")


def test_q8_0_group_of_both_units_equals_single_calls_bitwise():
    """Q8_0 rows of an even block count take the two-block unit, the others
    the one-block unit; the unit is chosen per op, so a group holding both
    gives every op the bits of its own single call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for i, (out, inf) in enumerate([(300, 896), (77, 800), (40, 4864), (9, 32), (130, 288)]):
        packed, _, x, bias = make("q8_0", out, inf, 110 + i, 2)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(2 * out, dtype=torch.float32, device="cuda")
        ys = torch.empty(2 * out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        singles.append((out, inf, w_d, x_d, ys, b_d, packed, x, bias))
    dmv.pesti_gemv_group("q8_0", ops, 2)
    for out, inf, w_d, x_d, ys, b_d, *_ in singles:
        dmv.pesti_gemv_q8_0(out, inf, w_d, x_d, ys, b_d, 2)
    torch.cuda.synchronize()
    for (o, _, _, _, yg, _, _), (out, inf, _, _, ys, _, packed, x, bias) in zip(ops, singles):
        assert torch.equal(yg, ys), o
        y_ref, s_ref = oracle.gemv_packed("q8_0", packed, out, inf, x, bias)
        assert_within(ys.cpu().numpy().reshape(2, out), y_ref, s_ref, GEMV_REL, f"q8_0 group {out}x{inf}")


def test_group_equals_single_calls_bitwise():
    """A grouped launch runs the same arithmetic as the single-matrix call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for i, (out, inf) in enumerate([(896, 896), (128, 896), (128, 896)]):
        packed, _, x, bias = make("q4_k", out, inf, 60 + i, 1)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(out, dtype=torch.float32, device="cuda")
        ys = torch.empty(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        singles.append((out, inf, w_d, x_d, ys, b_d))
    dmv.pesti_gemv_group("q4_k", ops, 1)
    for out, inf, w_d, x_d, ys, b_d in singles:
        dmv.pesti_gemv_q4_k(out, inf, w_d, x_d, ys, b_d, 1)
    torch.cuda.synchronize()
    for (o, _, _, _, yg, _, _), (_, _, _, _, ys, _) in zip(ops, singles):
        assert torch.equal(yg, ys)


def test_group_of_short_and_long_rows_equals_single_calls_bitwise():
    """At batch 1, rows of at most 1024 weights run in half units and longer
    ones in whole runs; the choice is made per op (a mixed group is two
    launches), so every op gives the bits of its own single call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for i, (out, inf) in enumerate([(896, 896), (896, 4864), (128, 512), (37, 2048), (300, 1024)]):
        packed, _, x, bias = make("q4_k", out, inf, 70 + i, 1)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(out, dtype=torch.float32, device="cuda")
        ys = torch.empty(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        singles.append((out, inf, w_d, x_d, ys, b_d))
    dmv.pesti_gemv_group("q4_k", ops, 1)
    for out, inf, w_d, x_d, ys, b_d in singles:
        dmv.pesti_gemv_q4_k(out, inf, w_d, x_d, ys, b_d, 1)
    torch.cuda.synchronize()
    for (o, _, _, _, yg, _, _), (_, _, _, _, ys, _) in zip(ops, singles):
        assert torch.equal(yg, ys), o


# ---------------------------------------------------------------------------
# tall matrices: launches where a lane group serves 2 or 4 rows, with a
# ragged last tile, checked on every row
# ---------------------------------------------------------------------------
TALL = [("q8_0", 65536 + 37, 64, 1), ("q8_0", 131072 + 53, 64, 3), ("q8_0", 131072 + 11, 96, 1),
        ("q4_k", 65536 + 37, 256, 2), ("q4_k", 131072 + 53, 896, 1), ("q4_k", 65536 + 29, 1280, 1),
        ("q6_k", 65536 + 37, 256, 1), ("q6_k", 131072 + 53, 256, 8), ("q6_k", 65536 + 5, 1280, 1),
        ("i8row", 131072 + 53, 64, 1), ("i8row", 65536 + 37, 160, 4),
        ("q5_k", 65536 + 37, 256, 2), ("q5_k", 131072 + 53, 896, 1),
        ("q2_k", 65536 + 37, 256, 3), ("q3_k", 131072 + 53, 896, 1), ("q3_k", 65536 + 5, 1280, 2),
        ("i4row", 131072 + 53, 64, 1), ("i4row", 65536 + 37, 800, 3)]


@pytest.mark.parametrize("fmt,out,inf,batch", TALL)
def test_tall_matrix_every_row(fmt, out, inf, batch):
    packed, scales, x, bias = make(fmt, out, inf, 70, batch)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall {fmt} {out}x{inf} b{batch}")


def test_group_with_tall_op_equals_single_calls_bitwise():
    """The tallest op of a group sets the rows per lane group for all of
    them; small ops then run with several rows per lane group, yet every op
    gives the same bits as its own single call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for i, (out, inf) in enumerate([(131072 + 53, 896), (896, 896), (37, 896), (4864, 896)]):
        packed, _, x, bias = make("q4_k", out, inf, 80 + i, 1)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(out, dtype=torch.float32, device="cuda")
        ys = torch.empty(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        singles.append((out, inf, w_d, x_d, ys, b_d))
    dmv.pesti_gemv_group("q4_k", ops, 1)
    for out, inf, w_d, x_d, ys, b_d in singles:
        dmv.pesti_gemv_q4_k(out, inf, w_d, x_d, ys, b_d, 1)
    torch.cuda.synchronize()
    for (o, _, _, _, yg, _, _), (_, _, _, _, ys, _) in zip(ops, singles):
        assert torch.equal(yg, ys), o


@pytest.mark.parametrize("nbytes", [0, 16, 4096, 1 << 20, (1 << 22) * 4 + 48, 80 << 20])
def test_stream_read_xor(nbytes):
    """The streaming-read hook reads every byte once: the XOR of its
    per-workgroup results is the XOR of the buffer's dwords."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import _lib
    rng = np.random.default_rng([21, nbytes])
    host = rng.integers(0, 2**32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to("cuda")
    partial = torch.full((_lib.READ_GROUPS,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    dmv.pesti_stream_read(buf, nbytes, partial)
    got = np.bitwise_xor.reduce(partial.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host) if host.size else np.uint32(0)
    assert int(got) == int(want)


# ---------------------------------------------------------------------------
# matrix-core mat-vec: Q2_K, Q3_K, Q4_K, Q5_K and Q6_K ops of at least 16384 rows with
# rows of at most 1024 weights, at batch 3..8 (Q2_K, Q3_K, Q4_K, Q5_K) or 5..8 (Q6_K), x split into
# binary16 high and low parts per 32-weight block; checked on every row.
# Smaller batches of the same shapes run the vector-ALU kernel.
# ---------------------------------------------------------------------------
MFMA_ROWS = 16384
MFMA_FORMATS = ("q4_k", "q6_k", "q5_k", "q2_k", "q3_k", "q8_0")
MFMA_CASES = [(MFMA_ROWS, 896, 3), (MFMA_ROWS + 37, 896, 4), (MFMA_ROWS + 5, 32, 3),
              (MFMA_ROWS + 11, 800, 3), (20000 + 7, 1024, 8), (MFMA_ROWS + 63, 768, 5),
              (MFMA_ROWS + 1, 256, 4), (MFMA_ROWS + 29, 288, 6), (MFMA_ROWS + 50, 544, 7),
              (MFMA_ROWS + 3, 160, 8)]


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
@pytest.mark.parametrize("out,inf,batch", MFMA_CASES)
def test_mfma_every_row(fmt, out, inf, batch):
    packed, _, x, bias = make(fmt, out, inf, 90, batch)
    y = run_gemv(fmt, packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"mfma {fmt} {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
@pytest.mark.parametrize("batch", [1, 2, 3, 4, 5, 6, 7, 8])
def test_mfma_every_batch_no_bias(fmt, batch):
    out, inf = MFMA_ROWS + 37, 896
    packed, _, x, _ = make(fmt, out, inf, 91, batch, with_bias=False)
    y = run_gemv(fmt, packed, None, out, inf, x)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"mfma {fmt} b{batch}")


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
def test_mfma_one_hot_x_gives_dequantized_column(fmt):
    """x = e_j: the block of j scales x_j to an exact binary16 power of two
    times its mantissa (here 1.0), every other block is zero, so y is
    column j of the float32 dequantized W, bit-exact."""
    out, inf = MFMA_ROWS + 37, 896
    packed, _, _, _ = make(fmt, out, inf, 92)
    w32 = oracle.dequantize_f32(fmt, packed, out, inf)
    cols = [0, 1, 15, 16, 31, 32, 767, 895]
    x = np.zeros((8, inf), np.float32)
    for b, j in enumerate(cols):
        x[b, j] = 1.0
    y = run_gemv(fmt, packed, None, out, inf, x)
    for b, j in enumerate(cols):
        assert np.array_equal(y[b], w32[:, j]), j


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
@pytest.mark.parametrize("k", [3, -20, 40])
def test_mfma_power_of_two_scaling_is_exact(fmt, k):
    out, inf = MFMA_ROWS + 3, 896
    packed, _, x, _ = make(fmt, out, inf, 93, 5)
    y1 = run_gemv(fmt, packed, None, out, inf, x)
    y2 = run_gemv(fmt, packed, None, out, inf, np.ldexp(x, k).astype(np.float32))
    assert np.array_equal(y2, np.ldexp(y1, k).astype(np.float32))


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
def test_mfma_padding_bytes_do_not_matter(fmt):
    if fmt == "q8_0":
        pytest.skip("Q8_0 rows are whole 32-weight blocks: no padding bytes")
    out, inf = MFMA_ROWS + 9, 896
    packed, _, x, bias = make(fmt, out, inf, 94, 5)
    rng = np.random.default_rng(95)
    nb = {"q4_k": 144, "q6_k": 210, "q5_k": 176, "q2_k": 84, "q3_k": 110}[fmt]
    other = packed.copy().reshape(out, -1)
    last = other[:, 3 * nb:4 * nb]

    def high_nibbles(lo, hi):   # randomize bits 4-7 of bytes lo..hi-1
        last[:, lo:hi] = (last[:, lo:hi] & 0x0F) | (rng.integers(0, 16, last[:, lo:hi].shape,
                                                                  dtype=np.uint8) << 4)
    if fmt == "q2_k":   # weights 896..1023: scale bytes 8..15, code bytes 48..79
        last[:, 8:16] = rng.integers(0, 256, last[:, 8:16].shape, dtype=np.uint8)
        last[:, 48:80] = rng.integers(0, 256, last[:, 48:80].shape, dtype=np.uint8)
    elif fmt == "q3_k":   # high bits 4..7, low-bit bytes 64..95, scales 8..15
        high_nibbles(0, 32)
        last[:, 64:96] = rng.integers(0, 256, last[:, 64:96].shape, dtype=np.uint8)
        high_nibbles(96, 108)
    elif fmt == "q5_k":
        last[:, 48 + 64:] = rng.integers(0, 256, last[:, 48 + 64:].shape, dtype=np.uint8)
        last[:, 16:48] = (last[:, 16:48] & 0x0F) | (rng.integers(0, 16, last[:, 16:48].shape, dtype=np.uint8) << 4)
        last[:, 12:16] = rng.integers(0, 256, last[:, 12:16].shape, dtype=np.uint8)
        last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, last[:, 4:12].shape, dtype=np.uint8) << 6)
    elif fmt == "q4_k":
        last[:, 16 + 64:] = rng.integers(0, 256, last[:, 16 + 64:].shape, dtype=np.uint8)
        last[:, 12:16] = rng.integers(0, 256, last[:, 12:16].shape, dtype=np.uint8)
        last[:, 4:12] = (last[:, 4:12] & 0x3F) | (rng.integers(0, 4, last[:, 4:12].shape, dtype=np.uint8) << 6)
    else:
        last[:, 64:128] = rng.integers(0, 256, last[:, 64:128].shape, dtype=np.uint8)
        last[:, 160:192] = rng.integers(0, 256, last[:, 160:192].shape, dtype=np.uint8)
        last[:, 200:208] = rng.integers(0, 256, last[:, 200:208].shape, dtype=np.uint8)
    y1 = run_gemv(fmt, packed, None, out, inf, x, bias)
    y2 = run_gemv(fmt, other, None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
@pytest.mark.parametrize("d_bits", [0x0000, 0x0001, 0x0400, 0x7BFF])
def test_mfma_forced_scales(fmt, d_bits):
    rng = np.random.default_rng([96, d_bits])
    out, inf = MFMA_ROWS + 21, 512
    packed = synth.quant_blocks(fmt, rng, out, inf, force_d=d_bits)
    x = synth.activations(rng, 5, inf)
    y = run_gemv(fmt, packed, None, out, inf, x)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"mfma {fmt} d={d_bits:#06x}")


def test_mfma_q6_k_all_codes_32_is_bias():
    """q = 32 everywhere: every code enters as exactly 0, so y is the bias."""
    out, inf = MFMA_ROWS + 5, 896
    packed, _, x, bias = make("q6_k", out, inf, 99, 5)
    blocks = packed.reshape(out, -1, 210)
    blocks[:, :, 0:128] = 0x00            # low 4 bits 0
    blocks[:, :, 128:192] = 0xAA          # high 2 bits 2 (q = 32) for every g
    y = run_gemv("q6_k", packed, None, out, inf, x, bias)
    assert np.array_equal(y, np.broadcast_to(bias, y.shape))


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
@pytest.mark.parametrize("kind", ["wide_range", "tiny", "huge", "sparse"])
def test_mfma_x_dynamic_range(fmt, kind):
    """The per-block power-of-two scaling keeps the binary16 split accurate
    whatever the magnitudes: elements 2^-40 .. 2^20 mixed within a block,
    vectors near the float32 extremes, blocks of zeros beside nonzeros."""
    out, inf, batch = MFMA_ROWS + 13, 896, 5
    packed, _, x, bias = make(fmt, out, inf, 97, batch)
    rng = np.random.default_rng([98, len(kind)])
    if kind == "wide_range":
        x = (x * np.exp2(rng.integers(-40, 21, x.shape))).astype(np.float32)
    elif kind == "tiny":
        x = np.ldexp(x, -110).astype(np.float32)
    elif kind == "huge":
        x = np.ldexp(x, 80).astype(np.float32)
        bias = None
    else:
        x = np.where(rng.random(x.shape) < 0.9, np.float32(0), x).astype(np.float32)
    y = run_gemv(fmt, packed, None, out, inf, x, bias).astype(np.float64)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
    if kind == "tiny":   # compare at unit scale: the 1e-6 floor would hide everything
        y, y_ref, s_ref = np.ldexp(y, 110), np.ldexp(y_ref, 110), np.ldexp(s_ref, 110)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"mfma {fmt} x {kind}")


@pytest.mark.parametrize("fmt", MFMA_FORMATS)
def test_mfma_group_mixed_row_lengths_equals_single_calls_bitwise(fmt):
    """Tall ops of different row lengths and a short op in one group: each
    op takes the kernel its own single call takes, and the same bits."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for i, (out, inf) in enumerate([(MFMA_ROWS + 7, 896), (300, 896), (MFMA_ROWS + 100, 256),
                                    (MFMA_ROWS, 800), (MFMA_ROWS + 1, 1280)]):
        packed, _, x, bias = make(fmt, out, inf, 100 + i, 5)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(5 * out, dtype=torch.float32, device="cuda")
        ys = torch.empty(5 * out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        singles.append((out, inf, w_d, x_d, ys, b_d, packed, x, bias))
    dmv.pesti_gemv_group(fmt, ops, 5)
    single = getattr(dmv, f"pesti_gemv_{fmt}")
    for out, inf, w_d, x_d, ys, b_d, *_ in singles:
        single(out, inf, w_d, x_d, ys, b_d, 5)
    torch.cuda.synchronize()
    for (o, _, _, _, yg, _, _), (out, inf, _, _, ys, _, packed, x, bias) in zip(ops, singles):
        assert torch.equal(yg, ys), o
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
        assert_within(ys.cpu().numpy().reshape(5, out), y_ref, s_ref, GEMV_REL, f"group {out}x{inf}")


@pytest.mark.parametrize("fmt,batch", [("q4_k", 4), ("q6_k", 6), ("q5_k", 3)])
def test_mfma_group_of_eight_tall_ops(fmt, batch):
    """Eight tall ops in one grouped launch (every op slot of the grid),
    ragged row counts and two row lengths of one super-block count, each
    checked on every row against the oracle and bitwise against its single
    call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, cases = [], []
    for i in range(8):
        out, inf = MFMA_ROWS + 13 * i + (i % 3), (512 if i % 2 else 480)
        packed, _, x, bias = make(fmt, out, inf, 120 + i, batch, with_bias=(i % 4 != 1))
        w_d, x_d = to_dev(packed.reshape(-1)), to_dev(x)
        b_d = to_dev(bias) if bias is not None else None
        yg = torch.empty(batch * out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        cases.append((out, inf, w_d, x_d, b_d, packed, x, bias, yg))
    dmv.pesti_gemv_group(fmt, ops, batch)
    single = getattr(dmv, f"pesti_gemv_{fmt}")
    for out, inf, w_d, x_d, b_d, packed, x, bias, yg in cases:
        ys = torch.empty(batch * out, dtype=torch.float32, device="cuda")
        single(out, inf, w_d, x_d, ys, b_d, batch)
        torch.cuda.synchronize()
        assert torch.equal(yg, ys), (out, inf)
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
        assert_within(yg.cpu().numpy().reshape(batch, out), y_ref, s_ref, GEMV_REL, f"group8 {fmt} {out}x{inf}")


# tall per-row INT4 matrices at batch 1..8 (matrix cores from batch 2; rows of
# whole 64-weight units, some ending mid 128-weight group), every row checked
I4_TALL_CASES = [(MFMA_ROWS + 37, 896, 3), (MFMA_ROWS + 5, 800, 4), (MFMA_ROWS, 64, 8),
                 (MFMA_ROWS + 11, 1024, 5), (MFMA_ROWS + 63, 288, 6), (MFMA_ROWS + 1, 544, 7),
                 (MFMA_ROWS + 29, 32, 3), (MFMA_ROWS + 9, 896, 2), (MFMA_ROWS + 2, 320, 2),
                 (MFMA_ROWS + 4, 192, 1)]


@pytest.mark.parametrize("out,inf,batch", I4_TALL_CASES)
def test_tall_i4row_every_row(out, inf, batch):
    packed, scales, x, bias = make("i4row", out, inf, 130, batch)
    y = run_gemv("i4row", packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("i4row", packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall i4row {out}x{inf} b{batch}")


# batch 1 on the 128-weight-unit kernel (rows of whole 128-weight units;
# 800 and 192 stay on the general kernel)
@pytest.mark.parametrize("inf", [128, 256, 384, 512, 640, 768, 896, 1024, 800, 192])
def test_tall_i4row_batch_1_every_row(inf):
    out = MFMA_ROWS + 37
    packed, scales, x, bias = make("i4row", out, inf, 136, 1)
    y = run_gemv("i4row", packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("i4row", packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall i4row b1 in={inf}")


def test_tall_i4row_batch_1_one_hot_and_sparse_codes():
    out, inf = MFMA_ROWS + 5, 896
    packed, scales, x, bias = make("i4row", out, inf, 137, 1)
    w32 = oracle.dequantize_f32("i4row", packed, out, inf, scales)
    for j in (0, 1, 127, 128, 129, 255, 256, 895):
        xo = np.zeros((1, inf), np.float32)
        xo[0, j] = 1.0
        assert np.array_equal(run_gemv("i4row", packed, scales, out, inf, xo)[0], w32[:, j]), j
    rng = np.random.default_rng(138)
    p = packed.reshape(out, -1).copy()
    p[rng.random(p.shape) < 0.98] = 0
    y = run_gemv("i4row", p, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("i4row", p, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, "tall i4row sparse b1")


def test_tall_i4row_batch_1_group_equals_single_calls_bitwise():
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, cases = [], []
    for i, (out, inf) in enumerate([(MFMA_ROWS + 7, 896), (300, 896), (MFMA_ROWS + 100, 800), (MFMA_ROWS + 3, 896)]):
        packed, scales, x, bias = make("i4row", out, inf, 145 + i, 1)
        w_d, s_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(scales), to_dev(x), to_dev(bias)
        yg = torch.empty(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, s_d))
        cases.append((out, inf, w_d, s_d, x_d, b_d, yg))
    dmv.pesti_gemv_group("i4row", ops, 1)
    for out, inf, w_d, s_d, x_d, b_d, yg in cases:
        ys = torch.empty(out, dtype=torch.float32, device="cuda")
        dmv.pesti_gemv_i4row(out, inf, w_d, s_d, x_d, ys, b_d, 1)
        torch.cuda.synchronize()
        assert torch.equal(yg, ys), (out, inf)


def test_tall_i4row_one_hot_and_scaling():
    out, inf = MFMA_ROWS + 21, 800
    packed, scales, x, _ = make("i4row", out, inf, 131, 8)
    w32 = oracle.dequantize_f32("i4row", packed, out, inf, scales)
    cols = [0, 1, 2, 31, 32, 63, 64, 799]
    onehot = np.zeros((8, inf), np.float32)
    for b, j in enumerate(cols):
        onehot[b, j] = 1.0
    y = run_gemv("i4row", packed, scales, out, inf, onehot)
    for b, j in enumerate(cols):
        assert np.array_equal(y[b], w32[:, j]), j
    for nb in (2, 4):
        y1 = run_gemv("i4row", packed, scales, out, inf, x[:nb])
        y2 = run_gemv("i4row", packed, scales, out, inf, np.ldexp(x[:nb], -9).astype(np.float32))
        assert np.array_equal(y2, np.ldexp(y1, -9).astype(np.float32))


def test_tall_i4row_sparse_codes_batch_2():
    """Rows of mostly zero codes: the matrix-core kernel takes the codes
    exactly, so the result stays within the stated bound."""
    out, inf = MFMA_ROWS + 13, 896
    packed, scales, x, bias = make("i4row", out, inf, 134, 2)
    rng = np.random.default_rng(135)
    p = packed.reshape(out, -1).copy()
    p[rng.random(p.shape) < 0.98] = 0
    y = run_gemv("i4row", p, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("i4row", p, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, "tall i4row sparse b2")


def test_tall_i4row_padding_codes_do_not_matter():
    """800 = 12.5 units of 64: the last unit's second half is padding."""
    out, inf = MFMA_ROWS + 3, 800
    packed, scales, x, bias = make("i4row", out, inf, 132, 3)
    other = packed.copy().reshape(out, -1)
    rng = np.random.default_rng(133)
    other[:, 400:416] = rng.integers(0, 256, (out, 16), dtype=np.uint8)
    y1 = run_gemv("i4row", packed, scales, out, inf, x, bias)
    y2 = run_gemv("i4row", other, scales, out, inf, x, bias)
    assert np.array_equal(y1, y2)


def test_tall_i4row_group_equals_single_calls_bitwise():
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, cases = [], []
    for i, (out, inf) in enumerate([(MFMA_ROWS + 7, 896), (300, 896), (MFMA_ROWS + 100, 800), (MFMA_ROWS, 1280)]):
        packed, scales, x, bias = make("i4row", out, inf, 140 + i, 4)
        w_d, s_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(scales), to_dev(x), to_dev(bias)
        yg = torch.empty(4 * out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, s_d))
        cases.append((out, inf, w_d, s_d, x_d, b_d, packed, scales, x, bias, yg))
    dmv.pesti_gemv_group("i4row", ops, 4)
    for out, inf, w_d, s_d, x_d, b_d, packed, scales, x, bias, yg in cases:
        ys = torch.empty(4 * out, dtype=torch.float32, device="cuda")
        dmv.pesti_gemv_i4row(out, inf, w_d, s_d, x_d, ys, b_d, 4)
        torch.cuda.synchronize()
        assert torch.equal(yg, ys), (out, inf)
        y_ref, s_ref = oracle.gemv_packed("i4row", packed, out, inf, x, bias, scales)
        assert_within(ys.cpu().numpy().reshape(4, out), y_ref, s_ref, GEMV_REL, f"i4row group {out}x{inf}")


# ---------------------------------------------------------------------------
# rows of 65..128 units (one wave per row, some lanes holding two units) and
# their neighbours at 64 and 129 units, short and medium matrices: every row
# checked, ragged row counts, batches chunked to fit LDS.
# ---------------------------------------------------------------------------
LONG_ROW_CASES = [("q4_k", 896, 4864, 1), ("q4_k", 2048, 8192, 2), ("q4_k", 3, 4160, 1),
               ("q4_k", 2049, 4864, 1), ("q4_k", 700, 8256, 1),
               ("q6_k", 896, 4864, 1), ("q6_k", 897, 4864, 3), ("q6_k", 2049, 4864, 1),
               ("q8_0", 896, 4864, 1), ("q8_0", 1, 2080, 2), ("q8_0", 1537, 4096, 5),
               ("q5_k", 1000, 4864, 1), ("q2_k", 896, 4864, 1), ("q3_k", 513, 5120, 1),
               ("i8row", 896, 8192, 8), ("i4row", 2048, 4864, 4), ("i4row", 5, 4160, 1)]


@pytest.mark.parametrize("fmt,out,inf,batch", LONG_ROW_CASES)
def test_long_rows_every_row(fmt, out, inf, batch):
    packed, scales, x, bias = make(fmt, out, inf, 150, batch)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias, scales)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"long rows {fmt} {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", ["q6_k", "q8_0"])
def test_long_rows_group_equals_single_calls_bitwise(fmt):
    """A group mixing rows of 65..128 units with longer and shorter rows
    (whose lengths set the launch's lanes per row) gives every op the bits
    of its own single call."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, cases = [], []
    for i, (out, inf) in enumerate([(896, 4864), (4864, 896), (2049, 4864), (128, 8192), (300, 10240)]):
        packed, scales, x, bias = make(fmt, out, inf, 160 + i, 2)
        w_d, x_d, b_d = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yg = torch.empty(2 * out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w_d, x_d, yg, b_d, None))
        cases.append((out, inf, w_d, x_d, b_d, packed, x, bias, yg))
    dmv.pesti_gemv_group(fmt, ops, 2)
    single = getattr(dmv, f"pesti_gemv_{fmt}")
    for out, inf, w_d, x_d, b_d, packed, x, bias, yg in cases:
        ys = torch.empty(2 * out, dtype=torch.float32, device="cuda")
        single(out, inf, w_d, x_d, ys, b_d, 2)
        torch.cuda.synchronize()
        assert torch.equal(yg, ys), (out, inf)
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
        assert_within(ys.cpu().numpy().reshape(2, out), y_ref, s_ref, GEMV_REL, f"long-row group {fmt} {out}x{inf}")


# ---------------------------------------------------------------------------
# exact cancellation: d*sc*q == dmin*m in every sub-block, so every weight
# is 0 and y must be the bias within 1e-4 * |b| + 1e-6
# ---------------------------------------------------------------------------
def _cancelling_row(fmt, rng, n_super):
    """Packed bytes of one row of n_super super-blocks in which every
    weight is d*sc*q - dmin*m = 0 exactly: dmin = k d (k = 1, 3 or 5, d
    with few enough significant bits that k d is a binary16 value), and in
    every sub-block one constant code c with sc = k s, m = c s."""
    import packing
    blocks = []
    for _ in range(n_super):
        k = int(rng.choice([1, 3, 5]))
        d_val = max(float(np.float16(abs(rng.normal(0.0, np.sqrt(1e-3))))), 2.0 ** -12)
        mant, ex = np.frexp(d_val)
        d_val = float(np.ldexp(np.round(mant * 256) / 256, ex))      # 8 significant bits
        d, dmin = packing.f16_bits(d_val), packing.f16_bits(k * d_val)
        assert float(np.uint16(dmin).view(np.float16)) == k * float(np.uint16(d).view(np.float16))
        if fmt in ("q4_k", "q5_k"):
            cmax, smax_bits = (15 if fmt == "q4_k" else 31), 63
            sc, m, q = [], [], []
            for _ in range(8):
                c = int(rng.integers(1, cmax + 1))
                s_ = int(rng.integers(1, max(1, min(smax_bits // k, 63 // c)) + 1))
                sc.append(k * s_)
                m.append(c * s_)
                q += [c] * 32
            pack = packing.pack_q4_k_block if fmt == "q4_k" else packing.pack_q5_k_block
            blocks.append(pack(d, dmin, sc, m, q))
        else:
            sc, m, cs = [], [], []
            for _ in range(16):
                c = int(rng.integers(1, 4))
                s_ = int(rng.integers(1, max(1, min(15 // k, 15 // c)) + 1))
                sc.append(k * s_)
                m.append(c * s_)
                cs.append(c)
            q = [0] * 256
            for h in range(2):
                for j in range(4):
                    for c2 in range(2):
                        for l in range(16):
                            q[128 * h + 32 * j + 16 * c2 + l] = cs[8 * h + 2 * j + c2]
            blocks.append(packing.pack_q2_k_block(d, dmin, sc, m, q))
    return np.frombuffer(b"".join(blocks), np.uint8)


CANCEL_CASES = [(40, 896, 1), (40, 896, 3), (40, 4864, 1), (40, 4864, 3), (MFMA_ROWS + 5, 896, 3),
                (MFMA_ROWS + 5, 896, 1)]


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q2_k"])
@pytest.mark.parametrize("out,inf,batch", CANCEL_CASES)
def test_exact_cancellation_gives_bias(fmt, out, inf, batch):
    """Rows whose weights are all exactly zero through d*sc*q == dmin*m:
    the vector-ALU kernels (40 rows) and the matrix-core kernels (tall, at
    batch 3) must return the bias within the bound's 1e-6 floor."""
    rng = np.random.default_rng([31, len(fmt), inf, batch])
    n_super = -(-inf // 256)
    distinct = np.stack([_cancelling_row(fmt, rng, n_super) for _ in range(48)])
    packed = np.resize(distinct, (out, distinct.shape[1]))
    x = synth.activations(rng, batch, inf)
    bias = synth.bias(rng, out)
    w64 = oracle.dequantize(fmt, distinct, 48, inf)
    assert not np.any(w64), "fixture: every weight must be exactly zero"
    y = run_gemv(fmt, packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} cancelling {out}x{inf} b{batch}")


@pytest.mark.parametrize("fmt", ["q4_k", "q5_k", "q2_k"])
@pytest.mark.parametrize("m,k,n", [(16, 896, 70), (33, 4864, 64), (16, 896, 16400), (64, 512, 16385)])
def test_gemm_quant_exact_cancellation_gives_bias(fmt, m, k, n):
    """The quantized small-M GEMM (K-split kernel for narrow layers, wide
    kernel from 1024 / 256 column tiles) on rows whose weights are all
    exactly zero: Y must be the bias within 1e-4 * |b| + 1e-6."""
    rng = np.random.default_rng([32, len(fmt), k, n])
    n_super = -(-k // 256)
    distinct = np.stack([_cancelling_row(fmt, rng, n_super) for _ in range(40)])
    packed = np.resize(distinct, (n, distinct.shape[1]))
    x16 = synth.f16_activations(rng, m, k)
    bias = synth.bias(rng, n)
    y = run_gemm_quant(fmt, packed, m, n, k, x16, bias)
    y_ref, s_ref = oracle.gemm_packed(fmt, packed, n, k, x16, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"{fmt} gemm cancelling m{m} k{k} n{n}")


# ---------------------------------------------------------------------------
# tall Q4_K, Q5_K and Q2_K matrices at batch 1: the 128-weight-unit kernel
# (rows of at most 1024 weights, at least 16384 rows)
# ---------------------------------------------------------------------------
TALL_ROWS = 16384
TALL_FORMATS = ("q4_k", "q5_k", "q2_k", "q3_k")


@pytest.mark.parametrize("fmt", TALL_FORMATS)
@pytest.mark.parametrize("inf", [128, 256, 384, 512, 640, 768, 800, 896, 1024])
def test_tall_batch_1_every_row(fmt, inf):
    out = TALL_ROWS + 37
    packed, scales, x, bias = make(fmt, out, inf, 140, 1)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall {fmt} b1 in={inf}")


@pytest.mark.parametrize("fmt", TALL_FORMATS)
def test_tall_batch_1_one_hot_gives_dequantized_column(fmt):
    out, inf = TALL_ROWS + 5, 896
    packed, _, _, _ = make(fmt, out, inf, 141)
    w32 = oracle.dequantize_f32(fmt, packed, out, inf)
    for j in (0, 31, 32, 63, 64, 127, 128, 255, 256, 895):
        x = np.zeros((1, inf), np.float32)
        x[0, j] = 1.0
        y = run_gemv(fmt, packed, None, out, inf, x)
        assert np.array_equal(y[0], w32[:, j]), j


@pytest.mark.parametrize("fmt", TALL_FORMATS)
@pytest.mark.parametrize("d_bits", [0x0000, 0x0001, 0x0400, 0x7BFF])
def test_tall_batch_1_forced_scales(fmt, d_bits):
    rng = np.random.default_rng([142, d_bits])
    out, inf = TALL_ROWS + 11, 768
    packed = synth.quant_blocks(fmt, rng, out, inf, force_d=d_bits)
    x = synth.activations(rng, 1, inf)
    y = run_gemv(fmt, packed, None, out, inf, x)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall {fmt} b1 d={d_bits:#x}")


def test_tall_q4_k_batch_1_padding_bytes_do_not_matter():
    out, inf = TALL_ROWS + 3, 800
    packed, _, x, bias = make("q4_k", out, inf, 143, 1)
    other = packed.copy().reshape(out, 4, 144)
    rng = np.random.default_rng(144)
    # super-block 3 holds weights 768..1023: 768..799 are real (sub-block 0);
    # sub-blocks 1..7's codes (low nibbles of bytes 16..47 beyond the first
    # 32 weights, and everything from byte 48) are padding
    other[:, 3, 48:] = rng.integers(0, 256, (out, 96), dtype=np.uint8)
    other[:, 3, 16:48] = (other[:, 3, 16:48] & 0x0F) | (rng.integers(0, 16, (out, 32), dtype=np.uint8) << 4)
    y1 = run_gemv("q4_k", packed, None, out, inf, x, bias)
    y2 = run_gemv("q4_k", other.reshape(out, -1), None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


def test_tall_q5_k_batch_1_padding_bytes_do_not_matter():
    out, inf = TALL_ROWS + 3, 800
    packed, _, x, bias = make("q5_k", out, inf, 146, 1)
    other = packed.copy().reshape(out, 4, 176)
    rng = np.random.default_rng(147)
    # super-block 3 holds weights 768..1023: 768..799 are real (run 0, low
    # nibbles of bytes 48..79, fifth bit 0 of bytes 16..47); every other
    # code bit of it is padding
    other[:, 3, 80:] = rng.integers(0, 256, (out, 96), dtype=np.uint8)
    other[:, 3, 48:80] = (other[:, 3, 48:80] & 0x0F) | (rng.integers(0, 16, (out, 32), dtype=np.uint8) << 4)
    other[:, 3, 16:48] = (other[:, 3, 16:48] & 0x01) | (rng.integers(0, 128, (out, 32), dtype=np.uint8) << 1)
    y1 = run_gemv("q5_k", packed, None, out, inf, x, bias)
    y2 = run_gemv("q5_k", other.reshape(out, -1), None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


def test_tall_q2_k_batch_1_padding_bytes_do_not_matter():
    out, inf = TALL_ROWS + 3, 800
    packed, _, x, bias = make("q2_k", out, inf, 148, 1)
    other = packed.copy().reshape(out, 4, 84)
    rng = np.random.default_rng(149)
    # super-block 3 holds weights 768..1023: 768..799 are real (half 0, bits
    # 0-1 of code bytes 16..47, scale bytes 0 and 1); every other code bit
    # and scale byte of it is padding (d, dmin at 80..83 are shared)
    other[:, 3, 48:80] = rng.integers(0, 256, (out, 32), dtype=np.uint8)
    other[:, 3, 16:48] = (other[:, 3, 16:48] & 0x03) | (rng.integers(0, 64, (out, 32), dtype=np.uint8) << 2)
    other[:, 3, 2:16] = rng.integers(0, 256, (out, 14), dtype=np.uint8)
    y1 = run_gemv("q2_k", packed, None, out, inf, x, bias)
    y2 = run_gemv("q2_k", other.reshape(out, -1), None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


def test_tall_q3_k_batch_1_padding_bytes_do_not_matter():
    out, inf = TALL_ROWS + 3, 800
    packed, _, x, bias = make("q3_k", out, inf, 160, 1)
    other = packed.copy().reshape(out, 4, 110)
    rng = np.random.default_rng(161)
    # super-block 3 holds weights 768..1023: 768..799 are real (half 0, field
    # j = 0: bits 0-1 of qs bytes 32..63, bit 0 of hmask bytes 0..31, the
    # scales of sub-blocks 0 and 1: low nibbles of scale bytes 0 and 1, bits
    # 0-1 of scale bytes 8 and 9); every other code and scale bit is padding
    # (d at 108..109 is shared)
    r = lambda hi, n: rng.integers(0, hi, (out, n), dtype=np.uint8)
    other[:, 3, 64:96] = r(256, 32)
    other[:, 3, 32:64] = (other[:, 3, 32:64] & 0x03) | (r(64, 32) << 2)
    other[:, 3, 0:32] = (other[:, 3, 0:32] & 0x01) | (r(128, 32) << 1)
    other[:, 3, 96:98] = (other[:, 3, 96:98] & 0x0F) | (r(16, 2) << 4)
    other[:, 3, 98:104] = r(256, 6)
    other[:, 3, 104:106] = (other[:, 3, 104:106] & 0x03) | (r(64, 2) << 2)
    other[:, 3, 106:108] = r(256, 2)
    y1 = run_gemv("q3_k", packed, None, out, inf, x, bias)
    y2 = run_gemv("q3_k", other.reshape(out, -1), None, out, inf, x, bias)
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("fmt", TALL_FORMATS)
def test_tall_batch_1_group_equals_single_calls_bitwise(fmt):
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    cases = [(TALL_ROWS + 7, 896), (TALL_ROWS + 100, 896), (TALL_ROWS + 1, 512), (300, 896)]
    ops, singles = [], []
    for n, (out, inf) in enumerate(cases):
        packed, _, x, bias = make(fmt, out, inf, 150 + n, 1)
        singles.append(run_gemv(fmt, packed, None, out, inf, x, bias))
        w, xd, bd = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yd = torch.zeros(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w, xd, yd, bd, None))
    dmv.pesti_gemv_group(fmt, ops, 1)
    torch.cuda.synchronize()
    for (out, inf, w, xd, yd, bd, _), y1 in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy(), y1[0])


# batch 2 on the same kernel: each dequantized weight feeds both columns
@pytest.mark.parametrize("fmt", TALL_FORMATS + ("q4_k_stream",))
@pytest.mark.parametrize("inf", [128, 384, 896, 1024, 800])
def test_tall_batch_2_every_row(fmt, inf):
    if fmt == "q4_k_stream" and inf % 128:
        pytest.skip("the stream layout's tall rows are whole 128-weight units")
    out = TALL_ROWS + 29
    packed, scales, x, bias = make(fmt, out, inf, 170, 2)
    y = run_gemv(fmt, packed, scales, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall {fmt} b2 in={inf}")


@pytest.mark.parametrize("fmt", TALL_FORMATS)
def test_tall_batch_2_one_hot_columns_and_group_bitwise(fmt):
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    out, inf = TALL_ROWS + 5, 896
    packed, _, _, _ = make(fmt, out, inf, 171)
    w32 = oracle.dequantize_f32(fmt, packed, out, inf)
    for j0, j1 in ((0, 895), (127, 128), (255, 256)):
        x = np.zeros((2, inf), np.float32)
        x[0, j0] = 1.0
        x[1, j1] = 1.0
        y = run_gemv(fmt, packed, None, out, inf, x)
        assert np.array_equal(y[0], w32[:, j0]) and np.array_equal(y[1], w32[:, j1]), (j0, j1)
    ops, singles = [], []
    for n, (o, i) in enumerate([(TALL_ROWS + 7, 896), (300, 896), (TALL_ROWS + 1, 512)]):
        pk, _, x, bias = make(fmt, o, i, 172 + n, 2)
        w, xd, bd = to_dev(pk.reshape(-1)), to_dev(x), to_dev(bias)
        yd = torch.zeros(2 * o, dtype=torch.float32, device="cuda")
        ops.append((o, i, w, xd, yd, bd, None))
        singles.append(run_gemv(fmt, pk, None, o, i, x, bias))
    dmv.pesti_gemv_group(fmt, ops, 2)
    torch.cuda.synchronize()
    for (o, _, _, _, yd, _, _), ys in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy().reshape(2, o), ys), o


@pytest.mark.parametrize("fmt", TALL_FORMATS)
def test_tall_batch_1_full_lm_head_sampled_rows(fmt):
    out, inf = synth.QWEN_VOCAB, 896
    rng = np.random.default_rng([145, out, inf])
    packed, _ = synth.matrix(fmt, rng, out, inf)
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv(fmt, packed, None, out, inf, x, bias)
    rows = np.unique(np.concatenate([rng.integers(0, out, 2048), [0, out - 1]]))
    y_ref, s_ref = oracle.gemv_packed(fmt, packed.reshape(out, -1)[rows], len(rows), inf, x, bias[rows])
    assert_within(y[:, rows], y_ref, s_ref, GEMV_REL, f"{fmt} lm head b1")


# ---------------------------------------------------------------------------
# Q4_K stream layout (the byte-minimal layout of 896-weight rows)
# ---------------------------------------------------------------------------
STREAM_DEQUANT = [(2, 128), (3, 384), (7, 896), (33, 896), (5, 4864), (1, 64), (9, 192)]


@pytest.mark.parametrize("rows,inf", STREAM_DEQUANT)
def test_stream_dequant_bit_exact(rows, inf):
    rng = np.random.default_rng([160, rows, inf])
    packed = synth.stream_blocks(rng, rows, inf)
    got = run_dequant("q4_k_stream", packed, None, rows, inf)
    assert np.array_equal(got, oracle.dequantize_f32("q4_k_stream", packed, rows, inf))


STREAM_GEMV = [(67, 896, 1), (67, 896, 3), (67, 896, 8), (1152, 896, 1), (4864, 896, 1), (300, 64, 1),
               (37, 192, 2), (130, 4864, 2), (11, 20480, 1), (MFMA_ROWS + 37, 896, 1), (MFMA_ROWS + 37, 896, 4),
               (77, 192, 1), (65, 1024, 1), (3, 960, 1), (130, 4864, 1), (5, 1088, 1)]


@pytest.mark.parametrize("out,inf,batch", STREAM_GEMV)
def test_stream_gemv_parity(out, inf, batch):
    rng = np.random.default_rng([161, out, inf, batch])
    packed = synth.stream_blocks(rng, out, inf)
    x = synth.activations(rng, batch, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q4_k_stream", packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("q4_k_stream", packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"q4_k_stream {out}x{inf} b{batch}")


def test_stream_one_hot_x_gives_dequantized_column():
    out, inf = 129, 896
    rng = np.random.default_rng(162)
    packed = synth.stream_blocks(rng, out, inf)
    w32 = oracle.dequantize_f32("q4_k_stream", packed, out, inf)
    cols = [0, 1, 127, 128, 255, 256, 640, 895]
    x = np.zeros((8, inf), np.float32)
    for b, j in enumerate(cols):
        x[b, j] = 1.0
    y = run_gemv("q4_k_stream", packed, None, out, inf, x)
    for b, j in enumerate(cols):
        assert np.array_equal(y[b], w32[:, j]), j


@pytest.mark.parametrize("out,inf", [(129, 896), (37, 512), (21, 1024), (9, 960)])
def test_stream_batch_1_one_hot_gives_dequantized_column(out, inf):
    """Batch 1 takes the half-unit stream kernel for rows of at most 1024
    weights: every sampled column comes back bit for bit."""
    rng = np.random.default_rng([167, out, inf])
    packed = synth.stream_blocks(rng, out, inf)
    w32 = oracle.dequantize_f32("q4_k_stream", packed, out, inf)
    for j in sorted({0, 1, 15, 16, 31, 32, 63, 64, 127, 128, 255, 256, inf - 1}):
        if j >= inf:
            continue
        x = np.zeros((1, inf), np.float32)
        x[0, j] = 1.0
        y = run_gemv("q4_k_stream", packed, None, out, inf, x)
        assert np.array_equal(y[0], w32[:, j]), j


def test_stream_batch_1_padding_at_the_end_does_not_matter():
    out, inf = 45, 896
    rng = np.random.default_rng(168)
    packed = synth.stream_blocks(rng, out, inf)
    other = packed.copy()
    other[-64:] = rng.integers(0, 256, 64, dtype=np.uint8)
    other[-144 + 12:-144 + 16] = rng.integers(0, 256, 4, dtype=np.uint8)
    x = synth.activations(rng, 1, inf)
    assert np.array_equal(run_gemv("q4_k_stream", packed, None, out, inf, x),
                          run_gemv("q4_k_stream", other, None, out, inf, x))


def test_stream_batch_1_group_of_short_rows_equals_single_calls_bitwise():
    """The step's Q/K/V and gate/up shapes in one grouped launch (half units)."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for n, (out, inf) in enumerate([(896, 896), (128, 896), (128, 896), (4864, 896), (35, 512)]):
        rng = np.random.default_rng([169, n])
        packed = synth.stream_blocks(rng, out, inf)
        x, bias = synth.activations(rng, 1, inf), synth.bias(rng, out)
        singles.append(run_gemv("q4_k_stream", packed, None, out, inf, x, bias))
        w, xd, bd = to_dev(packed), to_dev(x), to_dev(bias)
        yd = torch.zeros(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w, xd, yd, bd, None))
    dmv.pesti_gemv_group("q4_k_stream", ops, 1)
    torch.cuda.synchronize()
    for (out, inf, w, xd, yd, bd, _), y1 in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy(), y1[0])


def test_stream_padding_at_the_end_does_not_matter():
    out, inf = 45, 896           # 40320 weights: 157.5 super-blocks, the last half padding
    rng = np.random.default_rng(163)
    packed = synth.stream_blocks(rng, out, inf)
    other = packed.copy()
    other[-64:] = rng.integers(0, 256, 64, dtype=np.uint8)     # runs 2-3 of the last block
    other[-144 + 12:-144 + 16] = rng.integers(0, 256, 4, dtype=np.uint8)   # sub-blocks 4-7's scale bytes
    x = synth.activations(rng, 2, inf)
    assert np.array_equal(run_gemv("q4_k_stream", packed, None, out, inf, x),
                          run_gemv("q4_k_stream", other, None, out, inf, x))


def test_stream_forced_scales():
    for d_bits in (0x0000, 0x0001, 0x0400, 0x7BFF):
        rng = np.random.default_rng([164, d_bits])
        out, inf = 23, 896
        packed = synth.stream_blocks(rng, out, inf, force_d=d_bits)
        x = synth.activations(rng, 1, inf)
        y = run_gemv("q4_k_stream", packed, None, out, inf, x)
        y_ref, s_ref = oracle.gemv_packed("q4_k_stream", packed, out, inf, x)
        assert_within(y, y_ref, s_ref, GEMV_REL, f"stream d={d_bits:#x}")


def test_stream_group_equals_single_calls_bitwise():
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles = [], []
    for n, (out, inf) in enumerate([(896, 896), (128, 896), (128, 896), (33, 4864)]):
        rng = np.random.default_rng([165, n])
        packed = synth.stream_blocks(rng, out, inf)
        x, bias = synth.activations(rng, 1, inf), synth.bias(rng, out)
        singles.append(run_gemv("q4_k_stream", packed, None, out, inf, x, bias))
        w, xd, bd = to_dev(packed), to_dev(x), to_dev(bias)
        yd = torch.zeros(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w, xd, yd, bd, None))
    dmv.pesti_gemv_group("q4_k_stream", ops, 1)
    torch.cuda.synchronize()
    for (out, inf, w, xd, yd, bd, _), y1 in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy(), y1[0])


def test_stream_exact_cancellation_gives_bias():
    """Stream rows whose weights are all exactly zero (every sub-block's
    codes one constant c with d sc c = dmin m)."""
    out, inf = 40, 896
    rng = np.random.default_rng(166)
    nsb = -(-out * inf // 256)
    packed = _cancelling_row("q4_k", rng, nsb)
    assert not np.any(oracle.dequantize("q4_k_stream", packed, out, inf))
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q4_k_stream", packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("q4_k_stream", packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, "stream cancelling")


# ---------------------------------------------------------------------------
# tall Q4_K matrices in the stream layout at batch 1: the 128-weight-unit
# kernel when rows are a whole number of units (a unit is then half of one
# stream super-block), the general stream kernel otherwise
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("inf", [128, 256, 384, 640, 896, 1024, 960, 192])
def test_tall_stream_batch_1_every_row(inf):
    out = TALL_ROWS + 37            # odd row count: with 896 the stream ends on a half super-block
    rng = np.random.default_rng([170, inf])
    packed = synth.stream_blocks(rng, out, inf)
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q4_k_stream", packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("q4_k_stream", packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, f"tall q4_k_stream b1 in={inf}")


def test_tall_stream_batch_1_one_hot_gives_dequantized_column():
    out, inf = TALL_ROWS + 5, 896
    rng = np.random.default_rng(171)
    packed = synth.stream_blocks(rng, out, inf)
    w32 = oracle.dequantize_f32("q4_k_stream", packed, out, inf)
    for j in (0, 31, 32, 127, 128, 255, 256, 895):
        x = np.zeros((1, inf), np.float32)
        x[0, j] = 1.0
        y = run_gemv("q4_k_stream", packed, None, out, inf, x)
        assert np.array_equal(y[0], w32[:, j]), j


def test_tall_stream_batch_1_padding_at_the_end_does_not_matter():
    out, inf = TALL_ROWS + 1, 896   # 14681 stream units: the last super-block's second half is padding
    rng = np.random.default_rng(172)
    packed = synth.stream_blocks(rng, out, inf)
    other = packed.copy()
    other[-64:] = rng.integers(0, 256, 64, dtype=np.uint8)
    other[-144 + 12:-144 + 16] = rng.integers(0, 256, 4, dtype=np.uint8)
    x = synth.activations(rng, 1, inf)
    assert np.array_equal(run_gemv("q4_k_stream", packed, None, out, inf, x),
                          run_gemv("q4_k_stream", other, None, out, inf, x))


def test_tall_stream_batch_1_exact_cancellation_gives_bias():
    out, inf = TALL_ROWS + 3, 896
    rng = np.random.default_rng(173)
    packed = _cancelling_row("q4_k", rng, -(-out * inf // 256))
    assert not np.any(oracle.dequantize("q4_k_stream", packed, out, inf))
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q4_k_stream", packed, None, out, inf, x, bias)
    y_ref, s_ref = oracle.gemv_packed("q4_k_stream", packed, out, inf, x, bias)
    assert_within(y, y_ref, s_ref, GEMV_REL, "tall stream cancelling")


def test_tall_stream_batch_1_group_equals_single_calls_bitwise():
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    cases = [(TALL_ROWS + 7, 896), (TALL_ROWS + 100, 896), (TALL_ROWS + 1, 512), (TALL_ROWS + 2, 960),
             (300, 896)]
    ops, singles = [], []
    for n, (out, inf) in enumerate(cases):
        rng = np.random.default_rng([174, n])
        packed = synth.stream_blocks(rng, out, inf)
        x, bias = synth.activations(rng, 1, inf), synth.bias(rng, out)
        singles.append(run_gemv("q4_k_stream", packed, None, out, inf, x, bias))
        w, xd, bd = to_dev(packed), to_dev(x), to_dev(bias)
        yd = torch.zeros(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w, xd, yd, bd, None))
    dmv.pesti_gemv_group("q4_k_stream", ops, 1)
    torch.cuda.synchronize()
    for (out, inf, w, xd, yd, bd, _), y1 in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy(), y1[0])


def test_tall_stream_batch_1_full_lm_head_sampled_rows():
    out, inf = synth.QWEN_VOCAB, 896
    rng = np.random.default_rng([175, out, inf])
    packed = synth.stream_blocks(rng, out, inf)
    x = synth.activations(rng, 1, inf)
    bias = synth.bias(rng, out)
    y = run_gemv("q4_k_stream", packed, None, out, inf, x, bias)
    # rows 2k and 2k + 1 share their middle super-block: check sampled pairs
    # through the oracle on the slice of the stream that holds them
    # (7 units of 128 weights per row, 2 units per 144-byte super-block)
    starts = np.unique(np.concatenate([rng.integers(0, out // 2, 512) * 2, [0, out - 2]]))
    for r0 in starts:
        sb0 = (r0 * 7) // 2
        sb1 = -(-((r0 + 2) * 7) // 2)
        sub = packed[sb0 * 144: sb1 * 144]
        y_ref, s_ref = oracle.gemv_packed("q4_k_stream", sub, 2, inf, x, bias[r0:r0 + 2])
        assert_within(y[:, r0:r0 + 2], y_ref, s_ref, GEMV_REL, f"stream lm head rows {r0}, {r0 + 1}")


@pytest.mark.parametrize("fmt", ["q4_k", "q4_k_stream"])
def test_half_unit_row_limit_group_equals_single_calls_bitwise(fmt):
    """Ops of 2048 rows take half units at batch 1 and ops of 2049 rows
    whole runs; in one group each keeps the bits of its own single call,
    and every output meets the oracle's bound."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from gpu_util import to_dev
    ops, singles, cases = [], [], []
    for n, (out, inf) in enumerate([(2048, 896), (2049, 896), (2048, 512), (7, 1024)]):
        rng = np.random.default_rng([176, n])
        packed, _ = synth.matrix(fmt, rng, out, inf)
        x, bias = synth.activations(rng, 1, inf), synth.bias(rng, out)
        y1 = run_gemv(fmt, packed, None, out, inf, x, bias)
        y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, bias)
        assert_within(y1, y_ref, s_ref, GEMV_REL, f"{fmt} {out}x{inf}")
        singles.append(y1)
        w, xd, bd = to_dev(packed.reshape(-1)), to_dev(x), to_dev(bias)
        yd = torch.zeros(out, dtype=torch.float32, device="cuda")
        ops.append((out, inf, w, xd, yd, bd, None))
    dmv.pesti_gemv_group(fmt, ops, 1)
    torch.cuda.synchronize()
    for (out, inf, w, xd, yd, bd, _), y1 in zip(ops, singles):
        assert np.array_equal(yd.cpu().numpy(), y1[0]), (out, inf)
