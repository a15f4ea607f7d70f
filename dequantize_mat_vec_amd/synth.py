"""Seeded synthetic inputs for the quantized mat-vec path.

This module draws random numbers and places them at their byte offsets; it
holds none of the path's arithmetic (no dequantization, no dot products), so
both the HIP library's tests and the CPU oracle can be fed from it.

Workloads (the pages' models are not available, so seeded random tensors of
their shapes stand in for them):
* Qwen2.5-0.5B decode step: hidden 896, 24 layers, 14 query heads and 2 KV
  heads of 64 ("PESTI ..." README, section "Conformance"), FFN 4864,
  vocabulary 151936 (tied head).
* GPT-2 124M linear layers at prompt width ("inferno" README, section
  "Benchmarks": c_attn 768x2304, c_proj 768x768, mlp_fc 768x3072).

Distributions:
* block scales d (and dmin): binary16 of |N(0, 1e-3)| (variance 1e-3),
  rounded to nearest-even by numpy;
* every other byte of a block is uniform over 0..255, which makes the Q4_K
  6-bit scales/mins uniform over 0..63 and its codes uniform over 0..15, the
  Q6_K codes uniform over 0..63 and its int8 scales uniform over -128..127,
  and the Q8_0 codes uniform over -128..127;
* bytes of padding sub-blocks (rows padded to whole 256-weight super-blocks)
  are random too: results must not depend on them;
* per-row int8: one row w ~ N(0, 0.02^2) in float32 sets scale =
  max|w| / 127, and the codes are drawn independently, uniform in -127..127;
* x ~ N(0, 1) float32, bias ~ N(0, 0.02^2) float32, binary16 GEMM weights
  ~ N(0, 0.02^2) and activations ~ N(0, 1).
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20261202
D_VARIANCE = 1e-3

# Block geometry: (weights per block, bytes per block, byte offsets of the
# binary16 scale fields inside the block).
_GEOMETRY = {
    "q8_0": (32, 34, (0,)),
    "q2_k": (256, 84, (80, 82)),
    "q3_k": (256, 110, (108,)),
    "q4_k": (256, 144, (0, 2)),
    "q5_k": (256, 176, (0, 2)),
    "q6_k": (256, 210, (208,)),
}

FORMATS = ("q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k", "i8row", "i4row")


def rng_for(config_idx: int, layer_idx: int = 0, tensor_idx: int = 0,
            base: int = SEED_BASE) -> np.random.Generator:
    """Generator seeded by (base, config, layer, tensor)."""
    return np.random.default_rng([base, config_idx, layer_idx, tensor_idx])


def packed_row_bytes(fmt: str, in_features: int) -> int:
    """Bytes per packed row (whole blocks); i8row rows are in_features bytes,
    i4row rows 32 bytes per 64 weights."""
    if fmt == "i8row":
        return in_features
    if fmt == "i4row":
        return -(-in_features // 64) * 32
    qk, nbytes, _ = _GEOMETRY[fmt]
    return -(-in_features // qk) * nbytes


def f16_abs_normal(rng: np.random.Generator, shape, variance: float = D_VARIANCE) -> np.ndarray:
    """binary16 bit patterns (uint16) of |N(0, variance)|."""
    v = np.abs(rng.normal(0.0, np.sqrt(variance), size=shape))
    return v.astype(np.float16).view(np.uint16)


def quant_blocks(fmt: str, rng: np.random.Generator, rows: int, in_features: int,
                 force_d=None) -> np.ndarray:
    """Packed [rows, row_bytes] uint8 matrix in Q8_0 or a K-family format.

    force_d: optional binary16 bit pattern (or array of patterns, cycled over
    the blocks) written into every scale field instead of random draws - used
    to force zero, subnormal and maximal scales."""
    if in_features <= 0 or in_features % 32:
        raise ValueError("in_features must be a positive multiple of 32")
    qk, nbytes, d_offsets = _GEOMETRY[fmt]
    nblk = -(-in_features // qk)
    raw = rng.integers(0, 256, size=(rows, nblk, nbytes), dtype=np.uint8)
    for off in d_offsets:
        if force_d is None:
            bits = f16_abs_normal(rng, (rows, nblk))
        else:
            pats = np.atleast_1d(np.asarray(force_d, dtype=np.uint16))
            bits = np.resize(pats, rows * nblk).reshape(rows, nblk)
        raw[:, :, off] = (bits & 0xFF).astype(np.uint8)
        raw[:, :, off + 1] = (bits >> 8).astype(np.uint8)
    return raw.reshape(rows, nblk * nbytes)


def stream_blocks(rng: np.random.Generator, rows: int, in_features: int, force_d=None) -> np.ndarray:
    """Packed bytes (flat uint8) of a Q4_K matrix in the stream layout: the
    row-major weights cut into ceil(rows * in / 256) super-blocks in order,
    each drawn as quant_blocks draws a Q4_K block (the padding weights at
    the end of the stream are random too)."""
    nsb = -(-(rows * in_features) // 256)
    return quant_blocks("q4_k", rng, 1, nsb * 256, force_d).reshape(-1)


def i8row(rng: np.random.Generator, rows: int, in_features: int):
    """(int8 codes [rows, in], float32 scales [rows]) for the per-row format."""
    w = rng.normal(0.0, 0.02, size=(rows, in_features)).astype(np.float32)
    scales = (np.max(np.abs(w), axis=1).astype(np.float64) / 127.0).astype(np.float32)
    codes = rng.integers(-127, 128, size=(rows, in_features), dtype=np.int64).astype(np.int8)
    return codes, scales


def activations(rng: np.random.Generator, batch: int, n: int) -> np.ndarray:
    """x ~ N(0, 1) float32 [batch, n]."""
    return rng.standard_normal(size=(batch, n)).astype(np.float32)


def bias(rng: np.random.Generator, n: int) -> np.ndarray:
    """bias ~ N(0, 0.02^2) float32 [n]."""
    return rng.normal(0.0, 0.02, size=n).astype(np.float32)


def f16_weights(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """binary16 weights ~ N(0, 0.02^2), [rows, cols]."""
    return rng.normal(0.0, 0.02, size=(rows, cols)).astype(np.float16)


def f16_activations(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """binary16 activations ~ N(0, 1), [rows, cols]."""
    return rng.standard_normal(size=(rows, cols)).astype(np.float16)


def i4row(rng: np.random.Generator, rows: int, in_features: int):
    """(packed uint8 [rows, ceil(in/64)*32], float32 scales [rows]) for the
    per-row int4 format: random bytes (every code -8..7, padding included)
    and scale = max|w| / 7 of one w ~ N(0, 0.02^2) row."""
    rb = -(-in_features // 64) * 32
    w = rng.normal(0.0, 0.02, size=(rows, in_features)).astype(np.float32)
    scales = (np.max(np.abs(w), axis=1).astype(np.float64) / 7.0).astype(np.float32)
    return rng.integers(0, 256, size=(rows, rb), dtype=np.uint8), scales


def matrix(fmt: str, rng: np.random.Generator, rows: int, in_features: int):
    """(packed bytes, scales-or-None) for any format; i8row codes are returned
    as a uint8 view so every format travels as bytes."""
    if fmt == "i8row":
        codes, scales = i8row(rng, rows, in_features)
        return codes.view(np.uint8), scales
    if fmt == "i4row":
        return i4row(rng, rows, in_features)
    if fmt == "q4_k_stream":
        return stream_blocks(rng, rows, in_features), None
    return quant_blocks(fmt, rng, rows, in_features), None


# ---------------------------------------------------------------------------
# Workload shapes
# ---------------------------------------------------------------------------
QWEN_HIDDEN = 896
QWEN_FFN = 4864
QWEN_KV_OUT = 128          # 2 KV heads x 64
QWEN_LAYERS = 24
QWEN_VOCAB = 151936
GPT2_HIDDEN = 768
GPT2_VOCAB = 50257

# (name, out_features, in_features, has_bias) per decoder layer, in call order.
QWEN_LAYER_CALLS = (
    ("q", QWEN_HIDDEN, QWEN_HIDDEN, True),
    ("k", QWEN_KV_OUT, QWEN_HIDDEN, True),
    ("v", QWEN_KV_OUT, QWEN_HIDDEN, True),
    ("o", QWEN_HIDDEN, QWEN_HIDDEN, False),
    ("gate", QWEN_FFN, QWEN_HIDDEN, False),
    ("up", QWEN_FFN, QWEN_HIDDEN, False),
    ("down", QWEN_HIDDEN, QWEN_FFN, False),
)
TENSOR_INDEX = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6,
                "lm_head": 7, "bias": 8, "x": 9}

# GPT-2 linear layers as (name, in_features K, out_features N).
GPT2_LINEARS = (
    ("c_attn", 768, 2304),
    ("c_proj", 768, 768),
    ("mlp_fc", 768, 3072),
    ("mlp_proj", 3072, 768),
)


def decode_step_calls(layers: int = QWEN_LAYERS, layout: str = "rows"):
    """The decode step's mat-vec calls in stream order:
    [(layer, name, fmt, out, in, has_bias)].  Every layer's projections are
    Q4_K, except that the FFN down projection is Q6_K on even layers
    (0, 2, ..., 22); the step ends with the tied Q8_0 LM head.  With layout
    "stream" the Q4_K matrices of rows that are not whole super-blocks (the
    896-column Q, K, V, O, gate and up) are in the Q4_K stream layout."""
    if layout not in ("rows", "stream"):
        raise ValueError(f"unknown layout {layout!r}")
    calls = []
    for layer in range(layers):
        for name, out, inp, has_bias in QWEN_LAYER_CALLS:
            fmt = "q6_k" if (name == "down" and layer % 2 == 0) else "q4_k"
            if fmt == "q4_k" and layout == "stream" and inp % 256:
                fmt = "q4_k_stream"
            calls.append((layer, name, fmt, out, inp, has_bias))
    calls.append((layers, "lm_head", "q8_0", QWEN_VOCAB, QWEN_HIDDEN, False))
    return calls
