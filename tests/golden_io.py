"""Reader for the hand-worked fixtures under tests/golden/.

Grammar, one item per line ('#' starts a comment):
  format <q8_0|q2_k|...|q6_k|q4_k_stream|i8row|i4row>   rows <n>   in_features <n>
  hex <tokens>      packed bytes; a token is two hex digits, or XX*N for N copies
  codes <values>    i8row int8 codes of one row (values as below)
  scales <values>   i8row / i4row float32 scales (i4row codes travel as hex)
  f64 <values>      exact dequantized weights, row-major
  f32 <values>      float32 weights when they differ from rounding f64
  x / bias / y      a mat-vec case: input, bias and exact output
Keys other than format, rows and in_features may repeat; their values are
concatenated in order.  A value is a decimal or hex float literal, or NxV for N copies of V."""
from __future__ import annotations

from pathlib import Path

import numpy as np

GOLDEN_DIR = Path(__file__).resolve().parent / "golden"


def _value(tok: str) -> float:
    t = tok.strip()
    neg = t.startswith("-")
    body = t[1:] if neg else t
    v = float.fromhex(body) if body.lower().startswith("0x") else float(body)
    return -v if neg else v


def _values(tokens):
    out = []
    for tok in tokens:
        if "x" in tok and not tok.lower().lstrip("-").startswith("0x"):
            n, v = tok.split("x", 1)
            out.extend([_value(v)] * int(n))
        else:
            out.append(_value(tok))
    return out


def _hex(tokens):
    out = bytearray()
    for tok in tokens:
        if "*" in tok:
            b, n = tok.split("*")
            out.extend(bytes([int(b, 16)]) * int(n))
        else:
            out.append(int(tok, 16))
    return bytes(out)


def load(name: str) -> dict:
    fx = {"hex": b"", "codes": [], "name": name}
    for line in (GOLDEN_DIR / name).read_text().splitlines():
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *rest = line.split()
        if key == "format":
            fx["format"] = rest[0]
        elif key in ("rows", "in_features"):
            fx[key] = int(rest[0])
        elif key == "hex":
            fx["hex"] += _hex(rest)
        elif key == "codes":
            fx["codes"].append([int(v) for v in _values(rest)])
        elif key in ("scales", "f64", "f32", "x", "bias", "y"):
            # a key may span several lines: the values are concatenated
            vals = np.array(_values(rest), dtype=np.float64)
            fx[key] = np.concatenate([fx[key], vals]) if key in fx else vals
        else:
            raise ValueError(f"{name}: unknown key {key!r}")
    return fx


def packed(fx: dict):
    """(packed uint8 bytes, float32 scales or None) of a fixture."""
    if fx["format"] == "i8row":
        codes = np.array(fx["codes"], dtype=np.int64).astype(np.int8)
        return codes.view(np.uint8).reshape(-1), fx["scales"].astype(np.float32)
    data = np.frombuffer(fx["hex"], dtype=np.uint8).copy()
    if fx["format"] == "i4row":
        return data, fx["scales"].astype(np.float32)
    return data, None


def all_fixtures():
    return sorted(p.name for p in GOLDEN_DIR.glob("*.txt"))
