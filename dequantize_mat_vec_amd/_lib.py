"""ctypes binding of libpesti.so (the C ABI declared in include/pesti.h).

Argument marshalling only: every function here has the C entry point's name
and arguments, accepts torch tensors (device memory) or raw integer device
pointers, fills in the current torch stream when none is given, calls the
library and raises PestiError on a non-zero status.  All arithmetic happens
in the HIP kernels; there is no fallback of any kind - if the shared library
is missing, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os
from pathlib import Path

LIB_PATH = Path(__file__).resolve().with_name("libpesti.so")

PESTI_OK = 0
PESTI_ERR_NULL = -1
PESTI_ERR_SHAPE = -2
PESTI_ERR_BATCH = -3
PESTI_ERR_ALIGN = -4
PESTI_ERR_LAUNCH = -5
PESTI_ERR_DEVICE = -6
PESTI_ERR_WORKSPACE = -7

GEMM_SCRATCH_BYTES = 512 * 1024   # PESTI_GEMM_SCRATCH_BYTES

FORMAT_IDS = {"q8_0": 0, "q4_k": 1, "q6_k": 2, "i8row": 3, "q5_k": 4, "q2_k": 5, "q3_k": 6, "i4row": 7,
              "q4_k_stream": 8}
# formats of the small-M GEMM calls that take a format id
GEMM_FORMAT_IDS = {"f16": 16, "q8_0": 0, "q2_k": 5, "q3_k": 6, "q4_k": 1, "q5_k": 4, "q6_k": 2}

_i64, _i32, _vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p
_c_int, _c_char_p = ctypes.c_int, ctypes.c_char_p

_SIGNATURES = {
    "pesti_gemv_q8_0": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q4_k": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q4_k_stream": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q2_k": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q3_k": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q5_k": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_q6_k": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_i8row": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_i4row": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemv_group": (_c_int, [_i32, _i32, _vp, _i32, _vp]),
    "pesti_gemv_swiglu": (_c_int, [_i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp]),
    "pesti_gemm_f16_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q8_0_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q4_k_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q6_k_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q2_k_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q3_k_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_q5_k_smallm": (_c_int, [_i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_gemm_workspace_bytes": (_i64, [_i32, _i64, _i64, _i64]),
    "pesti_gemm_smallm_ws": (_c_int, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _i64, _vp]),
    "pesti_gemm_smallm_noalloc": (_c_int, [_i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp]),
    "pesti_dequant_q8_0": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q4_k": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q4_k_stream": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q2_k": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q3_k": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q5_k": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_q6_k": (_c_int, [_i64, _i64, _vp, _vp, _vp]),
    "pesti_dequant_i8row": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp]),
    "pesti_dequant_i4row": (_c_int, [_i64, _i64, _vp, _vp, _vp, _vp]),
    "pesti_stream_read": (_c_int, [_vp, _i64, _vp, _vp]),
    "pesti_row_bytes": (_i64, [_i32, _i64]),
    "pesti_matrix_bytes": (_i64, [_i32, _i64, _i64]),
    "pesti_strerror": (_c_char_p, [_c_int]),
    "pesti_abi_version": (_i32, []),
}

_lib = None

MAX_GROUP = 8


class GemvOp(ctypes.Structure):
    """pesti_gemv_op: one mat-vec of a grouped launch."""
    _fields_ = [("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64),
                ("w", ctypes.c_void_p), ("row_scales", ctypes.c_void_p),
                ("x", ctypes.c_void_p), ("y", ctypes.c_void_p), ("bias", ctypes.c_void_p)]


class PestiError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status} ({strerror(status)})")


def load(path: os.PathLike | None = None) -> ctypes.CDLL:
    """Load libpesti.so once; raise if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = Path(path) if path is not None else LIB_PATH
    if not p.exists():
        raise ImportError(f"{p} is missing: build the HIP library first "
                          "(python -m dequantize_mat_vec_amd.build)")
    # PyTorch's HIP runtime goes in first.  The library asks for the
    # runtime by its soname (libamdhip64.so.7), which then resolves to the
    # copy PyTorch already loaded; loaded the other way round, PyTorch
    # would bring in a second runtime, and pointers and streams would not
    # cross between the two.
    import torch  # noqa: F401
    lib = ctypes.CDLL(str(p))
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path is None:
        _lib = lib
    return lib


def _ptr(obj):
    """Device pointer of a torch tensor, an int, or None (NULL)."""
    if obj is None:
        return None
    if isinstance(obj, int):
        return obj
    if hasattr(obj, "data_ptr"):
        if not obj.is_cuda:
            raise ValueError("tensor arguments must live in device memory")
        if not obj.is_contiguous():
            raise ValueError("tensor arguments must be contiguous")
        return obj.data_ptr()
    raise TypeError(f"cannot pass {type(obj).__name__} as a device pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(name: str, status: int) -> int:
    if status != PESTI_OK:
        raise PestiError(name, status)
    return status


def strerror(status: int) -> str:
    return load().pesti_strerror(status).decode()


def pesti_abi_version() -> int:
    return load().pesti_abi_version()


def pesti_row_bytes(fmt, in_features: int) -> int:
    fid = FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)
    return load().pesti_row_bytes(fid, in_features)


def pesti_matrix_bytes(fmt, rows: int, in_features: int) -> int:
    fid = FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)
    return load().pesti_matrix_bytes(fid, rows, in_features)


def _gemv(name, out_features, in_features, blocks, x, y, bias, batch, stream):
    fn = getattr(load(), name)
    return _check(name, fn(out_features, in_features, _ptr(blocks), _ptr(x), _ptr(y),
                           _ptr(bias), batch, _stream(stream)))


def pesti_gemv_q8_0(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q8_0", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q4_k(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q4_k", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q4_k_stream(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q4_k_stream", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q2_k(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q2_k", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q3_k(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q3_k", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q5_k(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q5_k", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_q6_k(out_features, in_features, blocks, x, y, bias=None, batch=1, stream=None):
    return _gemv("pesti_gemv_q6_k", out_features, in_features, blocks, x, y, bias, batch, stream)


def pesti_gemv_i8row(out_features, in_features, codes, row_scales, x, y, bias=None, batch=1,
                     stream=None):
    return _check("pesti_gemv_i8row", load().pesti_gemv_i8row(
        out_features, in_features, _ptr(codes), _ptr(row_scales), _ptr(x), _ptr(y), _ptr(bias),
        batch, _stream(stream)))


def pesti_gemv_i4row(out_features, in_features, packed, row_scales, x, y, bias=None, batch=1,
                     stream=None):
    return _check("pesti_gemv_i4row", load().pesti_gemv_i4row(
        out_features, in_features, _ptr(packed), _ptr(row_scales), _ptr(x), _ptr(y), _ptr(bias),
        batch, _stream(stream)))


def pesti_gemv_swiglu(fmt, out_features, in_features, w_gate, w_up, x, h, batch=1,
                      gate_scales=None, up_scales=None, stream=None):
    """h = silu(W_gate x) * (W_up x) in one launch (row scales for i8row and i4row only)."""
    fid = FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)
    return _check("pesti_gemv_swiglu", load().pesti_gemv_swiglu(
        fid, out_features, in_features, _ptr(w_gate), _ptr(w_up), _ptr(gate_scales), _ptr(up_scales),
        _ptr(x), _ptr(h), batch, _stream(stream)))


def pesti_gemm_f16_smallm(m, out_features, in_features, w, x, y, bias=None, stream=None):
    return _check("pesti_gemm_f16_smallm", load().pesti_gemm_f16_smallm(
        m, out_features, in_features, _ptr(w), _ptr(x), _ptr(y), _ptr(bias), _stream(stream)))


def _gemm_q(name, m, out_features, in_features, blocks, x, y, bias, stream):
    return _check(name, getattr(load(), name)(m, out_features, in_features, _ptr(blocks), _ptr(x),
                                              _ptr(y), _ptr(bias), _stream(stream)))


def pesti_gemm_q8_0_smallm(m, out_features, in_features, blocks, x, y, bias=None, stream=None):
    return _gemm_q("pesti_gemm_q8_0_smallm", m, out_features, in_features, blocks, x, y, bias,
                   stream)


def pesti_gemm_q4_k_smallm(m, out_features, in_features, blocks, x, y, bias=None, stream=None):
    return _gemm_q("pesti_gemm_q4_k_smallm", m, out_features, in_features, blocks, x, y, bias,
                   stream)


def pesti_gemm_q6_k_smallm(m, out_features, in_features, blocks, x, y, bias=None, stream=None):
    return _gemm_q("pesti_gemm_q6_k_smallm", m, out_features, in_features, blocks, x, y, bias,
                   stream)


def _gemm_fid(fmt):
    return GEMM_FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)


def pesti_gemm_workspace_bytes(fmt, m, out_features, in_features):
    """Workspace bytes the split-K form needs (0: none); negative status on bad input."""
    return int(load().pesti_gemm_workspace_bytes(_gemm_fid(fmt), m, out_features, in_features))


def pesti_gemm_smallm_ws(fmt, m, out_features, in_features, w, x, y, bias=None, workspace=None,
                         workspace_bytes=None, stream=None):
    """Small-M GEMM of format `fmt` ("f16" or a block format) with a caller's
    workspace (a device tensor, or a pointer with workspace_bytes)."""
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    return _check("pesti_gemm_smallm_ws", load().pesti_gemm_smallm_ws(
        _gemm_fid(fmt), m, out_features, in_features, _ptr(w), _ptr(x), _ptr(y), _ptr(bias),
        _ptr(workspace), workspace_bytes, _stream(stream)))


def pesti_gemm_smallm_noalloc(fmt, m, out_features, in_features, w, x, y, bias=None, stream=None):
    """pesti_gemm_smallm_ws with the library's own scratch (allocates nothing;
    calls that overlap on one GPU race)."""
    return _check("pesti_gemm_smallm_noalloc", load().pesti_gemm_smallm_noalloc(
        _gemm_fid(fmt), m, out_features, in_features, _ptr(w), _ptr(x), _ptr(y), _ptr(bias), _stream(stream)))


def gemv_ops(ops):
    """ctypes array of pesti_gemv_op from (out, in, w, x, y, bias, row_scales)
    tuples whose pointer fields are tensors, ints or None."""
    arr = (GemvOp * max(len(ops), 1))()
    for i, (out, inf, w, x, y, bias, scales) in enumerate(ops):
        arr[i] = GemvOp(out, inf, _ptr(w), _ptr(scales), _ptr(x), _ptr(y), _ptr(bias))
    return arr


def pesti_gemv_group(fmt, ops, batch=1, stream=None):
    """Grouped launch.  `ops` is a list of (out, in, w, x, y, bias, row_scales)
    tuples, or a ctypes array built by gemv_ops()."""
    fid = FORMAT_IDS[fmt] if isinstance(fmt, str) else int(fmt)
    if isinstance(ops, ctypes.Array):
        arr, n = ops, len(ops)
    else:
        arr, n = gemv_ops(ops), len(ops)
    return _check("pesti_gemv_group", load().pesti_gemv_group(
        fid, n, ctypes.cast(arr, ctypes.c_void_p), batch, _stream(stream)))


READ_GROUPS = 4096


def pesti_stream_read(buf, nbytes, partial, stream=None):
    """Streaming read of `nbytes` bytes of `buf` (measurement hook); each of
    READ_GROUPS workgroups writes the XOR of what it read to `partial`."""
    return _check("pesti_stream_read", load().pesti_stream_read(_ptr(buf), nbytes, _ptr(partial),
                                                                _stream(stream)))


def _dequant(name, rows, in_features, blocks, w_out, stream):
    return _check(name, getattr(load(), name)(rows, in_features, _ptr(blocks), _ptr(w_out),
                                              _stream(stream)))


def pesti_dequant_q8_0(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q8_0", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q4_k(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q4_k", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q4_k_stream(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q4_k_stream", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q2_k(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q2_k", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q3_k(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q3_k", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q5_k(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q5_k", rows, in_features, blocks, w_out, stream)


def pesti_dequant_q6_k(rows, in_features, blocks, w_out, stream=None):
    return _dequant("pesti_dequant_q6_k", rows, in_features, blocks, w_out, stream)


def pesti_dequant_i8row(rows, in_features, codes, row_scales, w_out, stream=None):
    return _check("pesti_dequant_i8row", load().pesti_dequant_i8row(
        rows, in_features, _ptr(codes), _ptr(row_scales), _ptr(w_out), _stream(stream)))


def pesti_dequant_i4row(rows, in_features, packed, row_scales, w_out, stream=None):
    return _check("pesti_dequant_i4row", load().pesti_dequant_i4row(
        rows, in_features, _ptr(packed), _ptr(row_scales), _ptr(w_out), _stream(stream)))


# --- format-generic conveniences (still marshalling only) -------------------
def gemv(fmt, out_features, in_features, w, x, y, bias=None, batch=1, scales=None, stream=None):
    """Dispatch y = W x + b to the entry point of format `fmt`."""
    if fmt == "i8row":
        return pesti_gemv_i8row(out_features, in_features, w, scales, x, y, bias, batch, stream)
    if fmt == "i4row":
        return pesti_gemv_i4row(out_features, in_features, w, scales, x, y, bias, batch, stream)
    return _gemv(f"pesti_gemv_{fmt}", out_features, in_features, w, x, y, bias, batch, stream)


def gemm_quant(fmt, m, out_features, in_features, blocks, x, y, bias=None, stream=None):
    """Dispatch Y = X W^T + b (binary16 X, packed W) to the entry point of
    format `fmt` (q8_0 or a K-family format)."""
    return _gemm_q(f"pesti_gemm_{fmt}_smallm", m, out_features, in_features, blocks, x, y, bias,
                   stream)


def dequant(fmt, rows, in_features, w, w_out, scales=None, stream=None):
    if fmt == "i8row":
        return pesti_dequant_i8row(rows, in_features, w, scales, w_out, stream)
    if fmt == "i4row":
        return pesti_dequant_i4row(rows, in_features, w, scales, w_out, stream)
    return _dequant(f"pesti_dequant_{fmt}", rows, in_features, w, w_out, stream)
