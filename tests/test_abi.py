"""The C ABI library without a GPU: it loads, exports every symbol the header
declares, and its host-only logic (row sizes, status text, argument checks
that reject a call before any device work) behaves as documented."""
from __future__ import annotations

import ctypes
import re
from pathlib import Path

import pytest

import oracle
import dequantize_mat_vec_amd as dmv
from dequantize_mat_vec_amd import _lib, synth

HEADER = Path(__file__).resolve().parent.parent / "include" / "pesti.h"


def declared_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pesti_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(str(_lib.LIB_PATH))
    names = declared_functions()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib._SIGNATURES), "binding and header disagree"


def test_header_constants_match_binding():
    text = HEADER.read_text()
    for name in ("PESTI_OK", "PESTI_ERR_NULL", "PESTI_ERR_SHAPE", "PESTI_ERR_BATCH",
                 "PESTI_ERR_ALIGN", "PESTI_ERR_LAUNCH", "PESTI_ERR_DEVICE", "PESTI_ERR_WORKSPACE"):
        m = re.search(rf"#define {name} \(?(-?\d+)\)?", text)
        assert m and int(m.group(1)) == getattr(_lib, name), name
    for fmt, fid in list(_lib.FORMAT_IDS.items()) + list(_lib.GEMM_FORMAT_IDS.items()):
        m = re.search(rf"#define PESTI_FMT_{fmt.upper()} (\d+)", text)
        assert m and int(m.group(1)) == fid


def test_abi_version():
    assert dmv.pesti_abi_version() == 3


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k", "i8row", "i4row"])
@pytest.mark.parametrize("inf", [0, 32, 64, 96, 256, 288, 768, 896, 4864, 16384])
def test_row_bytes_agree_with_oracle_and_generator(fmt, inf):
    rb = dmv.pesti_row_bytes(fmt, inf)
    assert rb == oracle.row_bytes(fmt, inf) == synth.packed_row_bytes(fmt, inf)


def test_row_bytes_rejects_bad_input():
    assert dmv.pesti_row_bytes(0, 33) == -1
    assert dmv.pesti_row_bytes(0, -32) == -1
    assert dmv.pesti_row_bytes(9, 64) == -1


def test_strerror_covers_every_status():
    for st in range(-7, 1):
        assert dmv.strerror(st) and dmv.strerror(st) != "unknown status"
    assert dmv.strerror(-99) == "unknown status"


# Argument checks that fire before any device query: safe with or without a
# GPU because nothing is launched.
FAKE = 0x100000   # 16-byte aligned, never dereferenced (calls are rejected)


def _raw():
    return _lib.load()


@pytest.mark.parametrize("name", ["pesti_gemv_q8_0", "pesti_gemv_q2_k", "pesti_gemv_q3_k",
                                  "pesti_gemv_q4_k", "pesti_gemv_q5_k", "pesti_gemv_q6_k"])
def test_gemv_argument_checks(name):
    fn = getattr(_raw(), name)
    assert fn(-1, 64, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(8, -32, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(8, 64, FAKE, FAKE, FAKE, None, 9, None) == _lib.PESTI_ERR_BATCH
    assert fn(8, 64, FAKE, FAKE, FAKE, None, -1, None) == _lib.PESTI_ERR_BATCH
    assert fn(8, 48, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(8, 65536, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(8, 64, None, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(8, 64, FAKE, None, FAKE, None, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(8, 64, FAKE, FAKE, None, None, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(8, 64, FAKE + 4, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(8, 64, FAKE, FAKE + 8, FAKE, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(8, 64, FAKE, FAKE, FAKE + 4, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(8, 64, FAKE, FAKE, FAKE, FAKE + 2, 1, None) == _lib.PESTI_ERR_ALIGN
    # empty outputs succeed without touching anything (NULL pointers allowed)
    assert fn(0, 64, None, None, None, None, 1, None) == _lib.PESTI_OK
    assert fn(8, 64, None, None, None, None, 0, None) == _lib.PESTI_OK


def test_i8row_and_gemm_argument_checks():
    lib = _raw()
    assert lib.pesti_gemv_i8row(8, 64, FAKE, None, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_gemv_i8row(8, 64, FAKE, FAKE + 2, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_gemv_i4row(8, 64, FAKE, None, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_gemv_i4row(8, 64, FAKE, FAKE + 2, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_gemv_i4row(8, 48, FAKE, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_gemv_i4row(8, 64, FAKE + 8, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_gemv_i4row(0, 64, None, None, None, None, None, 1, None) == _lib.PESTI_OK
    assert lib.pesti_dequant_i4row(4, 64, FAKE, None, FAKE, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_dequant_i4row(4, 40, FAKE, FAKE, FAKE, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_gemm_f16_smallm(-1, 8, 64, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_BATCH
    assert lib.pesti_gemm_f16_smallm(5000, 8, 64, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_BATCH
    assert lib.pesti_gemm_f16_smallm(4, 8, 40, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_gemm_f16_smallm(4, 8, 64, None, FAKE, FAKE, None, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_gemm_f16_smallm(4, 8, 64, FAKE, FAKE, FAKE + 4, None, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_gemm_f16_smallm(0, 8, 64, None, None, None, None, None) == _lib.PESTI_OK


@pytest.mark.parametrize("name", ["pesti_gemm_q8_0_smallm", "pesti_gemm_q2_k_smallm",
                                  "pesti_gemm_q3_k_smallm", "pesti_gemm_q4_k_smallm",
                                  "pesti_gemm_q5_k_smallm", "pesti_gemm_q6_k_smallm"])
def test_gemm_quant_argument_checks(name):
    fn = getattr(_raw(), name)
    assert fn(-1, 8, 64, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_BATCH
    assert fn(5000, 8, 64, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_BATCH
    assert fn(4, -8, 64, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_SHAPE
    assert fn(4, 8, 40, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_SHAPE
    assert fn(4, 8, 32800, FAKE, FAKE, FAKE, None, None) == _lib.PESTI_ERR_SHAPE
    assert fn(4, 8, 64, None, FAKE, FAKE, None, None) == _lib.PESTI_ERR_NULL
    assert fn(4, 8, 64, FAKE, None, FAKE, None, None) == _lib.PESTI_ERR_NULL
    assert fn(4, 8, 64, FAKE, FAKE, None, None, None) == _lib.PESTI_ERR_NULL
    assert fn(4, 8, 64, FAKE, FAKE + 8, FAKE, None, None) == _lib.PESTI_ERR_ALIGN
    assert fn(4, 8, 64, FAKE + 2, FAKE, FAKE, None, None) == _lib.PESTI_ERR_ALIGN
    assert fn(4, 8, 64, FAKE, FAKE, FAKE, FAKE + 2, None) == _lib.PESTI_ERR_ALIGN
    assert fn(0, 8, 64, None, None, None, None, None) == _lib.PESTI_OK
    assert fn(4, 0, 64, None, None, None, None, None) == _lib.PESTI_OK


def test_swiglu_argument_checks():
    fn = _raw().pesti_gemv_swiglu
    Q4, Q8, I8 = _lib.FORMAT_IDS["q4_k"], _lib.FORMAT_IDS["q8_0"], _lib.FORMAT_IDS["i8row"]
    assert fn(9, 8, 64, FAKE, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(Q4, 8, 64, FAKE, FAKE, None, None, FAKE, FAKE, 9, None) == _lib.PESTI_ERR_BATCH
    assert fn(Q4, 8, 64, FAKE, FAKE, None, None, FAKE, FAKE, -1, None) == _lib.PESTI_ERR_BATCH
    assert fn(Q4, 8, 40, FAKE, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(Q4, 8, 4160, FAKE, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(Q8, 8, 2080, FAKE, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_SHAPE
    assert fn(Q4, 8, 64, None, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(Q4, 8, 64, FAKE, None, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(Q4, 8, 64, FAKE, FAKE, None, None, None, FAKE, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(Q4, 8, 64, FAKE, FAKE, None, None, FAKE, None, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(I8, 8, 64, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_NULL
    assert fn(Q4, 8, 64, FAKE + 8, FAKE, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(Q4, 8, 64, FAKE, FAKE + 8, None, None, FAKE, FAKE, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(Q4, 8, 64, FAKE, FAKE, None, None, FAKE, FAKE + 4, 1, None) == _lib.PESTI_ERR_ALIGN
    assert fn(Q4, 0, 64, None, None, None, None, None, None, 1, None) == _lib.PESTI_OK
    assert fn(Q4, 8, 64, None, None, None, None, None, None, 0, None) == _lib.PESTI_OK


@pytest.mark.parametrize("name", ["pesti_dequant_q8_0", "pesti_dequant_q2_k", "pesti_dequant_q3_k",
                                  "pesti_dequant_q4_k", "pesti_dequant_q5_k", "pesti_dequant_q6_k"])
def test_dequant_argument_checks(name):
    fn = getattr(_raw(), name)
    assert fn(-1, 64, FAKE, FAKE, None) == _lib.PESTI_ERR_SHAPE
    assert fn(4, 40, FAKE, FAKE, None) == _lib.PESTI_ERR_SHAPE
    assert fn(4, 64, None, FAKE, None) == _lib.PESTI_ERR_NULL
    assert fn(4, 64, FAKE, FAKE + 4, None) == _lib.PESTI_ERR_ALIGN
    assert fn(0, 64, None, None, None) == _lib.PESTI_OK


def test_binding_raises_on_error_status():
    with pytest.raises(_lib.PestiError) as e:
        dmv.pesti_gemv_q8_0(8, 48, FAKE, FAKE, FAKE, stream=0)
    assert e.value.status == _lib.PESTI_ERR_SHAPE


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        dmv.pesti_gemv_q8_0(1, 32, torch.zeros(34, dtype=torch.uint8), FAKE, FAKE, stream=0)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        _lib.load(tmp_path / "libpesti.so")


def test_group_argument_checks():
    lib = _raw()
    ops = _lib.gemv_ops([(8, 64, FAKE, FAKE, FAKE, None, None)] * 2)
    ptr = ctypes.cast(ops, ctypes.c_void_p)
    assert lib.pesti_gemv_group(0, 9, ptr, 1, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_gemv_group(9, 2, ptr, 1, None) == _lib.PESTI_ERR_SHAPE   # unknown format
    half_run = _lib.gemv_ops([(8, 96, FAKE, FAKE, FAKE, None, None)])       # 96 % 64 != 0
    assert lib.pesti_gemv_group(8, 1, ctypes.cast(half_run, ctypes.c_void_p), 1, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_gemv_group(7, 2, ptr, 1, None) == _lib.PESTI_ERR_NULL   # i4row without row scales
    assert lib.pesti_gemv_group(1, 2, None, 1, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_gemv_group(1, 2, ptr, 9, None) == _lib.PESTI_ERR_BATCH
    bad = _lib.gemv_ops([(8, 64, FAKE, FAKE, FAKE, None, None), (8, 48, FAKE, FAKE, FAKE, None, None)])
    assert lib.pesti_gemv_group(1, 2, ctypes.cast(bad, ctypes.c_void_p), 1, None) == _lib.PESTI_ERR_SHAPE
    bad = _lib.gemv_ops([(8, 64, FAKE, FAKE, FAKE + 4, None, None)])
    assert lib.pesti_gemv_group(2, 1, ctypes.cast(bad, ctypes.c_void_p), 1, None) == _lib.PESTI_ERR_ALIGN
    bad = _lib.gemv_ops([(8, 64, FAKE, FAKE, FAKE, None, None)])
    assert lib.pesti_gemv_group(3, 1, ctypes.cast(bad, ctypes.c_void_p), 1, None) == _lib.PESTI_ERR_NULL
    empty = _lib.gemv_ops([(0, 64, None, None, None, None, None)] * 3)
    assert lib.pesti_gemv_group(1, 3, ctypes.cast(empty, ctypes.c_void_p), 1, None) == _lib.PESTI_OK
    assert lib.pesti_gemv_group(1, 0, None, 1, None) == _lib.PESTI_OK
    assert lib.pesti_gemv_group(1, 2, ptr, 0, None) == _lib.PESTI_OK


def test_group_struct_layout_matches_header():
    text = HEADER.read_text()
    body = re.search(r"typedef struct pesti_gemv_op \{(.*?)\} pesti_gemv_op;", text, re.S).group(1)
    fields = re.findall(r"\b(\w+);", body)
    assert fields == [f[0] for f in _lib.GemvOp._fields_]
    assert ctypes.sizeof(_lib.GemvOp) == 56
    m = re.search(r"#define PESTI_MAX_GROUP (\d+)", text)
    assert int(m.group(1)) == _lib.MAX_GROUP


def test_one_hip_runtime_per_process():
    """Loading the library before anything else imports torch still leaves a
    single HIP runtime mapped (the library binds to PyTorch's copy)."""
    import subprocess
    import sys
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from dequantize_mat_vec_amd import _lib\n"
        "_lib.load()\n"
        "import torch\n"
        "paths = set()\n"
        "for line in open('/proc/self/maps'):\n"
        "    p = line.split()[-1]\n"
        "    if 'libamdhip64' in p: paths.add(p)\n"
        "print(len(paths), sorted(paths))\n" % str(HEADER.parent.parent))
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.split()[0] == "1", out.stdout


def test_stream_read_argument_checks():
    lib = _raw()
    part = FAKE + 0x1000
    assert lib.pesti_stream_read(FAKE, 20, part, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_stream_read(FAKE, -16, part, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_stream_read(FAKE, 64, None, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_stream_read(None, 64, part, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_stream_read(FAKE + 4, 64, part, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_stream_read(FAKE, 64, part + 2, None) == _lib.PESTI_ERR_ALIGN
    m = re.search(r"#define PESTI_READ_GROUPS (\d+)", HEADER.read_text())
    assert int(m.group(1)) == _lib.READ_GROUPS


def test_matrix_bytes():
    """Whole-matrix sizes: rows * row bytes for the row layouts; the stream
    layout holds rows * in weights in whole 144-byte super-blocks (896-weight
    rows: 504 bytes each, the last super-block padded)."""
    assert dmv.pesti_matrix_bytes("q4_k", 3, 896) == 3 * 576
    assert dmv.pesti_matrix_bytes("q4_k_stream", 2, 896) == 1008
    assert dmv.pesti_matrix_bytes("q4_k_stream", 3, 896) == 11 * 144
    assert dmv.pesti_matrix_bytes("q4_k_stream", 4864, 896) == 4864 * 504
    assert dmv.pesti_matrix_bytes("q4_k_stream", 5, 4864) == 5 * oracle_row_bytes_q4_k(4864)
    assert dmv.pesti_matrix_bytes("q4_k_stream", 3, 96) == -1
    assert dmv.pesti_row_bytes("q4_k_stream", 896) == -1
    assert dmv.pesti_matrix_bytes("i8row", 4, 64) == 256
    assert dmv.pesti_matrix_bytes(99, 4, 64) == -1


def oracle_row_bytes_q4_k(inf):
    return -(-inf // 256) * 144


def test_stream_dequant_argument_checks():
    lib = _raw()
    assert lib.pesti_dequant_q4_k_stream(2, 96, FAKE, FAKE, None) == _lib.PESTI_ERR_SHAPE
    assert lib.pesti_dequant_q4_k_stream(0, 896, FAKE, FAKE, None) == _lib.PESTI_OK
    assert lib.pesti_dequant_q4_k_stream(2, 896, None, FAKE, None) == _lib.PESTI_ERR_NULL
    assert lib.pesti_dequant_q4_k_stream(2, 896, FAKE + 4, FAKE, None) == _lib.PESTI_ERR_ALIGN
    assert lib.pesti_gemv_q4_k_stream(4, 96, FAKE, FAKE, FAKE, None, 1, None) == _lib.PESTI_ERR_SHAPE


def test_gemm_workspace_bytes_rule():
    """Host-only: the split-K workspace of the small-M GEMMs (splits * m * n
    float32 partials), by format and shape."""
    ws = dmv.pesti_gemm_workspace_bytes
    # Qwen down projection 896x4864: 56 column tiles, 4 splits at one row
    # tile of X, 2 at two, none at three
    for fmt in ("q8_0", "q2_k", "q4_k", "q5_k"):
        assert ws(fmt, 16, 896, 4864) == 4 * 16 * 896 * 4
        assert ws(fmt, 1, 896, 4864) == 4 * 1 * 896 * 4
        assert ws(fmt, 32, 896, 4864) == 2 * 32 * 896 * 4
        assert ws(fmt, 48, 896, 4864) == 0
    # Q3_K, Q6_K pair row tiles of X: workgroups = 56 * ceil(tiles / 2)
    for fmt in ("q3_k", "q6_k"):
        assert ws(fmt, 16, 896, 4864) == 4 * 16 * 896 * 4
        assert ws(fmt, 1, 896, 4864) == 4 * 1 * 896 * 4
        assert ws(fmt, 32, 896, 4864) == 4 * 32 * 896 * 4
        assert ws(fmt, 48, 896, 4864) == 2 * 48 * 896 * 4
        assert ws(fmt, 64, 896, 4864) == 2 * 64 * 896 * 4
        assert ws(fmt, 80, 896, 4864) == 0
    # binary16: only m = 16 row tiles (below 16 the vector-ALU path)
    assert ws("f16", 16, 896, 4864) == 4 * 16 * 896 * 4
    assert ws("f16", 32, 896, 4864) == 0
    assert ws("f16", 8, 896, 4864) == 0
    # rows of at most 128 k-steps, 96+ column tiles, empty shapes: no split
    assert ws("q6_k", 16, 896, 4096) == 0
    assert ws("q6_k", 16, 1536, 8192) == 0
    assert ws("q6_k", 16, 1520, 8192) == 2 * 16 * 1520 * 4
    assert ws("q6_k", 0, 896, 4864) == 0
    assert ws("q6_k", 16, 0, 4864) == 0
    # bad input
    assert ws("q6_k", 16, 896, 4865) == dmv.PESTI_ERR_SHAPE
    assert ws("q6_k", 4097, 896, 4864) == dmv.PESTI_ERR_BATCH
    assert ws(3, 16, 896, 4864) == dmv.PESTI_ERR_SHAPE   # i8row has no GEMM
    # the largest workspace any shape asks for is the allocation-free
    # variant's scratch (reached at 64 workgroups of paired 16x16 output
    # tiles with 4 splits)
    worst = max(ws(f, m, n, 8192) for f in ("f16", "q6_k") for m in range(1, 80, 3) for n in range(16, 1537, 16))
    assert worst == dmv.GEMM_SCRATCH_BYTES
    text = HEADER.read_text()
    assert re.search(r"#define PESTI_GEMM_SCRATCH_BYTES \(512 \* 1024\)", text)


def test_gemm_ws_argument_checks():
    """Rejected before any device work: unknown format, missing workspace."""
    lib = _lib.load()
    f = lib.pesti_gemm_smallm_ws
    assert f(3, 16, 896, 4864, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == dmv.PESTI_ERR_SHAPE
    assert f(16, 16, 896, 4864, FAKE, FAKE, FAKE, None, None, 0, None) == dmv.PESTI_ERR_WORKSPACE
    assert f(1, 16, 896, 4864, FAKE, FAKE, FAKE, None, FAKE, 4 * 16 * 896 * 4 - 16, None) == dmv.PESTI_ERR_WORKSPACE
    assert f(1, 16, 896, 4864, FAKE, FAKE, FAKE, None, FAKE + 4, 1 << 20, None) == dmv.PESTI_ERR_ALIGN
    assert f(1, 16, 896, 4865, FAKE, FAKE, FAKE, None, FAKE, 1 << 20, None) == dmv.PESTI_ERR_SHAPE
    g = lib.pesti_gemm_smallm_noalloc
    assert g(3, 16, 896, 4864, FAKE, FAKE, FAKE, None, None) == dmv.PESTI_ERR_SHAPE
    assert g(1, 4097, 896, 4864, FAKE, FAKE, FAKE, None, None) == dmv.PESTI_ERR_BATCH
    assert g(1, 16, 896, 4865, FAKE, FAKE, FAKE, None, None) == dmv.PESTI_ERR_SHAPE
