"""Helpers of the GPU parity tests: move seeded inputs to the device, call the
C ABI through the binding, and compare with the oracle."""
from __future__ import annotations

import sys

import numpy as np

GUARD = 64                      # canary floats on each side of y
CANARY_BITS = 0x7FC0DEAD        # a NaN payload no kernel writes


def announce(msg: str) -> None:
    """Name the case before a GPU step, so a crash still says which one."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    return torch, torch.device("cuda:0")


def to_dev(arr):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def guarded_y(n: int):
    """(buffer, view) where view is the n-float output between canaries."""
    torch, dev = torch_dev()
    buf = torch.full((GUARD + max(n, 0) + GUARD,), CANARY_BITS, dtype=torch.int32, device=dev)
    fbuf = buf.view(torch.float32)
    return fbuf, fbuf[GUARD:GUARD + n]


def guards_intact(fbuf, n: int) -> bool:
    torch, _ = torch_dev()
    bits = fbuf.view(torch.int32).cpu().numpy().view(np.uint32)
    return bool(np.all(bits[:GUARD] == CANARY_BITS) and np.all(bits[GUARD + n:] == CANARY_BITS))


def run_gemv(fmt, packed, scales, out, inf, x, bias=None, stream=None):
    """y (float32 numpy [batch, out]) from the HIP path, guards checked."""
    import dequantize_mat_vec_amd as dmv
    torch, _ = torch_dev()
    x = np.atleast_2d(x).astype(np.float32)
    batch = x.shape[0]
    w_d = to_dev(np.asarray(packed).reshape(-1).view(np.uint8))
    s_d = to_dev(scales.astype(np.float32)) if scales is not None else None
    x_d = to_dev(x)
    b_d = to_dev(bias.astype(np.float32)) if bias is not None else None
    fbuf, y_d = guarded_y(batch * out)
    dmv.gemv(fmt, out, inf, w_d, x_d, y_d, b_d, batch, scales=s_d, stream=stream)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, batch * out), "kernel wrote outside y"
    return y_d.cpu().numpy().reshape(batch, out)


def run_dequant(fmt, packed, scales, rows, inf):
    import dequantize_mat_vec_amd as dmv
    torch, dev = torch_dev()
    w_d = to_dev(np.asarray(packed).reshape(-1).view(np.uint8))
    s_d = to_dev(scales.astype(np.float32)) if scales is not None else None
    fbuf, out = guarded_y(rows * inf)
    dmv.dequant(fmt, rows, inf, w_d, out, scales=s_d)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, rows * inf), "dequant wrote outside its output"
    return out.cpu().numpy().reshape(rows, inf)


def run_gemm(x16, w16, bias=None):
    import dequantize_mat_vec_amd as dmv
    torch, _ = torch_dev()
    m, k = x16.shape
    n = w16.shape[0]
    x_d = to_dev(x16.view(np.uint16))
    w_d = to_dev(w16.view(np.uint16))
    b_d = to_dev(bias.astype(np.float32)) if bias is not None else None
    fbuf, y_d = guarded_y(m * n)
    dmv.pesti_gemm_f16_smallm(m, n, k, w_d, x_d, y_d, b_d)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, m * n), "GEMM wrote outside Y"
    return y_d.cpu().numpy().reshape(m, n)


def assert_within(y, y_ref, s_ref, rel, what=""):
    err = np.abs(y.astype(np.float64) - y_ref)
    bound = rel * s_ref + 1e-6
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        detail = ", ".join(f"{tuple(i)}: got {y[tuple(i)]!r} want {y_ref[tuple(i)]!r} "
                           f"err {err[tuple(i)]:.3g} bound {bound[tuple(i)]:.3g}" for i in idx)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; {detail}")
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"


def run_gemm_quant(fmt, packed, m, n, k, x16, bias=None):
    import dequantize_mat_vec_amd as dmv
    torch, _ = torch_dev()
    w_d = to_dev(np.asarray(packed).reshape(-1).view(np.uint8))
    x_d = to_dev(np.ascontiguousarray(x16).view(np.uint16))
    b_d = to_dev(bias.astype(np.float32)) if bias is not None else None
    fbuf, y_d = guarded_y(m * n)
    dmv.gemm_quant(fmt, m, n, k, w_d, x_d, y_d, b_d)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, m * n), "quantized GEMM wrote outside Y"
    return y_d.cpu().numpy().reshape(m, n)


def run_gemm_ws(fmt, w, m, n, k, x16, bias=None, workspace_bytes=None):
    """Y from pesti_gemm_smallm_ws (w: binary16 [n][k] for "f16", else packed
    rows) with a workspace of pesti_gemm_workspace_bytes(...) bytes (or
    `workspace_bytes`) between canaries; Y and workspace guards checked."""
    import dequantize_mat_vec_amd as dmv
    torch, _ = torch_dev()
    w_d = to_dev(np.asarray(w).reshape(-1).view(np.uint8))
    x_d = to_dev(np.ascontiguousarray(x16).view(np.uint16))
    b_d = to_dev(bias.astype(np.float32)) if bias is not None else None
    need = dmv.pesti_gemm_workspace_bytes(fmt, m, n, k)
    assert need >= 0 and need % 4 == 0
    nbytes = need if workspace_bytes is None else workspace_bytes
    wbuf, ws = guarded_y(nbytes // 4)
    fbuf, y_d = guarded_y(m * n)
    dmv.pesti_gemm_smallm_ws(fmt, m, n, k, w_d, x_d, y_d, b_d, ws if nbytes else None, nbytes)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, m * n), "GEMM wrote outside Y"
    assert guards_intact(wbuf, nbytes // 4), "GEMM wrote outside its workspace"
    return y_d.cpu().numpy().reshape(m, n)


def run_swiglu(fmt, w_gate, w_up, gate_scales, up_scales, out, inf, x):
    import dequantize_mat_vec_amd as dmv
    torch, _ = torch_dev()
    batch = x.shape[0]
    g_d = to_dev(np.asarray(w_gate).reshape(-1).view(np.uint8))
    u_d = to_dev(np.asarray(w_up).reshape(-1).view(np.uint8))
    gs = to_dev(gate_scales.astype(np.float32)) if gate_scales is not None else None
    us = to_dev(up_scales.astype(np.float32)) if up_scales is not None else None
    x_d = to_dev(np.ascontiguousarray(x, dtype=np.float32))
    fbuf, h_d = guarded_y(batch * out)
    dmv.pesti_gemv_swiglu(fmt, out, inf, g_d, u_d, x_d, h_d, batch, gs, us)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, batch * out), "SwiGLU wrote outside h"
    return h_d.cpu().numpy().reshape(batch, out)
