"""The allocation-free small-M GEMM (pesti_gemm_smallm_noalloc) against the
workspace call it mirrors (pesti_gemm_smallm_ws), through the C ABI: bit
for bit on two calls in a row, the second with a smaller input, and within
the oracle's bound."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import dequantize_mat_vec_amd as dmv
from dequantize_mat_vec_amd import synth
from gpu_util import announce, assert_within, guarded_y, guards_intact, run_gemm_ws, to_dev, torch_dev

pytestmark = pytest.mark.gpu

REL = {"f16": 2e-3}   # binary16 GEMM bound; the block formats take the mat-vec's 1e-4


def _inputs(fmt, m, k, n, seed):
    rng = np.random.default_rng([seed, m, k, n, len(fmt)])
    w = synth.f16_weights(rng, n, k) if fmt == "f16" else synth.quant_blocks(fmt, rng, n, k)
    return w, synth.f16_activations(rng, m, k), synth.bias(rng, n)


def _noalloc(fmt, w, m, n, k, x16, bias):
    torch, _ = torch_dev()
    w_d = to_dev(np.asarray(w).reshape(-1).view(np.uint8))
    x_d = to_dev(np.ascontiguousarray(x16).view(np.uint16))
    b_d = to_dev(bias.astype(np.float32))
    fbuf, y_d = guarded_y(m * n)
    dmv.pesti_gemm_smallm_noalloc(fmt, m, n, k, w_d, x_d, y_d, b_d)
    torch.cuda.synchronize()
    assert guards_intact(fbuf, m * n), "GEMM wrote outside Y"
    return y_d.cpu().numpy().reshape(m, n)


# (m, k, n) per call: the first uses 4 splits over 56 column tiles (the
# largest partial set of these cases), the second is smaller and ragged
CALLS = {"f16": [(16, 4864, 896), (16, 4160, 70)]}
QUANT_CALLS = [(16, 4864, 896), (5, 4160, 70)]


@pytest.mark.parametrize("fmt", ("f16", "q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k"))
def test_noalloc_equals_workspace_call_on_two_calls(fmt):
    for i, (m, k, n) in enumerate(CALLS.get(fmt, QUANT_CALLS)):
        announce(f"noalloc {fmt} call {i}: m{m} k{k} n{n}")
        need = dmv.pesti_gemm_workspace_bytes(fmt, m, n, k)
        assert 0 < need <= dmv.GEMM_SCRATCH_BYTES
        w, x, bias = _inputs(fmt, m, k, n, 41 + i)
        y = _noalloc(fmt, w, m, n, k, x, bias)
        y_ws = run_gemm_ws(fmt, w, m, n, k, x, bias)
        assert np.array_equal(y, y_ws), (fmt, i)
        y_ref, s_ref = (oracle.gemm_f16(x, w, bias) if fmt == "f16" else oracle.gemm_packed(fmt, w, n, k, x, bias))
        assert_within(y, y_ref, s_ref, REL.get(fmt, 1e-4), f"noalloc {fmt} m{m} k{k} n{n}")


def test_noalloc_shape_without_split_equals_plain_call():
    m, k, n = 64, 896, 4864
    w, x, bias = _inputs("q4_k", m, k, n, 43)
    assert dmv.pesti_gemm_workspace_bytes("q4_k", m, n, k) == 0
    assert np.array_equal(_noalloc("q4_k", w, m, n, k, x, bias), run_gemm_ws("q4_k", w, m, n, k, x, bias))


def test_noalloc_in_a_captured_graph():
    """The call it exists for: captured in a graph (no allocation inside the
    capture), replayed with new X written eagerly between replays; every
    replay equals the eager workspace call on the same X bit for bit."""
    torch, _ = torch_dev()
    fmt, m, k, n = "q6_k", 32, 4864, 896
    w, x, bias = _inputs(fmt, m, k, n, 44)
    w_d = to_dev(np.asarray(w).reshape(-1).view(np.uint8))
    x_d = to_dev(np.ascontiguousarray(x).view(np.uint16))
    b_d = to_dev(bias.astype(np.float32))
    y_d = torch.empty(m * n, dtype=torch.float32, device=x_d.device)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        dmv.pesti_gemm_smallm_noalloc(fmt, m, n, k, w_d, x_d, y_d, b_d)   # warm-up outside the capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            dmv.pesti_gemm_smallm_noalloc(fmt, m, n, k, w_d, x_d, y_d, b_d)
    for r in range(3):
        announce(f"noalloc graph replay {r}")
        xr = synth.f16_activations(np.random.default_rng([45, r]), m, k)
        x_d.copy_(to_dev(np.ascontiguousarray(xr).view(np.uint16)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        y = y_d.cpu().numpy().reshape(m, n).copy()
        assert np.array_equal(y, run_gemm_ws(fmt, w, m, n, k, xr, bias)), r
