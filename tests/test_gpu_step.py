"""The decode step exactly as the benchmark times it, against the oracle.

The benchmark's step is 24 layers of Q, K, V (with bias), O, gate, up
(Q4_K) and down (Q6_K on even layers, else Q4_K), then the 151936 x 896
Q8_0 LM head: 169 mat-vecs issued as 97 grouped launches (Q/K/V and
gate/up share one) over two weight copies, replayed from one captured HIP
graph per copy.  Every output of every call - every row of the LM head
included - is held to the mat-vec bound 1e-4 * sum|w x| + 1e-6 against the
float64 oracle on the same seeded inputs, for an eager step and for graph
replays of each copy, and for the ungrouped 169-launch plan.  The
per-call diff against an independent oracle is the conformance workflow
of "PESTI - Portable Execution Substrate for Transformer Inference"
("Development Workflow", "Conformance").
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import oracle
from gpu_util import announce, assert_within

pytestmark = pytest.mark.gpu

GEMV_REL = 1e-4


def _oracle_call(call, inputs):
    """(y64 [1][out], bound scale [1][out]) of one call (the oracle expands
    the LM head a chunk of rows at a time)."""
    _, _, fmt, out, inf, _ = call
    packed, x, b = inputs
    return oracle.gemv_packed(fmt, packed, out, inf, x, b)


@pytest.fixture(scope="module")
def step_setup():
    import torch
    import bench
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth

    announce("decode step: generating inputs and the oracle's outputs")
    calls = synth.decode_step_calls()
    host = bench.host_inputs(calls)
    with ThreadPoolExecutor(8) as ex:
        refs = list(ex.map(lambda i: _oracle_call(calls[i], host[i]), range(len(calls))))
    announce("decode step: oracle done, uploading two weight copies")
    lib = dmv.load()
    calls, weights, xs, ys, biases = bench.build_inputs(2, calls, host)
    torch.cuda.synchronize()
    return dict(lib=lib, calls=calls, host=host, refs=refs, weights=weights, xs=xs, ys=ys,
                biases=biases)


def _poison(ys):
    import torch
    for y in ys:
        y.fill_(float("nan"))
    torch.cuda.synchronize()


def _check_all(st, what, skip=()):
    calls, ys, refs = st["calls"], st["ys"], st["refs"]
    for i, (call, y, (y_ref, s_ref)) in enumerate(zip(calls, ys, refs)):
        if i in skip:
            continue
        layer, name, fmt, out, inf, _ = call
        got = y.cpu().numpy().reshape(1, out)
        assert_within(got, y_ref, s_ref, GEMV_REL, f"{what}: call {i} ({name}{layer}, {fmt} {out}x{inf})")


@pytest.mark.parametrize("grouping", ["stage", "none"])
def test_decode_step_matches_oracle(step_setup, grouping):
    """Eager steps on both weight copies, then graph replays of each copy
    (eager work and synchronizations in between): all 169 outputs."""
    import torch
    import bench
    st = step_setup
    launches = bench.plan_launches(st["calls"], grouping)
    assert len(launches) == (97 if grouping == "stage" else 169)
    step = bench.make_step(st["lib"], st["calls"], launches, st["weights"], st["xs"], st["ys"],
                           st["biases"])
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for copy in (0, 1):
            announce(f"decode step ({grouping}): eager, weight copy {copy}")
            _poison(st["ys"])
            step(copy, stream.cuda_stream)
            torch.cuda.synchronize()
            _check_all(st, f"eager copy {copy}")
        graphs = []
        for copy in (0, 1):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                step(copy, torch.cuda.current_stream().cuda_stream)
            graphs.append(g)
        torch.cuda.synchronize()
        for rep in range(2):
            for copy in (0, 1):
                announce(f"decode step ({grouping}): graph replay {rep}, weight copy {copy}")
                _poison(st["ys"])
                graphs[copy].replay()
                torch.cuda.synchronize()
                _check_all(st, f"graph replay {rep} copy {copy}")
    del graphs


def test_decode_step_fused_swiglu_matches_oracle(step_setup):
    """The step with each layer's gate/up launch fused into h = silu(gate) *
    up (written into the gate call's buffer) and the down projection reading
    h: h against the oracle's SwiGLU of the same x, the down projection
    against the oracle applied to the h the GPU produced, every other call
    against its own oracle output; one eager step and two graph replays."""
    import torch
    import bench
    st = step_setup
    calls = st["calls"]
    launches = bench.plan_launches(calls, "stage")
    step = bench.make_step(st["lib"], calls, launches, st["weights"], st["xs"], st["ys"], st["biases"],
                           ffn="swiglu")
    gate_of, down_of, ups = {}, {}, set()
    for i, (layer, name, *_rest) in enumerate(calls):
        if name == "gate":
            gate_of[layer] = i
        elif name == "down":
            down_of[layer] = i
        elif name == "up":
            ups.add(i)
    h_refs = {}
    for layer, gi in gate_of.items():
        _, _, fmt, out, inf, _ = calls[gi]
        h, (g, sg), (u, su) = oracle.swiglu_packed(fmt, st["host"][gi][0], st["host"][gi + 1][0], out, inf,
                                                   st["host"][gi][1])
        h_refs[layer] = (h, oracle.swiglu_tolerance(g, sg, u, su, h))

    def check(what):
        _check_all(st, what, skip=set(gate_of.values()) | set(down_of.values()) | ups)
        for layer, gi in gate_of.items():
            h_gpu = st["ys"][gi].cpu().numpy().reshape(1, -1)
            h_ref, tol = h_refs[layer]
            err = np.abs(h_gpu.astype(np.float64) - h_ref)
            assert np.all(err <= tol), f"{what}: SwiGLU of layer {layer}: max excess {(err - tol).max():.3g}"
            di = down_of[layer]
            _, _, fmt, out, inf, _ = calls[di]
            y_ref, s_ref = oracle.gemv_packed(fmt, st["host"][di][0], out, inf, h_gpu.astype(np.float32))
            got = st["ys"][di].cpu().numpy().reshape(1, out)
            assert_within(got, y_ref, s_ref, GEMV_REL, f"{what}: down{layer} on the GPU's h")

    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        announce("decode step (fused SwiGLU): eager, weight copy 0")
        _poison(st["ys"])
        step(0, stream.cuda_stream)
        torch.cuda.synchronize()
        check("fused SwiGLU eager")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(1, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for rep in range(2):
            announce(f"decode step (fused SwiGLU): graph replay {rep}, weight copy 1")
            _poison(st["ys"])
            g.replay()
            torch.cuda.synchronize()
            check(f"fused SwiGLU graph replay {rep}")
    del g


def test_decode_step_stream_layout_matches_oracle():
    """The step with the 896-column Q4_K matrices in the byte-minimal stream
    layout (504 bytes per row): eager, then two graph replays, all 169
    outputs against the oracle."""
    import torch
    import bench
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth
    announce("decode step (stream layout): inputs and the oracle's outputs")
    calls = synth.decode_step_calls(layout="stream")
    host = bench.host_inputs(calls)
    with ThreadPoolExecutor(8) as ex:
        refs = list(ex.map(lambda i: _oracle_call(calls[i], host[i]), range(len(calls))))
    lib = dmv.load()
    calls, weights, xs, ys, biases = bench.build_inputs(1, calls, host)
    st = dict(calls=calls, ys=ys, refs=refs)
    launches = bench.plan_launches(calls, "stage")
    step = bench.make_step(lib, calls, launches, weights, xs, ys, biases)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        announce("decode step (stream layout): eager")
        _poison(ys)
        step(0, stream.cuda_stream)
        torch.cuda.synchronize()
        _check_all(st, "stream layout eager")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for rep in range(2):
            announce(f"decode step (stream layout): graph replay {rep}")
            _poison(ys)
            g.replay()
            torch.cuda.synchronize()
            _check_all(st, f"stream layout graph replay {rep}")
    del g
