"""The decode-step launches captured in a HIP graph give the eager results on
every replay (with eager work and synchronizations between replays)."""
from __future__ import annotations

import numpy as np
import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu


def test_graph_replays_match_eager():
    import torch
    import bench
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth

    announce("test_graph_replays_match_eager")
    lib = dmv.load()
    calls = [c for c in synth.decode_step_calls(layers=3) if c[1] != "lm_head"]
    dev = torch.device("cuda:0")
    weights, xs, ys, biases = [[]], [], [], []
    for layer, name, fmt, out, inf, has_bias in calls:
        rng = synth.rng_for(50, layer, synth.TENSOR_INDEX[name])
        weights[0].append(torch.from_numpy(synth.quant_blocks(fmt, rng, out, inf).reshape(-1)).to(dev))
        xs.append(torch.from_numpy(synth.activations(rng, 1, inf)).to(dev))
        ys.append(torch.zeros(out, dtype=torch.float32, device=dev))
        biases.append(torch.from_numpy(synth.bias(rng, out)).to(dev) if has_bias else None)
    launches = bench.plan_launches(calls, "stage")
    step = bench.make_step(lib, calls, launches, weights, xs, ys, biases)
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step(0, stream.cuda_stream)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        for rep in range(4):
            for y in ys:
                y.fill_(float("nan"))          # eager work between replays
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            for y, e in zip(ys, eager):
                assert torch.equal(y, e), f"replay {rep} differs"
            # an eager step in between must not disturb the next replay
            step(0, stream.cuda_stream)
            torch.cuda.synchronize()


def test_graph_replays_match_eager_with_fused_swiglu():
    """The decode-step variant whose gate/up launch is the fused SwiGLU and
    whose down projection reads its output."""
    import torch
    import bench
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth

    announce("test_graph_replays_match_eager_with_fused_swiglu")
    lib = dmv.load()
    calls = [c for c in synth.decode_step_calls(layers=2) if c[1] != "lm_head"]
    dev = torch.device("cuda:0")
    weights, xs, ys, biases = [[]], [], [], []
    for layer, name, fmt, out, inf, has_bias in calls:
        rng = synth.rng_for(51, layer, synth.TENSOR_INDEX[name])
        weights[0].append(torch.from_numpy(synth.quant_blocks(fmt, rng, out, inf).reshape(-1)).to(dev))
        xs.append(torch.from_numpy(synth.activations(rng, 1, inf)).to(dev))
        ys.append(torch.zeros(out, dtype=torch.float32, device=dev))
        biases.append(torch.from_numpy(synth.bias(rng, out)).to(dev) if has_bias else None)
    launches = bench.plan_launches(calls, "stage")
    step = bench.make_step(lib, calls, launches, weights, xs, ys, biases, ffn="swiglu")
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        step(0, stream.cuda_stream)
        torch.cuda.synchronize()
        eager = [y.clone() for y in ys]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            step(0, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(ys, eager)):
            if calls[i][1] == "up":   # the fused launch writes h into the gate buffer only
                continue
            assert torch.equal(y, e), f"replay {rep}: launch output {i} differs from eager"


@pytest.mark.parametrize("fmt", ["q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k"])
def test_graph_replays_match_eager_gemm(fmt):
    """The quantized and binary16 GEMMs (K-split and wide-layer kernels, and
    the bias-only path) captured in one graph."""
    import torch
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth

    announce(f"test_graph_replays_match_eager_gemm[{fmt}]")
    dev = torch.device("cuda:0")
    rng = np.random.default_rng([52, len(fmt)])
    shapes = [(16, 896, 896), (64, 896, 16400), (20, 0, 40), (33, 4864, 896)]   # (m, k, n)
    args = []
    for m, k, n in shapes:
        w = synth.quant_blocks(fmt, rng, n, k) if k else np.zeros((n, 0), np.uint8)
        x = synth.f16_activations(rng, m, k) if k else np.zeros((m, 0), np.float16)
        args.append((m, k, n, torch.from_numpy(np.ascontiguousarray(w).reshape(-1)).to(dev),
                     torch.from_numpy(np.ascontiguousarray(x).view(np.uint16)).to(dev),
                     torch.zeros(m * n, dtype=torch.float32, device=dev),
                     torch.from_numpy(synth.bias(rng, n)).to(dev)))
    wh = torch.from_numpy(synth.f16_weights(rng, 2304, 768).view(np.uint16)).to(dev)
    xh = torch.from_numpy(synth.f16_activations(rng, 32, 768).view(np.uint16)).to(dev)
    yh = torch.zeros(32 * 2304, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()

    def run(sh):
        for m, k, n, w, x, y, b in args:
            dmv.gemm_quant(fmt, m, n, k, w if k else None, x if k else None, y, b, stream=sh)
        dmv.pesti_gemm_f16_smallm(32, 2304, 768, wh, xh, yh, None, stream=sh)

    with torch.cuda.stream(stream):
        run(stream.cuda_stream)
        torch.cuda.synchronize()
        eager = [a[5].clone() for a in args] + [yh.clone()]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            run(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
    outs = [a[5] for a in args] + [yh]
    for rep in range(3):
        for y in outs:
            y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (y, e) in enumerate(zip(outs, eager)):
            assert torch.equal(y, e), f"replay {rep}: output {i} differs from eager"
