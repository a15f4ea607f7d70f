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
