#!/usr/bin/env python3
"""Benchmark: one Qwen2.5-0.5B-shaped decode step of quantized mat-vecs.

A step is the decode step's linear work at batch 1, in stream order: for each
of 24 layers Q, K, V (with bias), O, gate, up (Q4_K) and down (Q4_K, Q6_K on
even layers), then the tied 151936 x 896 Q8_0 LM head - 169 mat-vecs.  The
mat-vecs of one dependency stage (Q/K/V; gate/up) share one grouped launch
of the C ABI, so a step is 97 dependent launches (--grouping none: 169).  Weights are seeded random bytes of those shapes (the pages' model file
is not available), resident in HBM; two copies of the step's weights are
alternated so that the 256 MB last-level cache cannot hold a step's bytes.

Prints one JSON line: HBM GB/s over the step (nominal algorithmic bytes per
step / time per step), microseconds per step, the roofline of the dominant
kernel (the kernel with the most time per step, timed by replaying a graph
of only its launches between HIP events on the launch stream) and the CPU
oracle's rate on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)

HBM_PEAK_GBS = 8000.0
METRIC = "batch-1 dequant-GEMV HBM GB/s (% of peak), µs per Qwen2.5-0.5B decode step"
CONFIG_INDEX = 2          # the decode-step workload
NOMINAL_BYTES_PER_WEIGHT = {"q8_0": 34 / 32, "q2_k": 84 / 256, "q3_k": 110 / 256, "q4_k": 144 / 256,
                            "q4_k_stream": 144 / 256,
                            "q5_k": 176 / 256, "q6_k": 210 / 256, "i8row": 1.0,
                            "i4row": 0.5}


def call_bytes(fmt, out, inf, batch, has_bias):
    """Nominal algorithmic bytes of one mat-vec: packed weights at the
    format's bits per weight (no row padding), x, y and bias."""
    w = out * inf * NOMINAL_BYTES_PER_WEIGHT[fmt] + (4 * out if fmt in ("i8row", "i4row") else 0)
    return int(w + 4 * batch * (inf + out) + (4 * out if has_bias else 0))


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--mode", choices=("graph", "plain"), default="graph",
                   help="launch the step as a captured HIP graph or as plain launches")
    p.add_argument("--copies", type=int, default=2, help="weight copies alternated per step")
    p.add_argument("--grouping", choices=("stage", "none"), default="stage",
                   help="one launch per dependency stage (Q/K/V, O, gate/up, down) or per call")
    p.add_argument("--layout", choices=("rows", "stream"), default="stream",
                   help="Q4_K matrices of 896-weight rows in the row layout (whole super-blocks per "
                        "row, 576 bytes) or the byte-minimal stream layout (504 bytes per row)")
    p.add_argument("--ffn", choices=("separate", "swiglu"), default="separate",
                   help="gate and up as two mat-vecs (the 169-call step) or one fused launch "
                        "writing silu(gate) * up, which the down projection then reads")
    p.add_argument("--kernel-steps", type=int, default=20,
                   help="replays of each per-kernel graph (per-kernel times)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    p.add_argument("--cpu-leg", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--parity-leg", metavar="NPZ", help=argparse.SUPPRESS)
    p.add_argument("--suite-oracle-leg", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--no-parity", action="store_true",
                   help="skip the oracle check of the step's sampled outputs before timing")
    p.add_argument("--suite", action="store_true",
                   help="instead of the decode step, time every other workload (int8, Q4_K FFN, "
                        "f16 GEMM, LM-head sweep) and print one JSON line per case")
    p.add_argument("--launch-floor", action="store_true",
                   help="instead of the decode step, time graphs of 96 dependent batch-1 Q4_K "
                        "mat-vec launches (896 columns, 1 to 4864 rows) and of 96 one-element "
                        "fill kernels, one JSON line per case")
    p.add_argument("--suite-filter", default="",
                   help="only suite cases whose name contains this (comma-separated alternatives)")
    p.add_argument("--summarize-pmc", nargs="+", metavar="CSV",
                   help="write the counter summary from rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE "
                        "and optionally the read request sizes) and exit")
    p.add_argument("--copy-calibration-mib", type=int, default=0,
                   help="before the step, copy this many MiB device-to-device three times "
                        "(a kernel of known traffic for scaling HBM counters)")
    return p.parse_args(argv)


# ---------------------------------------------------------------------------
# workload
# ---------------------------------------------------------------------------
def host_inputs(calls):
    """Host (numpy) inputs of the step's calls from the seeded generator:
    [(packed weight bytes, x [1][in] float32, bias or None)] in call order."""
    from dequantize_mat_vec_amd import synth
    out = []
    for layer, name, fmt, rows, inf, has_bias in calls:
        tidx = synth.TENSOR_INDEX[name]
        packed, _ = synth.matrix(fmt, synth.rng_for(CONFIG_INDEX, layer, tidx), rows, inf)
        x = synth.activations(synth.rng_for(CONFIG_INDEX, layer, 100 + tidx), 1, inf)
        b = synth.bias(synth.rng_for(CONFIG_INDEX, layer, 200 + tidx), rows) if has_bias else None
        out.append((packed, x, b))
    return out


def build_inputs(copies, calls=None, host=None):
    """Step inputs.  Each weight copy is one contiguous device buffer holding
    the step's tensors in the order they are used (Q, K, V, O, gate, up,
    down per layer, then the LM head), each at a 256-byte boundary, as a
    mapped model file would lay them out; weights[c][i] is a view of call
    i's tensor in copy c."""
    import numpy as np
    import torch
    from dequantize_mat_vec_amd import synth
    dev = torch.device("cuda:0")
    calls = synth.decode_step_calls() if calls is None else calls
    host = host_inputs(calls) if host is None else host
    offsets, total = [], 0
    xs, ys, biases = [], [], []
    for (packed, x, b), (_, _, _, out, _, _) in zip(host, calls):
        offsets.append(total)
        total += -(-packed.size // 256) * 256
        xs.append(torch.from_numpy(x.reshape(-1)).to(dev))
        ys.append(torch.empty(out, dtype=torch.float32, device=dev))
        biases.append(torch.from_numpy(b).to(dev) if b is not None else None)
    buf_host = np.zeros(total, dtype=np.uint8)
    for off, (p, _, _) in zip(offsets, host):
        buf_host[off:off + p.size] = p.reshape(-1)
    host_t = torch.from_numpy(buf_host)
    weights = []
    for _ in range(copies):
        buf = host_t.to(dev)
        weights.append([buf[off:off + p.size] for off, (p, _, _) in zip(offsets, host)])
    torch.cuda.synchronize()
    return calls, weights, xs, ys, biases


def plan_launches(calls, grouping):
    """Launches of one step as (format, [call indices]).  With grouping
    "stage", the projections of one dependency stage that read the same
    activations share a launch: Q/K/V, then O, then gate/up, then down, per
    layer (97 launches); with "none" every call is its own launch (169)."""
    if grouping == "none":
        return [(fmt, [i]) for i, (_, _, fmt, _, _, _) in enumerate(calls)]
    launches, i = [], 0
    stage_of = {"q": 0, "k": 0, "v": 0, "o": 1, "gate": 2, "up": 2, "down": 3, "lm_head": 4}
    while i < len(calls):
        layer, name, fmt, _, _, _ = calls[i]
        group = [i]
        j = i + 1
        while (j < len(calls) and calls[j][0] == layer and calls[j][2] == fmt
               and stage_of[calls[j][1]] == stage_of[name]):
            group.append(j)
            j += 1
        launches.append((fmt, group))
        i = j
    return launches


def make_step(lib, calls, launches, weights, xs, ys, biases, ffn="separate"):
    """A function issuing the step's launches on a stream handle; the op
    tables are built once so a step is only the C calls.  With ffn
    "swiglu" each layer's gate/up launch is the fused pesti_gemv_swiglu,
    writing h = silu(gate) * up into the gate call's output buffer, and the
    down projection reads h as its x (the step's data dependence in a
    model)."""
    import ctypes
    from dequantize_mat_vec_amd import _lib
    h_of_layer = {}
    if ffn == "swiglu":
        for fmt, idx in launches:
            names = [calls[i][1] for i in idx]
            if names == ["gate", "up"]:
                h_of_layer[calls[idx[0]][0]] = idx[0]
    plans = []
    for wl in weights:
        plan = []
        for fmt, idx in launches:
            names = [calls[i][1] for i in idx]
            if ffn == "swiglu" and names == ["gate", "up"]:
                g, u = idx
                _, _, _, out, inf, _ = calls[g]
                plan.append(("swiglu", (_lib.FORMAT_IDS[fmt], out, inf, wl[g].data_ptr(), wl[u].data_ptr(),
                                        xs[g].data_ptr(), ys[g].data_ptr())))
                continue
            arr = (_lib.GemvOp * len(idx))()
            for k, i in enumerate(idx):
                layer, name, _, out, inf, _ = calls[i]
                b = biases[i]
                x_ptr = xs[i].data_ptr()
                if name == "down" and layer in h_of_layer:
                    x_ptr = ys[h_of_layer[layer]].data_ptr()
                arr[k] = _lib.GemvOp(out, inf, wl[i].data_ptr(), None, x_ptr,
                                     ys[i].data_ptr(), b.data_ptr() if b is not None else None)
            plan.append(("group", (_lib.FORMAT_IDS[fmt], len(idx), ctypes.cast(arr, ctypes.c_void_p), arr)))
        plans.append(plan)
    fn = lib.pesti_gemv_group
    fn_swiglu = lib.pesti_gemv_swiglu

    def step(copy, stream_handle, only=None):
        """One step (or, with `only`, just the launches whose indices are in it)."""
        for idx, (kind, a) in enumerate(plans[copy]):
            if only is not None and idx not in only:
                continue
            if kind == "group":
                st = fn(a[0], a[1], a[2], 1, stream_handle)
            else:
                fid, out, inf, wg, wu, x, h = a
                st = fn_swiglu(fid, out, inf, wg, wu, None, None, x, h, 1, stream_handle)
            if st != 0:
                raise RuntimeError(f"launch {idx} failed with status {st}")
    return step


HALF_UNIT_MAX_ROWS = 2048   # the library's PESTI_HALF_UNIT_MAX_ROWS


def kernel_name(fmt, infs, outs):
    """Label of the mat-vec kernel instance one batch-1 launch uses: lanes
    per row L by the longest row (one row per lane group at batch 1); Q8_0
    rows of an even block count take two blocks per unit (q8_0x2), Q4_K ops
    of at most 2048 rows of at most 1024 weights half units (q4_kh; q4_ksh in
    the stream layout)."""
    if fmt == "q8_0" and all(inf % 64 == 0 for inf in infs):
        fmt = "q8_0x2"
    half = all(inf <= 1024 for inf in infs) and all(out <= HALF_UNIT_MAX_ROWS for out in outs)
    if fmt == "q4_k" and half:
        fmt = "q4_kh"
    if fmt == "q4_k_stream" and half:
        fmt = "q4_ksh"
    units = max({"q8_0x2": inf // 64, "q8_0": inf // 32, "q4_k": -(-inf // 64), "q4_kh": 2 * -(-inf // 64),
                 "q4_k_stream": inf // 64, "q4_ksh": 2 * (inf // 64),
                 "q6_k": 4 * -(-inf // 256)}[fmt] for inf in infs)
    lanes = 16 if units <= 16 else (32 if units <= 32 else 64)
    rows = 1
    return f"gemv_kernel<{fmt}, L={lanes}, B=1, R={rows}>"


# ---------------------------------------------------------------------------
# Suite: the other workloads, one call shape at a time
# ---------------------------------------------------------------------------
MFMA_F16_PEAK_TFLOPS = 2500.0
SUITE_REPLAYS = 10   # graph replays per suite case (median, p10, p90 of their per-call times)


def suite_cases():
    """(name, kind, params) for every non-step workload."""
    from dequantize_mat_vec_amd import synth
    cases = [("i8row 896x896 b1", "gemv", ("i8row", 896, 896, 1)),
             ("q4_k 4864x896 b1 (gate/up)", "gemv", ("q4_k", 4864, 896, 1)),
             ("q4_k 896x4864 b1 (down)", "gemv", ("q4_k", 896, 4864, 1)),
             # sustained rate at the FFN shapes: 8 independent matrices (each
             # with its own x and y) in one grouped launch
             ("q4_k 4864x896 b1 (gate/up) x8 grouped", "group", ("q4_k", 4864, 896, 8)),
             ("q4_k 896x4864 b1 (down) x8 grouped", "group", ("q4_k", 896, 4864, 8)),
             ("q8_0 4864x896 b1 x8 grouped", "group", ("q8_0", 4864, 896, 8))]
    for m in (8, 32, 64):
        for name, k, n in synth.GPT2_LINEARS:
            cases.append((f"f16 gemm {name} m{m} ({k}->{n})", "gemm", (m, k, n)))
    for fmt in ("q8_0", "q4_k", "q6_k"):
        for b in (1, 2, 4, 8):
            cases.append((f"{fmt} lm-head 151936x896 b{b}", "gemv", (fmt, synth.QWEN_VOCAB, 896, b)))
    for fmt in ("q2_k", "q3_k", "q5_k"):
        for b in (1, 2, 4, 8):
            cases.append((f"{fmt} lm-head 151936x896 b{b}", "gemv", (fmt, synth.QWEN_VOCAB, 896, b)))
        cases.append((f"{fmt} 4864x896 b1 (gate/up)", "gemv", (fmt, 4864, 896, 1)))
    for b in (1, 2, 4, 8):
        cases.append((f"i4row lm-head 151936x896 b{b}", "gemv", ("i4row", synth.QWEN_VOCAB, 896, b)))
    cases += [("i4row 4864x896 b1 (gate/up)", "gemv", ("i4row", 4864, 896, 1)),
              ("i4row 896x4864 b1 (down)", "gemv", ("i4row", 896, 4864, 1))]
    cases.append(("q8_0 gpt2 lm-head 50257x768 b1", "gemv", ("q8_0", synth.GPT2_VOCAB, 768, 1)))
    # prompt-width products on quantized weights, with the binary16-weight
    # GEMM at the same shapes for comparison
    qshapes = (("gate/up", synth.QWEN_FFN, synth.QWEN_HIDDEN), ("down", synth.QWEN_HIDDEN, synth.QWEN_FFN),
               ("lm-head", synth.QWEN_VOCAB, synth.QWEN_HIDDEN))
    for m in (16, 64):
        for label, n, k in qshapes:
            for fmt in ("q8_0", "q2_k", "q3_k", "q4_k", "q5_k", "q6_k"):
                cases.append((f"{fmt} gemm {label} {n}x{k} m{m}", "qgemm", (fmt, m, n, k)))
            cases.append((f"f16 gemm {label} {n}x{k} m{m}", "gemm", (m, k, n)))
    # the Q4_K shapes of 896-weight rows again in the stream layout (504
    # bytes per row, no padding); appended so that earlier cases keep their
    # seeds
    cases += [("q4_k_stream lm-head 151936x896 b1", "gemv", ("q4_k_stream", synth.QWEN_VOCAB, 896, 1)),
              ("q4_k_stream 4864x896 b1 (gate/up)", "gemv", ("q4_k_stream", 4864, 896, 1)),
              ("q4_k_stream 4864x896 b1 (gate/up) x8 grouped", "group", ("q4_k_stream", 4864, 896, 8))]
    return cases


def suite_case_inputs(idx, name, kind, prm, rows_limit=None):
    """Host inputs of one suite case from the seeded generator (the GPU run
    and the oracle's timing leg draw the same values).  rows_limit caps the
    matrix's rows (the oracle is timed on a slice of the largest ones).
    Returns a dict of numpy arrays and sizes."""
    import numpy as np
    from dequantize_mat_vec_amd import synth
    rng = synth.rng_for(4 if "lm-head" in name else (0 if kind == "gemv" and prm[0] == "i8row" else 1), idx, 0)
    d = {"kind": kind, "nops": 1}
    if kind == "group":
        fmt, out, inf, nops = prm
        out = out if rows_limit is None else min(out, rows_limit)
        packed, scales = synth.matrix(fmt, rng, out, inf)
        d.update(fmt=fmt, out=out, inf=inf, nops=nops, batch=1, packed=packed, scales=scales,
                 xs=[synth.activations(rng, 1, inf) for _ in range(nops)],
                 algo=nops * call_bytes(fmt, out, inf, 1, False), flops=2.0 * out * inf * nops)
    elif kind == "gemv":
        fmt, out, inf, batch = prm
        out = out if rows_limit is None else min(out, rows_limit)
        packed, scales = synth.matrix(fmt, rng, out, inf)
        d.update(fmt=fmt, out=out, inf=inf, batch=batch, packed=packed, scales=scales,
                 x=synth.activations(rng, batch, inf), algo=call_bytes(fmt, out, inf, batch, False),
                 flops=2.0 * out * inf * batch)
    elif kind == "qgemm":
        fmt, m, n, k = prm
        n = n if rows_limit is None else min(n, rows_limit)
        packed = synth.quant_blocks(fmt, rng, n, k)
        d.update(fmt=fmt, m=m, n=n, k=k, packed=packed, x16=synth.f16_activations(rng, m, k),
                 bias=synth.bias(rng, n),
                 algo=int(n * k * NOMINAL_BYTES_PER_WEIGHT[fmt]) + 2 * m * k + 4 * m * n + 4 * n,
                 flops=2.0 * m * n * k)
    else:
        m, k, n = prm
        n = n if rows_limit is None else min(n, rows_limit)
        w16 = synth.f16_weights(rng, n, k)
        d.update(m=m, n=n, k=k, w16=w16, packed=w16.view(np.uint8), x16=synth.f16_activations(rng, m, k),
                 bias=synth.bias(rng, n), algo=2 * n * k + 2 * m * k + 4 * m * n + 4 * n,
                 flops=2.0 * m * n * k)
    return d


def run_suite(lib, args):
    """Each case: enough weight copies to pass 640 MB (so the 256 MB
    last-level cache holds none between uses), a HIP graph of `reps`
    launches cycling over them, timed between two events over 10 replays;
    µs per call = graph time / reps (median, p10, p90 over replays).  The
    same copies are then read by the library's streaming-read hook: the
    size-matched read ceiling the case is compared with.  Unless
    --no-cpu-baseline, each line also carries the oracle's time per call
    on the same inputs, measured in child processes (one BLAS thread and
    the whole CPU share)."""
    import ctypes
    import numpy as np
    import torch
    from dequantize_mat_vec_amd import _lib
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    out_lines = []
    oracle_times = {} if args.no_cpu_baseline else run_suite_oracle(args)
    for idx, (name, kind, prm) in enumerate(suite_cases()):
        if args.suite_filter and not any(f in name for f in args.suite_filter.split(",")):
            continue
        inp = suite_case_inputs(idx, name, kind, prm)
        nops, algo, flops = inp["nops"], inp["algo"], inp["flops"]
        packed = inp["packed"]
        nbytes = packed.size * (nops if kind == "group" else 1)
        if kind == "group":
            fmt, out, inf, batch = inp["fmt"], inp["out"], inp["inf"], 1
            packed = np.concatenate([packed.reshape(-1)] * nops)
            xg = [torch.from_numpy(v).to(dev) for v in inp["xs"]]
            yg = [torch.empty(out, dtype=torch.float32, device=dev) for _ in range(nops)]
        elif kind == "gemv":
            fmt, out, inf, batch = inp["fmt"], inp["out"], inp["inf"], inp["batch"]
            x = torch.from_numpy(inp["x"]).to(dev)
            y = torch.empty(batch * out, dtype=torch.float32, device=dev)
            sc = torch.from_numpy(inp["scales"]).to(dev) if inp["scales"] is not None else None
        else:
            if kind == "qgemm":
                fmt = inp["fmt"]
            m, n, k = inp["m"], inp["n"], inp["k"]
            x16 = torch.from_numpy(inp["x16"].view(np.uint16)).to(dev)
            b = torch.from_numpy(inp["bias"]).to(dev)
            y = torch.empty(m * n, dtype=torch.float32, device=dev)
            # the GEMMs run with a workspace (split K where the shape asks for it)
            gfid = _lib.GEMM_FORMAT_IDS[fmt if kind == "qgemm" else "f16"]
            ws_bytes = lib.pesti_gemm_workspace_bytes(gfid, m, n, k)
            if ws_bytes < 0:
                raise RuntimeError(f"{name}: workspace query status {ws_bytes}")
            gws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        copies = max(2, int(np.ceil(640e6 / nbytes)))
        host = torch.from_numpy(np.ascontiguousarray(packed).reshape(-1))
        ws = [host.to(dev) for _ in range(copies)]
        reps = int(min(max(copies, 40), 400))
        if kind == "group":
            per = nbytes // nops
            tables = []
            for w in ws:
                arr = (_lib.GemvOp * nops)()
                for k in range(nops):
                    arr[k] = _lib.GemvOp(out, inf, w.data_ptr() + k * per, None, xg[k].data_ptr(),
                                         yg[k].data_ptr(), None)
                tables.append(arr)

        def launch(i, sh):
            if kind == "group":
                st = lib.pesti_gemv_group(_lib.FORMAT_IDS[fmt], nops,
                                          ctypes.cast(tables[i % copies], ctypes.c_void_p), 1, sh)
            elif kind == "gemv":
                st = (getattr(lib, f"pesti_gemv_{fmt}")(out, inf, ws[i % copies].data_ptr(), sc.data_ptr(),
                                                       x.data_ptr(), y.data_ptr(), None, batch, sh)
                      if fmt in ("i8row", "i4row") else
                      getattr(lib, f"pesti_gemv_{fmt}")(out, inf, ws[i % copies].data_ptr(),
                                                       x.data_ptr(), y.data_ptr(), None, batch, sh))
            else:
                st = lib.pesti_gemm_smallm_ws(gfid, m, n, k, ws[i % copies].data_ptr(), x16.data_ptr(),
                                              y.data_ptr(), b.data_ptr(), gws.data_ptr(), ws_bytes, sh)
            if st != 0:
                raise RuntimeError(f"{name}: status {st}")

        def timed(fn_launch):
            """Per-call µs of `reps` launches captured in one graph, over
            SUITE_REPLAYS replays: (median, p10, p90)."""
            with torch.cuda.stream(stream):
                fn_launch(0, stream.cuda_stream)
                torch.cuda.synchronize()
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    for i in range(reps):
                        fn_launch(i, torch.cuda.current_stream().cuda_stream)
                g.replay()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                per = []
                for _ in range(SUITE_REPLAYS):
                    e0.record(stream)
                    g.replay()
                    e1.record(stream)
                    torch.cuda.synchronize()
                    per.append(e0.elapsed_time(e1) * 1e3 / reps)
            del g
            q = np.percentile(per, [50, 10, 90])
            return float(q[0]), float(q[1]), float(q[2])

        med, p10, p90 = timed(launch)
        # Size-matched streaming-read ceiling: the same stored bytes, read from
        # the same rotating copies by a plain vector-load kernel.
        partial = torch.empty(_lib.READ_GROUPS, dtype=torch.int32, device=dev)
        rbytes = nbytes - nbytes % 16

        def read_launch(i, sh):
            st = lib.pesti_stream_read(ws[i % copies].data_ptr(), rbytes, partial.data_ptr(), sh)
            if st != 0:
                raise RuntimeError(f"stream read: status {st}")

        read_us = timed(read_launch)[0]
        gbs = algo / med / 1e3
        rec = {"case": name, "us_per_call": round(med, 3), "us_p10": round(p10, 3), "us_p90": round(p90, 3),
               "GB/s": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
               "TFLOP/s": round(flops / med / 1e6, 3), "algorithmic_bytes": int(algo),
               "stored_bytes": int(nbytes), "read_ceiling_GB/s": round(rbytes / read_us / 1e3, 1),
               "stored_GB/s": round(nbytes / med / 1e3, 1),
               "frac_of_read_ceiling": round(read_us * nbytes / rbytes / med, 4) if rbytes else None,
               "weight_copies": copies}
        if kind in ("gemm", "qgemm"):
            rec["mfma_frac"] = round(flops / med / 1e6 / MFMA_F16_PEAK_TFLOPS, 5)
        if name in oracle_times:
            one, many = oracle_times[name]
            rec["cpu_baseline"] = {
                "kind": "oracle", "unit": "us/call",
                "us_per_call_1thread": one["us_per_call"], "us_per_call_all_cores": many["us_per_call"],
                "cores": many["threads"], "gpu_speedup_1thread": round(one["us_per_call"] / med, 1),
                "gpu_speedup_all_cores": round(many["us_per_call"] / med, 1), "sample": one["sample"]}
        print(json.dumps(rec), flush=True)
        out_lines.append(rec)
        del ws
        torch.cuda.empty_cache()
    return out_lines


SUITE_ORACLE_ROWS = 8192     # rows of the largest matrices the oracle is timed on


def suite_oracle_leg(filt):
    """Runs in a child process (BLAS/OpenMP threads set by the parent): the
    oracle's time per call of every suite case on the same seeded inputs.
    Matrices of more than SUITE_ORACLE_ROWS rows are timed on their first
    SUITE_ORACLE_ROWS rows and scaled by rows (the oracle's cost is linear
    in the rows it expands).  One JSON line per case."""
    import oracle
    threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    for idx, (name, kind, prm) in enumerate(suite_cases()):
        if filt and not any(f in name for f in filt.split(",")):
            continue
        full = {"group": prm[1], "gemv": prm[1], "qgemm": prm[2], "gemm": prm[2]}[kind]
        inp = suite_case_inputs(idx, name, kind, prm, SUITE_ORACLE_ROWS)
        rows = {"group": "out", "gemv": "out"}.get(kind, "n")
        timed_rows = inp[rows]

        def once():
            if kind == "group":
                for xv in inp["xs"]:
                    oracle.gemv_packed(inp["fmt"], inp["packed"], inp["out"], inp["inf"], xv, None,
                                       inp["scales"])
            elif kind == "gemv":
                oracle.gemv_packed(inp["fmt"], inp["packed"], inp["out"], inp["inf"], inp["x"], None,
                                   inp["scales"])
            elif kind == "qgemm":
                oracle.gemm_packed(inp["fmt"], inp["packed"], inp["n"], inp["k"], inp["x16"], inp["bias"])
            else:
                oracle.gemm_f16(inp["x16"], inp["w16"], inp["bias"])

        reps, spent = 0, 0.0
        while spent < 0.3 or reps < 2:
            t0 = time.perf_counter()
            once()
            spent += time.perf_counter() - t0
            reps += 1
        us = spent / reps * 1e6 * full / timed_rows
        sample = (f"float64 oracle, {threads} thread(s), {reps} call(s)"
                  + (f" on the first {timed_rows} of {full} rows, scaled by rows" if timed_rows < full else ""))
        print(json.dumps({"case": name, "us_per_call": round(us, 1), "threads": threads, "sample": sample}),
              flush=True)


def run_suite_oracle(args):
    """{case: (1-thread timing, all-cores timing)} from two child runs of
    suite_oracle_leg."""
    host = host_cpu()
    share = int(os.environ.get("OMP_NUM_THREADS") or host["affinity"])
    res = {}
    for threads in (1, share):
        env = dict(os.environ)
        for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
            env[k] = str(threads)
        env["HIP_VISIBLE_DEVICES"] = ""
        cmd = [sys.executable, os.path.abspath(__file__), "--suite-oracle-leg", "--suite-filter",
               args.suite_filter]
        # each case's line is echoed to stderr as it arrives (progress of a
        # leg that can take minutes)
        with subprocess.Popen(cmd, env=env, stdout=subprocess.PIPE, stderr=subprocess.PIPE,
                              text=True) as proc:
            for line in proc.stdout:
                if line.startswith("{"):
                    r = json.loads(line)
                    res.setdefault(r["case"], []).append(r)
                    print(f"oracle, {threads} thread(s): {r['case']}: {r['us_per_call']} us", file=sys.stderr,
                          flush=True)
            err = proc.stderr.read()
            rc = proc.wait(timeout=60)
        if rc != 0:
            raise RuntimeError(f"suite oracle leg failed: {err[-2000:]}")
    print(json.dumps({"suite_oracle_host": host}), flush=True)
    return {k: tuple(v) for k, v in res.items() if len(v) == 2}


# ---------------------------------------------------------------------------
# HBM traffic from rocprofv3 counters
# ---------------------------------------------------------------------------
PMC_SUMMARY = os.path.join(HERE, "profiles", "decode_step_pmc.txt")
SRC_DIR = os.path.join(HERE, "dequantize_mat_vec_amd", "csrc")


def source_digest():
    """sha256 over the HIP sources: counters taken on other sources are stale."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(SRC_DIR)):
        if name.endswith((".hip", ".h")):
            h.update(name.encode())
            with open(os.path.join(SRC_DIR, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def run_launch_floor(lib):
    """Per-launch cost of the decode step's dependent launches against their
    floor: a graph of 96 dependent batch-1 Q4_K mat-vecs (896 columns, each
    launch its own x; launch i reads weight copy i mod C - at 896 rows and
    fewer C = 64 copies that stay in the last-level cache, at 4864 rows
    C = 229 copies that exceed it), and a graph of 96 dependent fills of one
    float (torch's fill kernel: launch and completion only)."""
    import numpy as np
    import torch
    import dequantize_mat_vec_amd as dmv
    from dequantize_mat_vec_amd import synth
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    n, inf = 96, 896

    def time_graph(issue):
        with torch.cuda.stream(stream):
            issue()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=stream):
                issue()
            for _ in range(3):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(10):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
        return e0.elapsed_time(e1) / 10 / n * 1e3

    for rows in (1, 16, 128, 896, 4864):
        rng = synth.rng_for(9, rows, 0)
        packed = synth.quant_blocks("q4_k", rng, rows, inf).reshape(-1)
        nb = packed.size
        copies = int(640e6 // nb) + 1 if nb > 1e6 else 64
        big = torch.from_numpy(np.tile(packed, copies)).to(dev)
        xs = [torch.from_numpy(synth.activations(rng, 1, inf)).to(dev) for _ in range(n)]
        y = torch.empty(rows, dtype=torch.float32, device=dev)

        def issue():
            for i in range(n):
                c = i % copies
                dmv.pesti_gemv_q4_k(rows, inf, big[c * nb:(c + 1) * nb], xs[i], y, None, 1, stream=stream)
        us = time_graph(issue)
        print(json.dumps({"case": f"q4_k {rows}x{inf} b1, 96 dependent launches", "us_per_launch": round(us, 3),
                          "weight_copies": copies}), flush=True)
        del big
    z = torch.empty(1, device=dev)

    def fills():
        for i in range(n):
            z.fill_(float(i))
    print(json.dumps({"case": "fill of one float, 96 dependent launches", "us_per_launch": round(time_graph(fills), 3)}),
          flush=True)


def summarize_pmc(fetch_csv, write_csv, requests_csv=None, calib_mib=256):
    """Per-launch HBM bytes of every mat-vec kernel shape in a bench run, from
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each scaled by what the
    same counter reads for the device-to-device copy of calib_mib MiB that
    the run starts with (it moves calib_mib MiB each way); with requests_csv
    also the read bytes counted by request size (add_request_bytes)."""
    import csv
    import statistics
    known_kib = calib_mib * 1024.0
    out = {"source_sha256": source_digest(), "calibration": {}, "kernels": {}}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = list(csv.DictReader(open(path)))
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > known_kib / 4]
        factor = known_kib / statistics.median(copies)
        out["calibration"][counter] = {"copy_mib": calib_mib, "counter_kib": statistics.median(copies),
                                       "factor": round(factor, 5)}
        per = {}
        for r in rows:
            if "gemv_kernel" not in r["Kernel_Name"]:
                continue
            key = f"{r['Kernel_Name'].split('(')[0]} grid={r['Grid_Size']}"
            per.setdefault(key, []).append(float(r["Counter_Value"]) * factor * 1024.0)
        for key, vals in per.items():
            d = out["kernels"].setdefault(key, {})
            d[counter.lower() + "_bytes"] = round(statistics.median(vals))
            d["dispatches"] = len(vals)
    if requests_csv:
        add_request_bytes(out, requests_csv, calib_mib)
    with open(PMC_SUMMARY, "w") as f:
        f.write(json.dumps(out, indent=1) + "\n")
    return out


REQUEST_COUNTERS = (("TCC_EA0_RDREQ_32B_sum", 32), ("TCC_EA0_RDREQ_64B_sum", 64),
                    ("TCC_EA0_RDREQ_128B_sum", 128))


def add_request_bytes(out, path, calib_mib):
    """Read bytes per dispatch counted by request size, 32 n32 + 64 n64 +
    128 n128, from one counter pass over the three L2-to-fabric read request
    counters.  Unlike a single scale factor fitted to the copy's 128-byte
    requests, this counts a 32- or 64-byte request at its own size; the
    copy's figure is kept to show the sum needs no scaling."""
    import csv
    import statistics
    rows = list(csv.DictReader(open(path)))
    per_dispatch = {}
    for r in rows:
        size = dict(REQUEST_COUNTERS).get(r["Counter_Name"])
        if size is None:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"].split("(")[0], r["Grid_Size"])
        per_dispatch[key] = per_dispatch.get(key, 0.0) + size * float(r["Counter_Value"])
    copies = [v for (_, name, _), v in per_dispatch.items()
              if "copyBuffer" in name and v > calib_mib * (1 << 20) / 4]
    out["calibration"]["read_requests"] = {
        "copy_mib": calib_mib, "bytes": round(statistics.median(copies)) if copies else None,
        "ratio_to_copy_size": round(statistics.median(copies) / (calib_mib * (1 << 20)), 5) if copies else None}
    per = {}
    for (_, name, grid), v in per_dispatch.items():
        if "gemv_kernel" in name:
            per.setdefault(f"{name} grid={grid}", []).append(v)
    for key, vals in per.items():
        out["kernels"].setdefault(key, {})["read_request_bytes"] = round(statistics.median(vals))


def dominant_traffic(kernel_label, read_key="fetch_size_bytes"):
    """Average HBM bytes per launch of the dominant kernel from the committed
    counter summary (reads by read_key, plus writes), or None if it is
    missing, lacks that figure or was taken on other sources."""
    if not os.path.exists(PMC_SUMMARY):
        return None
    try:
        summ = json.load(open(PMC_SUMMARY))
    except ValueError:
        return None
    if summ.get("source_sha256") != source_digest():
        return None
    fmt = kernel_label.split("<")[1].split(",")[0]
    lanes = kernel_label.split("L=")[1].split(",")[0]
    tag = {"q8_0": "FmtQ8_0", "q8_0x2": "FmtQ8_0x2", "q4_k": "FmtQ4_K", "q4_kh": "FmtQ4_KH",
           "q4_k_stream": "FmtQ4_KS", "q4_ksh": "FmtQ4_KSH", "q6_k": "FmtQ6_K"}[fmt]
    # one entry per launch shape of the kernel; every shape of the decode step
    # occurs equally often (once per layer), so the per-launch average is
    # the plain mean over shapes
    shapes = [d for key, d in summ["kernels"].items() if f"{tag}, {lanes}, 1," in key]
    if not shapes or any(read_key not in d for d in shapes):
        return None
    vals = [d[read_key] + d.get("write_size_bytes", 0) for d in shapes]
    return sum(vals) / len(vals)


# ---------------------------------------------------------------------------
# Parity of the timed step: sampled outputs of the step's own buffers,
# checked by the oracle in the CPU leg's process
# ---------------------------------------------------------------------------
PARITY_LAYERS = (0, 1, 23)      # every kernel shape of the step: Q6_K down on 0, Q4_K down on 1
PARITY_HEAD_ROWS = 8192
GEMV_REL = 1e-4


def parity_sample(calls, ys, skip_names=()):
    """Outputs of the step just run, read back from its own y buffers: every
    row of every call of PARITY_LAYERS and PARITY_HEAD_ROWS rows of the LM
    head spread over its length (both ends included); calls named in
    skip_names are left out.  {call index: (rows, y values)}."""
    import numpy as np
    sample = {}
    for i, (layer, name, _, out, _, _) in enumerate(calls):
        if name in skip_names:
            continue
        if name == "lm_head":
            rng = np.random.default_rng([CONFIG_INDEX, 7])
            rows = np.unique(np.concatenate([np.linspace(0, out - 1, PARITY_HEAD_ROWS // 2).astype(np.int64),
                                             rng.integers(0, out, PARITY_HEAD_ROWS // 2)]))
        elif layer in PARITY_LAYERS:
            rows = np.arange(out)
        else:
            continue
        sample[i] = (rows, ys[i].cpu().numpy()[rows])
    return sample


def parity_leg(path):
    """Runs in the CPU leg's child process: regenerates the sampled calls'
    inputs from the seeds, runs the float64 oracle on the sampled rows and
    holds every output to 1e-4 * sum|w x| + 1e-6."""
    import numpy as np
    from dequantize_mat_vec_amd import synth
    import oracle
    data = np.load(path)
    calls = synth.decode_step_calls(layout=str(data["layout"]) if "layout" in data.files else "rows")
    n_out, worst, failures = 0, 0.0, []
    for i in data["calls"]:
        i = int(i)
        layer, name, fmt, out, inf, _ = calls[i]
        rows, y = data[f"rows_{i}"], data[f"y_{i}"]
        packed, x, b = host_inputs([calls[i]])[0]
        if fmt == "q4_k_stream":   # rows have no fixed stride: the whole (small) matrix
            y_ref, s_ref = oracle.gemv_packed(fmt, packed, out, inf, x, b)
            y_ref, s_ref = y_ref[:, rows], s_ref[:, rows]
        else:
            sub = packed.reshape(out, -1)[rows]
            y_ref, s_ref = oracle.gemv_packed(fmt, sub, len(rows), inf, x, None if b is None else b[rows])
        ratio = np.abs(y.astype(np.float64) - y_ref[0]) / (GEMV_REL * s_ref[0] + 1e-6)
        bad = ~(ratio <= 1.0)
        n_out += len(rows)
        worst = max(worst, float(np.nanmax(np.where(np.isfinite(ratio), ratio, np.inf))))
        if np.any(bad):
            failures.append(f"{name}{layer} ({fmt} {out}x{inf}): {int(bad.sum())} rows, "
                            f"first row {int(rows[np.argmax(bad)])}")
    return {"ok": not failures, "calls": int(len(data["calls"])), "outputs": n_out,
            "worst_err_over_bound": round(worst, 4), "failures": failures[:8]}


def run_parity(calls, ys, skip_names=(), layout="rows"):
    """parity_sample() in this process, the check in a child process (the
    oracle runs only in the CPU leg)."""
    import tempfile
    import numpy as np
    sample = parity_sample(calls, ys, skip_names)
    fd, path = tempfile.mkstemp(suffix=".npz")
    os.close(fd)
    try:
        arrays = {"calls": np.array(sorted(sample), dtype=np.int64), "layout": np.array(layout)}
        for i, (rows, y) in sample.items():
            arrays[f"rows_{i}"] = rows
            arrays[f"y_{i}"] = y
        np.savez(path, **arrays)
        env = dict(os.environ)
        env["HIP_VISIBLE_DEVICES"] = ""
        cmd = [sys.executable, os.path.abspath(__file__), "--parity-leg", path]
        res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
        if res.returncode != 0:
            raise RuntimeError(f"parity check failed to run: {res.stderr[-2000:]}")
        return json.loads(res.stdout.strip().splitlines()[-1])
    finally:
        os.unlink(path)


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on a bounded sample of the same step
# ---------------------------------------------------------------------------
def cpu_leg(seconds, layout):
    """Runs in a child process (BLAS/OpenMP threads set by the parent): times
    the oracle (float64 dequantize + dot) on whole calls of the step in
    stream order (the LM head as a 16384-row slice), with the step's Q4_K
    layout, passing over the step again until `seconds` of work is done."""
    from dequantize_mat_vec_amd import synth
    import oracle
    calls = synth.decode_step_calls(layout=layout)
    done_bytes, spent, ncalls, passes = 0, 0.0, 0, 0
    first = last = None
    while spent < seconds:
        passes += 1
        for layer, name, fmt, out, inf, has_bias in calls:
            if spent >= seconds:
                break
            tidx = synth.TENSOR_INDEX[name]
            rng = synth.rng_for(CONFIG_INDEX, layer, tidx)
            rows = min(out, 16384) if name == "lm_head" else out
            packed, _ = synth.matrix(fmt, rng, rows, inf)
            x = synth.activations(synth.rng_for(CONFIG_INDEX, layer, 100 + tidx), 1, inf)
            b = synth.bias(synth.rng_for(CONFIG_INDEX, layer, 200 + tidx), rows) if has_bias else None
            t0 = time.perf_counter()
            oracle.gemv_packed(fmt, packed, rows, inf, x, b)
            spent += time.perf_counter() - t0
            done_bytes += call_bytes(fmt, rows, inf, 1, has_bias)
            ncalls += 1
            last = f"{name}{layer}" if name != "lm_head" else f"lm_head[{rows} rows]"
            first = first or last
    return {"value": done_bytes / spent / 1e9, "seconds": spent, "bytes": done_bytes,
            "calls": ncalls, "passes": passes, "first": first, "last": last}


def host_cpu():
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"model": model, "os_cpu_count": os.cpu_count(),
            "affinity": len(os.sched_getaffinity(0))}


def run_cpu_leg(seconds, threads, layout):
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        env[k] = str(threads)
    env["HIP_VISIBLE_DEVICES"] = ""
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-leg",
           "--cpu-sample-seconds", str(seconds), "--layout", layout]
    res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
    if res.returncode != 0:
        raise RuntimeError(f"cpu baseline failed: {res.stderr[-2000:]}")
    return json.loads(res.stdout.strip().splitlines()[-1])


def run_cpu_baseline(seconds, layout):
    """The oracle on the host cores, twice: one BLAS/OpenMP thread (the
    reported value) and the process's whole CPU share (OMP_NUM_THREADS if
    set, else the affinity mask)."""
    host = host_cpu()
    share = int(os.environ.get("OMP_NUM_THREADS") or host["affinity"])
    one = run_cpu_leg(seconds, 1, layout)
    many = run_cpu_leg(seconds / 2, share, layout)

    def sample(r, threads):
        return (f"float64 oracle, {threads} thread(s), {r['calls']} calls of the decode step in "
                f"stream order ({r['first']} .. {r['last']}, {r['passes']} pass(es), Q4_K {layout} layout), "
                f"{r['bytes']} nominal bytes in {r['seconds']:.1f} s")
    return {"value": round(one["value"], 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": sample(one, 1), "host": host,
            "all_cores": {"value": round(many["value"], 4), "unit": "GB/s", "cores": share,
                          "sample": sample(many, share)}}


# ---------------------------------------------------------------------------
def main(argv=None):
    args = parse_args(argv)
    if args.cpu_leg:
        print(json.dumps(cpu_leg(args.cpu_sample_seconds, args.layout)))
        return 0
    if args.parity_leg:
        print(json.dumps(parity_leg(args.parity_leg)))
        return 0
    if args.suite_oracle_leg:
        suite_oracle_leg(args.suite_filter)
        return 0
    if args.summarize_pmc:
        if len(args.summarize_pmc) not in (2, 3):
            print("--summarize-pmc takes FETCH_CSV WRITE_CSV [REQUESTS_CSV]", file=sys.stderr)
            return 2
        print(json.dumps(summarize_pmc(*args.summarize_pmc), indent=1))
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the decode-step mat-vec runs on a single MI355X)", file=sys.stderr)
        return 2

    import torch
    import dequantize_mat_vec_amd as dmv
    lib = dmv.load()
    torch.cuda.set_device(0)
    if args.suite:
        run_suite(lib, args)
        return 0
    if args.launch_floor:
        run_launch_floor(lib)
        return 0
    if args.ffn == "swiglu" and (args.grouping != "stage" or args.layout != "rows"):
        print("--ffn swiglu fuses the gate/up stage: it needs --grouping stage and --layout rows",
              file=sys.stderr)
        return 2
    from dequantize_mat_vec_amd import synth
    calls, weights, xs, ys, biases = build_inputs(args.copies, synth.decode_step_calls(layout=args.layout))
    launches = plan_launches(calls, args.grouping)
    step = make_step(lib, calls, launches, weights, xs, ys, biases, args.ffn)
    bytes_per_step = sum(call_bytes(fmt, out, inf, 1, hb) for _, _, fmt, out, inf, hb in calls)
    stream = torch.cuda.Stream()
    sh = stream.cuda_stream

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    graphs = None
    with torch.cuda.stream(stream):
        for i in range(2):
            step(i % args.copies, sh)
        torch.cuda.synchronize()
        if args.mode == "graph":
            graphs = []
            for c in range(args.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(c, torch.cuda.current_stream().cuda_stream)
                graphs.append(g)
            torch.cuda.synchronize()

        def run(i):
            if graphs is not None:
                graphs[i % args.copies].replay()
            else:
                step(i % args.copies, sh)

        for i in range(args.warmup):
            run(i)
        torch.cuda.synchronize()
        parity = None
        if not args.no_parity:
            # the oracle's check of the buffers the timed steps use: one more
            # step (weight copy 0), its outputs poisoned first
            for y in ys:
                y.fill_(float("nan"))
            run(0)
            torch.cuda.synchronize()
            # with the fused SwiGLU the gate buffer holds h and the down
            # projection reads it: those calls are checked by the test suite
            parity = run_parity(calls, ys, ("gate", "up", "down") if args.ffn == "swiglu" else (), args.layout)
        t0 = time.perf_counter()
        for i in range(args.steps):
            run(i)
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0

        # Per-kernel durations.  Inside a HIP graph the step's kernels run
        # back to back, so a kernel's duration is measured by replaying a
        # graph of only that kernel's launches of the step (same buffers,
        # weight copies alternated) between two HIP events on the launch
        # stream: time per replay / launches per replay.
        names = [kernel_name(fmt, [calls[i][4] for i in idx], [calls[i][3] for i in idx])
                 for fmt, idx in launches]
        if args.ffn == "swiglu":
            names = [n.replace("R=1>", "R=1, gate/up paired, SwiGLU>")
                     if [calls[i][1] for i in idx] == ["gate", "up"] else n
                     for n, (_, idx) in zip(names, launches)]
        per_kernel = {}
        for name in sorted(set(names)):
            only = {i for i, n in enumerate(names) if n == name}
            subs = []
            for c in range(args.copies):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    step(c, torch.cuda.current_stream().cuda_stream, only)
                subs.append(g)
            for i in range(3):
                subs[i % args.copies].replay()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(args.kernel_steps):
                subs[i % args.copies].replay()
            e1.record(stream)
            torch.cuda.synchronize()
            per_kernel[name] = (e0.elapsed_time(e1), only)

    per_name = {}
    for name, (ms, only) in per_kernel.items():
        per_name[name] = {
            "ms": ms, "launches": len(only) * args.kernel_steps,
            "bytes": args.kernel_steps * sum(
                call_bytes(calls[i][2], calls[i][3], calls[i][4], 1, calls[i][5])
                for li in only for i in launches[li][1])}
    dom_name, dom = max(per_name.items(), key=lambda kv: kv[1]["ms"])
    avg_s = dom["ms"] / dom["launches"] / 1e3
    bytes_per_launch = dom["bytes"] / dom["launches"]
    achieved = bytes_per_launch / avg_s / 1e9

    traffic = dominant_traffic(dom_name)
    traffic_req = dominant_traffic(dom_name, "read_request_bytes")
    ms_per_step = elapsed / args.steps * 1e3
    value = bytes_per_step / (ms_per_step / 1e3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 (Q4_K/Q6_K/Q8_0 weights)",
        "data": "synthetic (seeded random blocks of the model's shapes)",
        "config": {"workload": "Qwen2.5-0.5B decode step, linear layers, batch 1: 24 x "
                               "{Q,K,V,O,gate,up Q4_K; down Q4_K/Q6_K} + 151936x896 Q8_0 LM head "
                               "= 169 mat-vecs", "bytes_per_step": bytes_per_step,
                   "launch": args.mode, "launches_per_step": len(launches),
                   "grouping": args.grouping, "ffn": args.ffn, "q4_k_layout": args.layout,
                   "weight_copies": args.copies},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (None if traffic is None else int(traffic)),
                     "traffic_by_request_size": (None if traffic_req is None else int(traffic_req)),
                     "bytes_per_launch": int(bytes_per_launch),
                     "avg_launch_us": round(avg_s * 1e6, 3)},
        "kernels": {k: {"launches_per_step": v["launches"] // args.kernel_steps,
                        "avg_us": round(v["ms"] / v["launches"] * 1e3, 3),
                        "GB/s": round(v["bytes"] / (v["ms"] / 1e3) / 1e9, 1)}
                    for k, v in sorted(per_name.items(), key=lambda kv: -kv[1]["ms"])},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = run_cpu_baseline(args.cpu_sample_seconds, args.layout)
    else:
        result["cpu_baseline"] = None
    result["parity"] = None if parity is None else parity["ok"]
    result["parity_detail"] = parity
    print(json.dumps(result), flush=True)
    return 0 if parity is None or parity["ok"] else 1


if __name__ == "__main__":
    sys.exit(main())
