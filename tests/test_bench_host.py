"""Host logic of the benchmark (no GPU): the decode step's call list and
launch plan, its nominal byte count, kernel labels, the counter summary's
scaling and the one-GPU rule."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from dequantize_mat_vec_amd import synth  # noqa: E402


def test_decode_step_has_169_calls_in_stream_order():
    calls = synth.decode_step_calls()
    assert len(calls) == 24 * 7 + 1
    names = [c[1] for c in calls[:7]]
    assert names == ["q", "k", "v", "o", "gate", "up", "down"]
    assert calls[-1][1:] == ("lm_head", "q8_0", 151936, 896, False)
    # Q6_K down projections on even layers only, Q4_K everywhere else
    for layer, name, fmt, out, inf, has_bias in calls[:-1]:
        want = "q6_k" if name == "down" and layer % 2 == 0 else "q4_k"
        assert fmt == want, (layer, name)
        assert has_bias == (name in ("q", "k", "v"))
        assert (out, inf) == {"q": (896, 896), "k": (128, 896), "v": (128, 896), "o": (896, 896),
                              "gate": (4864, 896), "up": (4864, 896), "down": (896, 4864)}[name]


def test_plan_groups_each_dependency_stage():
    calls = synth.decode_step_calls()
    stage = bench.plan_launches(calls, "stage")
    assert len(stage) == 97
    kinds = [tuple(calls[i][1] for i in idx) for _, idx in stage]
    assert kinds[:4] == [("q", "k", "v"), ("o",), ("gate", "up"), ("down",)]
    assert kinds[-1] == ("lm_head",)
    covered = sorted(i for _, idx in stage for i in idx)
    assert covered == list(range(len(calls)))          # every call once, in order
    for fmt, idx in stage:
        assert all(calls[i][2] == fmt for i in idx)    # one format per launch
        assert len({calls[i][0] for i in idx}) == 1    # one layer per launch
    none = bench.plan_launches(calls, "none")
    assert len(none) == 169 and all(len(idx) == 1 for _, idx in none)


def test_nominal_bytes_of_the_step():
    """Weights at 4.5 (Q4_K), 6.5625 (Q6_K) and 8.5 (Q8_0) bits per weight:
    24 layers of Q/K/V/O/gate/up/down plus the 151936 x 896 LM head hold
    359 403 520 bytes; x, y and the Q/K/V biases add the rest."""
    calls = synth.decode_step_calls()
    weights = sum(out * inf * bench.NOMINAL_BYTES_PER_WEIGHT[fmt] for _, _, fmt, out, inf, _ in calls)
    assert weights == 359403520
    total = sum(bench.call_bytes(fmt, out, inf, 1, hb) for _, _, fmt, out, inf, hb in calls)
    xy = sum(4 * (inf + out) for _, _, _, out, inf, _ in calls)
    bias = sum(4 * out for _, _, _, out, _, hb in calls if hb)
    assert total == weights + xy + bias == 362324992


def test_call_bytes_per_format():
    assert bench.call_bytes("q8_0", 10, 64, 1, False) == 10 * 68 + 4 * (64 + 10)
    assert bench.call_bytes("q4_k", 3, 256, 2, True) == 3 * 144 + 8 * (256 + 3) + 12
    assert bench.call_bytes("i8row", 5, 32, 1, False) == 5 * 32 + 20 + 4 * 37   # codes + row scales
    assert bench.call_bytes("i4row", 5, 64, 1, False) == 5 * 32 + 20 + 4 * 69


@pytest.mark.parametrize("fmt,inf,lanes,label", [("q4_k", 896, 32, "q4_kh"), ("q4_k", 4864, 64, "q4_k"),
                                                ("q6_k", 4864, 64, "q6_k"), ("q6_k", 896, 16, "q6_k"),
                                                ("q8_0", 896, 16, "q8_0x2"), ("q8_0", 4864, 64, "q8_0x2"),
                                                ("q8_0", 800, 32, "q8_0"), ("q4_k", 2048, 32, "q4_k"),
                                                ("q4_k", 512, 16, "q4_kh")])
def test_kernel_label_lanes(fmt, inf, lanes, label):
    """Q8_0 rows of an even block count run the two-blocks-per-unit kernel,
    Q4_K rows of at most 1024 weights the half-unit one."""
    assert bench.kernel_name(fmt, [inf], [896]) == f"gemv_kernel<{label}, L={lanes}, B=1, R=1>"


def test_half_units_only_for_ops_of_at_most_2048_rows():
    """The step's Q/K/V and O launches run in half units, its 4864-row
    gate/up launch in whole runs."""
    assert bench.kernel_name("q4_k", [896, 896, 896], [896, 128, 128]) == "gemv_kernel<q4_kh, L=32, B=1, R=1>"
    assert bench.kernel_name("q4_k", [896, 896], [4864, 4864]) == "gemv_kernel<q4_k, L=16, B=1, R=1>"
    assert bench.kernel_name("q4_k_stream", [896], [2048]) == "gemv_kernel<q4_ksh, L=32, B=1, R=1>"
    assert bench.kernel_name("q4_k_stream", [896], [2049]) == "gemv_kernel<q4_k_stream, L=16, B=1, R=1>"


def test_counter_summary_scales_by_the_copy(tmp_path, monkeypatch):
    """FETCH_SIZE / WRITE_SIZE (KiB per dispatch) are scaled by what the
    same counter reads for a copy of known size; medians per kernel shape."""
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "pmc.txt"))
    fields = ["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]

    def write(path, counter, copy_kib, kernel_kib):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=fields)
            w.writeheader()
            for v in (copy_kib, copy_kib):
                w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": "512",
                            "Counter_Name": counter, "Counter_Value": v})
            for v in kernel_kib:
                w.writerow({"Kernel_Name": "void pesti::gemv_kernel<pesti::FmtQ4_K, 16, 1, 1, 1, false>(x)",
                            "Grid_Size": "14336", "Counter_Name": counter, "Counter_Value": v})
    fetch, write_csv = tmp_path / "f.csv", tmp_path / "w.csv"
    write(fetch, "FETCH_SIZE", 131072.0, [100.0, 300.0, 200.0])    # copy reads half: factor 2
    write(write_csv, "WRITE_SIZE", 262144.0, [4.0, 4.0, 4.0])      # factor 1
    out = bench.summarize_pmc(str(fetch), str(write_csv), calib_mib=256)
    assert out["calibration"]["FETCH_SIZE"]["factor"] == 2.0
    assert out["calibration"]["WRITE_SIZE"]["factor"] == 1.0
    (key, d), = out["kernels"].items()
    assert key.endswith("grid=14336")
    assert d["fetch_size_bytes"] == 2 * 200 * 1024 and d["write_size_bytes"] == 4 * 1024
    assert d["dispatches"] == 3
    assert json.load(open(tmp_path / "pmc.txt"))["source_sha256"] == bench.source_digest()


def test_read_request_bytes_count_each_size(tmp_path, monkeypatch):
    """The request-size pass sums 32 n32 + 64 n64 + 128 n128 per dispatch
    (three counter rows of one dispatch), median per kernel shape, with no
    scaling; the copy's sum is reported against its size."""
    monkeypatch.setattr(bench, "PMC_SUMMARY", str(tmp_path / "pmc.txt"))
    fields = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"]
    simple = tmp_path / "s.csv"
    with open(simple, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerow({"Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": "512",
                    "Counter_Name": "FETCH_SIZE", "Counter_Value": 262144.0})
    req = tmp_path / "r.csv"
    copy_n128 = 256 * (1 << 20) // 128
    kernel = "void pesti::gemv_kernel<pesti::FmtQ4_KS, 16, 1, 1, 1, false>(x)"
    with open(req, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for name, val in (("TCC_EA0_RDREQ_32B_sum", 0), ("TCC_EA0_RDREQ_64B_sum", 0),
                          ("TCC_EA0_RDREQ_128B_sum", copy_n128)):
            w.writerow({"Dispatch_Id": 1, "Kernel_Name": "__amd_rocclr_copyBuffer", "Grid_Size": "512",
                        "Counter_Name": name, "Counter_Value": val})
        for disp, (n32, n64, n128) in ((2, (1, 2, 10)), (3, (3, 0, 20)), (4, (0, 0, 1))):
            for name, val in (("TCC_EA0_RDREQ_32B_sum", n32), ("TCC_EA0_RDREQ_64B_sum", n64),
                              ("TCC_EA0_RDREQ_128B_sum", n128)):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": kernel, "Grid_Size": "14336",
                            "Counter_Name": name, "Counter_Value": val})
    out = bench.summarize_pmc(str(simple), str(simple), str(req), calib_mib=256)
    assert out["calibration"]["read_requests"]["ratio_to_copy_size"] == 1.0
    (key, d), = out["kernels"].items()
    assert key.endswith("grid=14336")
    # dispatch sums 32 + 128 + 1280 = 1440, 96 + 2560 = 2656, 128: median 1440
    assert d["read_request_bytes"] == 1440


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_default_contract_arguments():
    a = bench.parse_args([])
    assert (a.gpus, a.steps, a.warmup, a.mode, a.grouping, a.ffn) == (1, 50, 10, "graph", "stage", "separate")


class _HostY:
    """Stands in for a device y buffer: .cpu().numpy() gives the values."""

    def __init__(self, v):
        self.v = v

    def cpu(self):
        return self

    def numpy(self):
        return self.v


def _oracle_outputs(calls, sample_calls):
    import numpy as np
    import oracle
    ys = [None] * len(calls)
    host = bench.host_inputs([calls[i] for i in sample_calls])
    for i, (packed, x, b) in zip(sample_calls, host):
        _, _, fmt, out, inf, _ = calls[i]
        y, _ = oracle.gemv_packed(fmt, packed, out, inf, x, b)
        ys[i] = _HostY(y[0].astype(np.float32))
    return ys


def test_parity_leg_accepts_rounded_oracle_and_rejects_a_planted_error(tmp_path, monkeypatch):
    """The benchmark's parity check (sample of the step's outputs, checked by
    the oracle in the CPU leg): float32-rounded oracle outputs pass, one
    output moved past the bound fails and is named."""
    import numpy as np
    monkeypatch.setattr(bench, "PARITY_HEAD_ROWS", 64)
    calls = synth.decode_step_calls(layers=2)
    # layer 23 does not exist in a 2-layer step; the sample takes layers 0, 1
    # and the head
    sample_calls = list(range(len(calls)))
    ys = _oracle_outputs(calls, sample_calls)
    monkeypatch.setattr(synth, "decode_step_calls", lambda layers=2, layout="rows": calls)
    sample = bench.parity_sample(calls, ys)
    assert sorted(sample) == sample_calls
    head_rows = sample[len(calls) - 1][0]
    assert head_rows[0] == 0 and head_rows[-1] == 151935 and len(head_rows) >= 32

    def check(sample):
        path = tmp_path / "s.npz"
        arrays = {"calls": np.array(sorted(sample), dtype=np.int64)}
        for i, (rows, y) in sample.items():
            arrays[f"rows_{i}"] = rows
            arrays[f"y_{i}"] = y
        np.savez(path, **arrays)
        return bench.parity_leg(str(path))

    res = check(sample)
    assert res["ok"] and res["calls"] == len(calls) and res["worst_err_over_bound"] < 1.0
    rows, y = sample[6]                       # layer 0's Q6_K down projection
    y = y.copy()
    y[17] += 1e-2 * (np.abs(y[17]) + 1.0)
    sample[6] = (rows, y)
    res = check(sample)
    assert not res["ok"] and "down0" in res["failures"][0] and "first row 17" in res["failures"][0]


def test_parity_sample_skips_the_fused_calls():
    import numpy as np
    calls = synth.decode_step_calls(layers=2)
    ys = [_HostY(np.zeros(c[3], np.float32)) for c in calls]
    sample = bench.parity_sample(calls, ys, ("gate", "up", "down"))
    assert all(calls[i][1] not in ("gate", "up", "down") for i in sample)


def test_stream_layout_step_keeps_the_plan_and_the_nominal_bytes():
    """With the stream layout the 896-column Q4_K calls change format only:
    same launches, same nominal bytes per step (the stored bytes shrink)."""
    rows = synth.decode_step_calls()
    stream = synth.decode_step_calls(layout="stream")
    assert [c[:2] + c[3:] for c in rows] == [c[:2] + c[3:] for c in stream]
    changed = [c for c in stream if c[2] == "q4_k_stream"]
    assert {c[1] for c in changed} == {"q", "k", "v", "o", "gate", "up"} and len(changed) == 24 * 6
    assert len(bench.plan_launches(stream, "stage")) == 97
    assert (sum(bench.call_bytes(f, o, i, 1, b) for _, _, f, o, i, b in rows)
            == sum(bench.call_bytes(f, o, i, 1, b) for _, _, f, o, i, b in stream))


def test_stream_kernel_label():
    """Stream-layout rows of at most 1024 weights run in half units at batch
    1, longer ones in whole runs."""
    assert bench.kernel_name("q4_k_stream", [896], [896]) == "gemv_kernel<q4_ksh, L=32, B=1, R=1>"
    assert bench.kernel_name("q4_k_stream", [512], [896]) == "gemv_kernel<q4_ksh, L=16, B=1, R=1>"
    assert bench.kernel_name("q4_k_stream", [4864], [896]) == "gemv_kernel<q4_k_stream, L=64, B=1, R=1>"
