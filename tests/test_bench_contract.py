"""The benchmark's output contract, checked on the CPU: each bench line is one
JSON object with the fixed keys, a roofline object of the right kind for its
op, the workload named in its config; a request for several GPUs is refused
with an explanation; and every committed counter summary names a kernel and
workload the benchmark knows, with the code hash and traffic it reports."""
import json
import os
import re
import subprocess
import sys

import pytest

import bench
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better", "scaling",
        "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"}
ROOF = {"bound", "achieved", "peak", "unit", "frac", "traffic", "hbm_gbs", "hbm_frac", "mfma_busy", "valu_trans_f32",
        "mfma_exec_over_conv", "valu_active"}


def _timing(op, peak=2500.0):
    settle = {"extra_launches": 100, "seconds": 1.0}
    if op == "decode":
        return {"gbs": 5000.0, "ms_per_step": 1.0, "bytes": 5 << 30, "splits_workspace_bytes": 0,
                "median_launch_ms": 1.0, "min_launch_ms": 0.9, "warmup_settle": settle,
                "cold_median_launch_ms": 1.2}
    return {"tflops": 1000.0, "ms_per_step": 0.3, "flops": 2.7e11, "peak": peak, "median_launch_ms": 0.3,
            "min_launch_ms": 0.29, "warmup_settle": settle, "cold_median_launch_ms": 0.32}


def _check(line, name, bound, unit):
    assert KEYS <= set(line), KEYS - set(line)
    assert ROOF <= set(line["roofline"]), ROOF - set(line["roofline"])
    json.loads(json.dumps(line))  # one JSON object
    assert line["config"]["workload"] == name
    assert line["n_gpus"] == 1 and line["data"] == "synthetic" and line["higher_is_better"] is True
    r = line["roofline"]
    assert r["bound"] == bound and r["unit"] == unit and line["unit"] == unit
    assert r["frac"] == round(r["achieved"] / r["peak"], 4)
    assert r["traffic"] is None or isinstance(r["traffic"], int)
    # counter-derived fields come together from one hash-checked summary
    if r["traffic"] is None:
        assert r["hbm_gbs"] is None and r["hbm_frac"] is None
    else:
        assert r["hbm_gbs"] == round(r["traffic"] / (line["ms_per_step"] * 1e-3) / 1e9, 1)
        assert r["hbm_frac"] == round(r["hbm_gbs"] / bench.HBM_PEAK_GBS, 4)
    assert r["mfma_busy"] is None or 0.0 < r["mfma_busy"] <= 1.0
    assert r["valu_trans_f32"] is None or isinstance(r["valu_trans_f32"], int)
    assert r["mfma_exec_over_conv"] is None or r["mfma_exec_over_conv"] >= 0.99
    assert r["valu_active"] is None or 0.0 < r["valu_active"] < 1.0
    assert "warmup_settle" in line
    c = line["cold_cache"]
    assert c is None or (c["unit"] == unit and c["value"] > 0 and c["median_launch_ms"] > 0)


@pytest.mark.parametrize("op,name", [("fwd", workloads.HEADLINE), ("bwd", workloads.HEADLINE),
                                     ("fwd", "c2_fp32_b1h8n1024d64"), ("bwd", "c2_fp32_b1h8n1024d64"),
                                     ("decode", "d1_bf16_decode_b8h32q1k32768d128")])
def test_bench_line_contract(op, name):
    w = workloads.WORKLOADS[name]
    line = bench.line_for(w, _timing(op, bench.PEAK_TFLOPS[w.dtype]), 10, 5, None, op)
    if op == "decode":
        _check(line, name, "hbm", "GB/s")
        assert line["roofline"]["peak"] == bench.HBM_PEAK_GBS
    else:
        _check(line, name, "mfma", "TFLOP/s")
        assert line["roofline"]["peak"] == bench.PEAK_TFLOPS[w.dtype]
    assert line["dtype"] == w.dtype


def test_varlen_line_contract():
    name = next(iter(workloads.VARLEN_WORKLOADS))
    w = workloads.VARLEN_WORKLOADS[name]
    line = bench.line_varlen(w, _timing("varlen"), 10, 5, None)
    _check(line, name, "mfma", "TFLOP/s")


def test_several_gpus_are_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and not r.stdout.strip()


def test_committed_counter_summaries_are_well_formed():
    paths = [p for p in os.listdir(os.path.join(ROOT, "profiles")) if p.endswith("__hbm_traffic_and_counters.md")]
    assert paths, "no committed counter summary"
    known = set(workloads.WORKLOADS) | set(workloads.VARLEN_WORKLOADS)
    for p in paths:
        tag, wl, _ = p.split("__")
        assert wl in known, p
        text = open(os.path.join(ROOT, "profiles", p)).read()
        assert re.search(r"^kernel_code_sha256: [0-9a-f]{64}$", text, re.M), p
        assert re.search(r"^traffic_bytes_per_launch: \d+$", text, re.M), p
        assert re.search(r"^mfma_busy_pct: [0-9.]+$", text, re.M), p
        assert re.search(r"^valu_trans_f32_per_launch: \d+$", text, re.M), p
        assert re.search(r"^mfma_flop_executed_over_convention: [0-9.]+$", text, re.M), p
        assert re.search(r"^valu_active_pct: [0-9.]+$", text, re.M), p
        assert "rocprofv3 --pmc FETCH_SIZE" in text and "rocprofv3 --pmc WRITE_SIZE" in text, p
        trace = os.path.join(ROOT, "profiles", f"{tag}__{wl}__kernel_trace.md")
        assert os.path.exists(trace), f"{p}: no kernel trace summary beside it"
