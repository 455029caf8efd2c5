"""Benchmark of exact tiled attention on one MI355X.

Default (--op fwd): a step is one fa_fwd call over the whole batch of the
workload (all of the hot path: Q-tile load, K/V streaming, both MFMA
contractions, online softmax, causal skipping, epilogue), inputs already
resident in HBM.  Throughput is the metric's convention: FLOPs =
4*B*H*Nq*Nk*D, halved when causal, per second, in TFLOP/s.

--op bwd: a step is one fa_bwd call (delta/LSE preprocessing, dQ kernel,
dK/dV kernel) on the forward's O and LSE; FLOPs = 2.5x the forward
convention (five products of the forward's size).

--op decode: a step is one fa_fwd_splitkv call (key-range partials, then
the merge) on a decoding workload (few query rows, long KV cache); the
path is bound by HBM, so the value is algorithmic bytes (Q, K, V read once,
O and LSE written once) per second in GB/s against 8 TB/s.

--op varlen: a step is one fa_fwd_varlen call over a packed batch of
sequences of mixed lengths; FLOPs = the forward convention summed over the
sequences.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--settle-seconds S]
                    [--workload NAME] [--op fwd|bwd|decode|varlen] [--no-cpu-baseline] [--all]

Warm-up: W launches, then more until S seconds have passed and the launch
time has settled (the shader clock ramps up over the first few hundred
milliseconds of load); the extra launches are reported in ``warmup_settle``,
``warmup`` stays W.  Prints one JSON line per workload.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of dense MFMA peak, bf16 causal N=4096 D=128"
METRIC_BWD = "attention bwd TFLOP/s (2.5x the forward FLOP convention) and % of dense MFMA peak"
METRIC_DECODE = "attention decode (split-KV) algorithmic HBM GB/s and % of 8 TB/s"
METRIC_VARLEN = "attention fwd over packed variable-length sequences, TFLOP/s and % of dense MFMA peak"
HBM_PEAK_GBS = 8000.0
# Published MI355X dense peaks (TFLOP/s) by compute dtype.
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--settle-seconds", type=float, default=1.0,
                   help="after the --warmup launches, keep launching until at least this long has passed "
                        "since the first one and two successive batches agree within 2%% (the GPU's clock "
                        "and caches reach steady state); reported in the line's warmup_settle field")
    p.add_argument("--workload", default=workloads.HEADLINE)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0,
                   help="target CPU time of the oracle sample")
    p.add_argument("--all", action="store_true", help="one line per measured workload (c1..c5)")
    p.add_argument("--op", choices=("fwd", "bwd", "decode", "varlen"), default="fwd")
    p.add_argument("--copy-calib-mib", type=int, default=0,
                   help="after timing, run 3 plain device copies of this many MiB (a reference "
                        "kernel of known traffic for rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    return p.parse_args()


def kernel_tag(w, op: str = "fwd") -> str:
    if op == "varlen":
        return f"fa_fwd_varlen_{w.dtype}_d{w.D}_{'causal' if w.causal else 'noncausal'}"
    if op == "decode":
        return f"fa_fwd_splitkv_{w.dtype}_d{w.D}"
    if op == "bwd" and w.dtype == "fp32":
        return f"fa_bwd_32_d{w.D}_{'causal' if w.causal else 'noncausal'}"
    if op == "bwd":
        return f"fa_bwd_16_{w.dtype}_d{w.D}_{'causal' if w.causal else 'noncausal'}"
    if w.dtype == "fp32":
        return f"fa_fwd_32_d{w.D}_{'causal' if w.causal else 'noncausal'}"
    # the forward kernel these workloads' grids run (all fill the CUs)
    kern = "fa_fwd_rs" if w.D in (128, 256) else "fa_fwd_16"
    return f"{kern}_{w.dtype}_d{w.D}_{'causal' if w.causal else 'noncausal'}"


CSRC = os.path.join(ROOT, "exact_tiled_attention_15_amd", "csrc")
# The code of a kernel: the shared device helpers and its source file, with
# the compile flags of the build units that compile that file.
KERNEL_SOURCES = (os.path.join(CSRC, "fa_device.h"), os.path.join(CSRC, "fa_kernels.hip"))
KERNEL_SOURCES_BWD = (os.path.join(CSRC, "fa_device.h"), os.path.join(CSRC, "fa_bwd.hip"))
KERNEL_SOURCES_BWD32 = (os.path.join(CSRC, "fa_device.h"), os.path.join(CSRC, "fa_bwd32.hip"))


def kernel_sources(w: workloads.Workload, op: str = "fwd"):
    """The source files whose code an op's kernels on this workload run
    (decode and varlen run the forward file's kernels; decode also depends on
    the key-range plan of the C ABI source)."""
    if op == "bwd":
        return KERNEL_SOURCES_BWD32 if w.dtype == "fp32" else KERNEL_SOURCES_BWD
    if op == "decode":
        return KERNEL_SOURCES + (os.path.join(CSRC, "fa_api.cpp"),)
    return KERNEL_SOURCES


def kernel_code_sha256(paths=KERNEL_SOURCES) -> str:
    """SHA-256 of the kernel sources with // comments and blank lines removed,
    followed by the compile flags (no paths) of every build unit that
    compiles one of them: it names the code the counters were taken on, and
    survives comment edits."""
    import hashlib

    import exact_tiled_attention_15_amd.build as build

    lines = []
    for path in paths:
        for line in open(path, encoding="utf-8"):
            code = line.split("//", 1)[0].rstrip()
            if code:
                lines.append(code)
        for name, src, extra in build.UNITS:
            if os.path.basename(src) == os.path.basename(path):
                flags = [f for f in build.FLAGS + build.DEVICE_FLAGS + extra if not os.path.isabs(f)]
                lines.append(f"unit {name}: {' '.join(flags)}")
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


COUNTER_KEYS = ("kernel_code_sha256", "traffic_bytes_per_launch", "mfma_busy_pct", "valu_trans_f32_per_launch",
                "mfma_flop_executed_over_convention", "valu_active_pct")


def committed_counters(w, op: str = "fwd"):
    """The machine-readable fields of the committed rocprofv3 counter summary
    of this op's kernels on this workload (HBM bytes per launch from the
    FETCH_SIZE / WRITE_SIZE passes; MFMA-busy percent and transcendental VALU
    instructions per launch from the SQ pass), or {} when there is none or
    the kernel code has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kernel_tag(w, op)}__{w.name}__hbm_traffic_and_counters.md")
    if not os.path.exists(path):
        return {}
    fields = {}
    for line in open(path):
        if ":" in line and line.split(":")[0] in COUNTER_KEYS:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    if fields.get("kernel_code_sha256") != kernel_code_sha256(kernel_sources(w, op)):
        return {}
    return fields


def counter_fields(w, op: str, ms_per_step: float):
    """Roofline extras from the committed counters: the HBM rate those bytes
    make at this run's step time (GB/s, against the 8 TB/s datasheet peak),
    the MFMA-busy fraction and the transcendental (exp) instruction count of
    the SQ pass, and from the wave-cycle pass the executed MFMA FLOPs over the
    convention's and the share of wave-cycles issuing VALU/MFMA instructions;
    None where the summary lacks them or is stale."""
    c = committed_counters(w, op)
    traffic = int(c["traffic_bytes_per_launch"]) if "traffic_bytes_per_launch" in c else None
    busy = float(c["mfma_busy_pct"]) / 100.0 if "mfma_busy_pct" in c else None
    trans = int(c["valu_trans_f32_per_launch"]) if "valu_trans_f32_per_launch" in c else None
    ratio = float(c["mfma_flop_executed_over_convention"]) if "mfma_flop_executed_over_convention" in c else None
    valu = float(c["valu_active_pct"]) / 100.0 if "valu_active_pct" in c else None
    gbs = round(traffic / (ms_per_step * 1e-3) / 1e9, 1) if traffic is not None and ms_per_step > 0 else None
    return {"traffic": traffic, "hbm_gbs": gbs, "hbm_frac": round(gbs / HBM_PEAK_GBS, 4) if gbs else None,
            "mfma_busy": busy, "valu_trans_f32": trans, "mfma_exec_over_conv": ratio, "valu_active": valu}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info

        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return os.cpu_count() or 1


def cpu_baseline(w: workloads.Workload, target_s: float, op: str = "fwd"):
    """The float64 oracle, as it stands, on whole (b, h) heads of the same
    workload, head after head until about ``target_s`` seconds have passed."""
    import oracle

    q, k, v = workloads.make_inputs(w)
    do = workloads.make_dout(w) if op == "bwd" else None
    heads = 0
    t_total = 0.0
    BH = w.B * w.H
    while heads < BH and t_total < target_s:
        b, h = divmod(heads, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        qh, kh, vh = (x[sl].double().numpy() for x in (q, k, v))
        t0 = time.perf_counter()
        if op == "bwd":
            oracle.attention_backward(qh, kh, vh, do[sl].double().numpy(), w.causal)
        else:
            oracle.attention_forward(qh, kh, vh, w.causal)
        t_total += time.perf_counter() - t0
        heads += 1
    if op == "decode":
        wh = w.replace(B=1, H=heads)
        return {
            "value": round(workloads.algorithmic_bytes(wh) / t_total / 1e9, 4),
            "unit": "GB/s",
            "cores": blas_threads(),
            "kind": "oracle",
            "sample": f"{heads} of {BH} (b,h) heads of {w.name}, float64, {t_total:.1f} s",
        }
    conv = workloads.conv_flops_bwd if op == "bwd" else workloads.conv_flops
    flops = conv(1, heads, w.Nq, w.Nk, w.D, w.causal)
    return {
        "value": round(flops / t_total / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{heads} of {BH} (b,h) heads of {w.name}, full rows, float64, {t_total:.1f} s",
    }


def settle(step, warmup: int, seconds: float, batch: int = 20, cap_s: float = 10.0):
    """Warm-up: ``warmup`` launches, then batches of ``batch`` launches until
    at least ``seconds`` have passed since the first launch and two
    successive batches take the same time within 2% (the clock and caches at
    steady state), or ``cap_s`` has passed.  Returns the extra launches and
    the seconds spent, reported beside the requested warm-up count."""
    import torch

    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    extra, prev = 0, None
    while True:
        elapsed = time.perf_counter() - t0
        if elapsed >= cap_s:
            break
        tb = time.perf_counter()
        for _ in range(batch):
            step()
        torch.cuda.synchronize()
        dt = time.perf_counter() - tb
        extra += batch
        settled = prev is not None and abs(dt - prev) <= 0.02 * prev
        prev = dt
        if time.perf_counter() - t0 >= seconds and settled:
            break
    return {"extra_launches": extra, "seconds": round(time.perf_counter() - t0, 3)}


COLD_FLUSH_MIB = 512  # bytes written between cold calls: more than the L2s and the MALL hold


def cold_timing(step, stream, calls: int):
    """Per-call durations (ms) with the caches cold: before each call a
    COLD_FLUSH_MIB MiB device buffer is overwritten on the same stream, which
    evicts the inputs from every L2 and from the MALL (inputs stay in HBM).
    The call is queued right behind that write, so the device never idles
    between the two (an idle gap lets the shader clock drop, and the call
    then measured 15% slower for that reason alone); HIP events bracket the
    call, and the device is synchronized after each call."""
    import torch

    flush = torch.empty(COLD_FLUSH_MIB << 20, dtype=torch.uint8, device=torch.device("cuda:0"))
    out = []
    for _ in range(calls):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        flush.zero_()
        a.record(stream)
        step()
        b.record(stream)
        torch.cuda.synchronize()
        out.append(a.elapsed_time(b))
    del flush
    return out


def bench_one(w: workloads.Workload, steps: int, warmup: int, op: str = "fwd", settle_s: float = 1.0):
    import torch

    import exact_tiled_attention_15_amd as fa

    fa.load_library()
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in workloads.make_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    code = fa._dtype_code(q)

    def fwd_step():
        rc = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                       w.B, w.H, w.Nq, w.Nk, w.D, int(w.causal), code, sptr)
        if rc != 0:
            raise fa.FaError(rc)

    step = fwd_step
    if op == "bwd":
        fwd_step()  # the backward consumes the forward's O and LSE
        do = workloads.make_dout(w).to(dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws_bytes = fa.fa_bwd_workspace_size(w.B, w.H, w.Nq)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
        scale = 1.0 / w.D**0.5

        def bwd_step():
            rc = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                           ws_bytes, w.B, w.H, w.Nq, w.Nk, w.D, scale, int(w.causal), code, sptr)
            if rc != 0:
                raise fa.FaError(rc)

        step = bwd_step
    elif op == "decode":
        ws_bytes = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.Nq, w.Nk, w.D, 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
        scale = 1.0 / w.D**0.5

        def decode_step():
            rc = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                   ws.data_ptr(), ws_bytes, w.B, w.H, w.Nq, w.Nk, w.D, scale, 0, int(w.causal),
                                   code, sptr)
            if rc != 0:
                raise fa.FaError(rc)

        step = decode_step

    warm = settle(step, warmup, settle_s)
    # Whole timed region: K back-to-back launches between two events on the
    # launch stream.
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_region = e0.elapsed_time(e1) / steps
    # Per-launch events (same stream) for the median launch duration.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in evs]
    cold = statistics.median(cold_timing(step, stream, min(steps, 20)))
    conv = workloads.conv_flops_bwd if op == "bwd" else workloads.conv_flops
    flops = conv(w.B, w.H, w.Nq, w.Nk, w.D, w.causal)
    tflops = flops / (ms_region * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    if op == "decode":
        nbytes = workloads.algorithmic_bytes(w)
        return {
            "cold_median_launch_ms": cold,
            "ms_per_step": ms_region,
            "wall_s": wall,
            "median_launch_ms": statistics.median(per),
            "min_launch_ms": min(per),
            "gbs": nbytes / (ms_region * 1e-3) / 1e9,
            "bytes": nbytes,
            "flops": flops,
            "splits_workspace_bytes": ws_bytes,
            "warmup_settle": warm,
        }
    return {
        "cold_median_launch_ms": cold,
        "ms_per_step": ms_region,
        "wall_s": wall,
        "median_launch_ms": statistics.median(per),
        "min_launch_ms": min(per),
        "tflops": tflops,
        "peak": peak,
        "flops": flops,
        "warmup_settle": warm,
    }


def bench_varlen(w: workloads.VarlenWorkload, steps: int, warmup: int, settle_s: float = 1.0):
    import torch

    import exact_tiled_attention_15_amd as fa

    fa.load_library()
    dev = torch.device("cuda:0")
    q, k, v, cu_q, cu_k = (t.to(dev) for t in workloads.make_varlen_inputs(w))
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sptr = stream.cuda_stream
    code = fa._dtype_code(q)
    H, tq, D = q.shape
    tk = k.shape[1]
    mq = max(w.lens_q)
    scale = 1.0 / D**0.5

    def step():
        rc = fa.fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                              cu_q.data_ptr(), cu_k.data_ptr(), w.B, H, tq, tk, mq, D, scale, int(w.causal), code,
                              sptr)
        if rc != 0:
            raise fa.FaError(rc)

    warm = settle(step, warmup, settle_s)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    cold = statistics.median(cold_timing(step, stream, min(steps, 20)))
    flops = workloads.varlen_flops(w)
    return {"ms_per_step": ms, "tflops": flops / (ms * 1e-3) / 1e12, "flops": flops, "peak": PEAK_TFLOPS[w.dtype],
            "warmup_settle": warm, "cold_median_launch_ms": cold}


def cpu_baseline_varlen(w: workloads.VarlenWorkload, target_s: float):
    """The float64 varlen oracle on whole sequences (all heads), sequence
    after sequence until about ``target_s`` seconds have passed."""
    import oracle

    q, k, v, cu_q, cu_k = workloads.make_varlen_inputs(w)
    t_total, n, flops = 0.0, 0, 0.0
    while n < w.B and t_total < target_s:
        q0, q1, k0, k1 = (int(x) for x in (cu_q[n], cu_q[n + 1], cu_k[n], cu_k[n + 1]))
        t0 = time.perf_counter()
        oracle.attention_varlen(q[:, q0:q1].double().numpy(), k[:, k0:k1].double().numpy(),
                                v[:, k0:k1].double().numpy(), [0, q1 - q0], [0, k1 - k0], w.causal)
        t_total += time.perf_counter() - t0
        flops += workloads.conv_flops(1, w.H, q1 - q0, k1 - k0, w.D, w.causal)
        n += 1
    return {"value": round(flops / t_total / 1e12, 6), "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "sample": f"{n} of {w.B} sequences of {w.name}, all heads, float64, {t_total:.1f} s"}


def cold_cache(r, unit: str):
    """Secondary figure: the median per-call time with the caches flushed
    before each call (cold_timing) and the rate it gives, or None when it was
    not measured."""
    ms = r.get("cold_median_launch_ms")
    if ms is None:
        return None
    work = r["bytes"] / 1e9 if unit == "GB/s" else r["flops"] / 1e12
    return {"median_launch_ms": round(ms, 5), "value": round(work / (ms * 1e-3), 3), "unit": unit,
            "flush_mib": COLD_FLUSH_MIB}


def line_varlen(w, r, steps, warmup, cpu):
    return {
        "metric": METRIC_VARLEN,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "D": w.D, "causal": w.causal, "seed": w.seed,
                   "total_q": int(sum(w.lens_q)), "total_k": int(sum(w.lens_k)), "lens_q": list(w.lens_q),
                   "flops_per_step": r["flops"], "parallelism": "single GPU", "op": "varlen"},
        "warmup_settle": r.get("warmup_settle"),
        "cold_cache": cold_cache(r, "TFLOP/s"),
        "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 3), "peak": r["peak"], "unit": "TFLOP/s",
                     "frac": round(r["tflops"] / r["peak"], 4), **counter_fields(w, "varlen", r["ms_per_step"])},
        "cpu_baseline": cpu,
    }


def line_for(w, r, steps, warmup, cpu, op="fwd"):
    props = {}
    try:
        import torch

        p = torch.cuda.get_device_properties(0)
        props = {"gpu": p.name, "cus": p.multi_processor_count,
                 "gcn_arch": getattr(p, "gcnArchName", "")}
    except Exception:
        pass
    if op == "decode":
        return {
            "metric": METRIC_DECODE,
            "value": round(r["gbs"], 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": steps,
            "warmup": warmup,
            "ms_per_step": round(r["ms_per_step"], 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                       "causal": w.causal, "seed": w.seed, "bytes_per_step": r["bytes"],
                       "splits_workspace_bytes": r["splits_workspace_bytes"], "parallelism": "single GPU",
                       "median_launch_ms": round(r["median_launch_ms"], 5),
                       "min_launch_ms": round(r["min_launch_ms"], 5), "op": op, **props},
            "warmup_settle": r.get("warmup_settle"),
            "cold_cache": cold_cache(r, "GB/s"),
            "roofline": {"bound": "hbm", "achieved": round(r["gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(r["gbs"] / HBM_PEAK_GBS, 4), **counter_fields(w, op, r["ms_per_step"])},
            "cpu_baseline": cpu,
        }
    return {
        "metric": METRIC_BWD if op == "bwd" else METRIC,
        "value": round(r["tflops"], 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "D": w.D,
                   "causal": w.causal, "seed": w.seed, "q_scale": w.q_scale,
                   "flops_per_step": r["flops"], "parallelism": "single GPU",
                   "median_launch_ms": round(r["median_launch_ms"], 5),
                   "min_launch_ms": round(r["min_launch_ms"], 5), "op": op, **props},
        "warmup_settle": r.get("warmup_settle"),
        "cold_cache": cold_cache(r, "TFLOP/s"),
        "roofline": {"bound": "mfma", "achieved": round(r["tflops"], 3), "peak": r["peak"],
                     "unit": "TFLOP/s", "frac": round(r["tflops"] / r["peak"], 4),
                     **counter_fields(w, op, r["ms_per_step"])},
        "cpu_baseline": cpu,
    }


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {a.gpus}); the attention forward "
              "shards over (batch, head) with no communication, so there is no multi-GPU "
              "step to time here.", file=sys.stderr)
        sys.exit(2)
    if a.op == "varlen":
        names = (list(workloads.VARLEN_WORKLOADS) if a.all or a.workload == workloads.HEADLINE else [a.workload])
        for i, n in enumerate(names):
            w = workloads.VARLEN_WORKLOADS[n]
            r = bench_varlen(w, a.steps, a.warmup, a.settle_seconds)
            cpu = None if a.no_cpu_baseline or i else cpu_baseline_varlen(w, a.cpu_seconds)
            print(json.dumps(line_varlen(w, r, a.steps, a.warmup, cpu)), flush=True)
        copy_calibration(a.copy_calib_mib)
        return
    names = ([n for n in workloads.WORKLOADS if n[:2] in ("c1", "c2", "c3", "c4", "c5") and "t_" not in n[:4]]
             if a.all else [a.workload])
    if a.op == "decode":
        names = ([n for n in workloads.WORKLOADS if n.startswith("d")] if a.all or a.workload == workloads.HEADLINE
                 else [a.workload])
    for n in names:
        w = workloads.WORKLOADS[n]
        r = bench_one(w, a.steps, a.warmup, a.op, a.settle_seconds)
        cpu = None
        if not a.no_cpu_baseline and n == names[0]:
            cpu = cpu_baseline(w, a.cpu_seconds, a.op)
        print(json.dumps(line_for(w, r, a.steps, a.warmup, cpu, a.op)), flush=True)
    copy_calibration(a.copy_calib_mib)


def copy_calibration(mib: int):
    """Three plain device copies of `mib` MiB: a reference kernel of known
    traffic for the rocprofv3 FETCH_SIZE / WRITE_SIZE counters."""
    if mib <= 0:
        return
    import torch

    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copy calibration: 3 x {mib} MiB device copies", file=sys.stderr)


if __name__ == "__main__":
    main()
