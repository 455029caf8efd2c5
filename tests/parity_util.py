"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
binding and compare with the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import math
import sys

import numpy as np

import oracle
import workloads

# Tolerances on max |GPU - oracle|: fp32 O 1e-4 / LSE 1e-5; bf16, fp16 O 2e-2 / LSE 1e-3.
TOL = {"fp32": (1e-4, 1e-5), "fp16": (2e-2, 1e-3), "bf16": (2e-2, 1e-3)}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_gpu(ts):
    return tuple(t.to("cuda:0").contiguous() for t in ts)


def run_gpu(q, k, v, causal, poison=True, softmax_scale=None):
    import torch

    import exact_tiled_attention_15_amd as fa

    B, H, Nq, D = q.shape
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if poison:
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
    fa.forward(q, k, v, causal, out=out, lse=lse, softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return out, lse


def compare_full(w: workloads.Workload, inputs_cpu, o_gpu, lse_gpu, tag="", scale=None):
    o = o_gpu.float().cpu().double().numpy()
    l = lse_gpu.cpu().double().numpy()
    assert np.isfinite(o).all(), f"{tag}: non-finite O"
    assert np.isfinite(l).all(), f"{tag}: non-finite LSE"
    O, L = oracle.attention_forward(*inputs_cpu, w.causal, scale=scale)
    eo = float(np.max(np.abs(o - O)))
    el = float(np.max(np.abs(l - L)))
    to, tl = TOL[w.dtype]
    log(f"  {tag} {w.name}: max|dO|={eo:.3e} (tol {to}) max|dLSE|={el:.3e} (tol {tl})")
    assert eo <= to, f"{tag}: O error {eo} > {to}"
    assert el <= tl, f"{tag}: LSE error {el} > {tl}"
    return eo, el


def sample_rows(w: workloads.Workload, n_heads=6, n_rand=24, seed=123):
    """Rows at the edges of 64/128-row tiles, the ends, and random ones."""
    r = np.random.default_rng(seed)
    BH = w.B * w.H
    heads = sorted(set([0, BH - 1] + list(r.integers(0, BH, n_heads - 2))))
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 129, 255, 256, w.Nq // 2, w.Nq - 129, w.Nq - 128,
             w.Nq - 65, w.Nq - 64, w.Nq - 2, w.Nq - 1}
    rows = []
    for bh in heads:
        b, h = divmod(int(bh), w.H)
        idx = {i for i in fixed if 0 <= i < w.Nq} | set(int(x) for x in r.integers(0, w.Nq, n_rand))
        rows += [(b, h, i) for i in sorted(idx)]
    return rows


def compare_sampled(w, inputs_cpu, o_gpu, lse_gpu, rows, tag=""):
    import torch

    assert bool(torch.isfinite(o_gpu).all()), f"{tag}: non-finite O"
    assert bool(torch.isfinite(lse_gpu).all()), f"{tag}: non-finite LSE"
    q, k, v = inputs_cpu
    O, L = oracle.attention_rows(q, k, v, w.causal, rows)
    idx = torch.tensor(rows, dtype=torch.long)
    og = o_gpu[idx[:, 0], idx[:, 1], idx[:, 2]].float().cpu().double().numpy()
    lg = lse_gpu[idx[:, 0], idx[:, 1], idx[:, 2]].cpu().double().numpy()
    eo = float(np.max(np.abs(og - O)))
    el = float(np.max(np.abs(lg - L)))
    to, tl = TOL[w.dtype]
    log(f"  {tag} {w.name} ({len(rows)} sampled rows): max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= to, f"{tag}: O error {eo} > {to}"
    assert el <= tl, f"{tag}: LSE error {el} > {tl}"
    return eo, el


def _oracle_pool():
    """Threads for head-by-head oracle calls (numpy releases the GIL in its
    matrix products and exponentials); BLAS limited to a few threads each so
    the pool does not oversubscribe the host's cores."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    n = max(1, min(8, (os.cpu_count() or 2) // 2))
    return ThreadPoolExecutor(n), threadpool_limits(limits=2)


def compare_whole(w, inputs_cpu, o_gpu, lse_gpu, tag="", scale=None):
    """Every element of O and LSE against the oracle, one (b, h) head at a
    time (the oracle's own row-chunked definition on each head), with the
    maximum errors over the whole tensors."""
    import torch

    assert bool(torch.isfinite(o_gpu).all()), f"{tag}: non-finite O"
    assert bool(torch.isfinite(lse_gpu).all()), f"{tag}: non-finite LSE"
    q, k, v = inputs_cpu
    og = o_gpu.float().cpu()
    lg = lse_gpu.cpu()

    def head(bh):
        b, h = divmod(bh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        O, L = oracle.attention_forward(q[sl], k[sl], v[sl], w.causal, scale=scale)
        eo = float(np.max(np.abs(og[sl].double().numpy() - O)))
        el = float(np.max(np.abs(lg[sl].double().numpy() - L)))
        return eo, el

    pool, limits = _oracle_pool()
    with pool, limits:
        errs = list(pool.map(head, range(w.B * w.H)))
    eo = max(e[0] for e in errs)
    el = max(e[1] for e in errs)
    to, tl = TOL[w.dtype]
    log(f"  {tag} {w.name} (whole tensors, {w.B * w.H} heads): max|dO|={eo:.3e} (tol {to}) "
        f"max|dLSE|={el:.3e} (tol {tl})")
    assert eo <= to, f"{tag}: O error {eo} > {to}"
    assert el <= tl, f"{tag}: LSE error {el} > {tl}"
    return eo, el
