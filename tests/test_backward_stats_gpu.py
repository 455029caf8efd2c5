"""GPU check of the backward's row statistics, read back from the workspace:
LSE log2(e) and delta = sum_d dO O per query row (the layout include/fa.h
states), against their definitions in float64 on the values the GPU stored
(the forward's O and LSE, rounded dO).  At D = 32 and 64 (16-bit), and at
D = 128 on grids of at least as many 256-row workgroups as CUs, the dQ
kernel computes them from the fragments it holds; at D = 256, on smaller
D = 128 grids and for fp32 a separate kernel does.  Dense shapes with ragged
row tails and several 256-row tiles, causal and not, and packed sequences
with empty query sets and sequences without keys (LSE = -inf, delta = 0),
each at D = 128 also on a grid large enough for the dQ kernel's own
statistics (384 and 640 workgroups of 256 rows).

Tolerance: LSE log2(e) is one fp32 product (relative 2^-23 of |LSE log2 e|
plus the rounding of log2 e itself: 2e-7 relative is ample); delta sums D
products of exactly representable 16-bit (or fp32) values in fp32, whose
error is below D 2^-24 sum_d |dO O| (1e-5 of that sum, plus 1e-7, bounds it
with room at D <= 256)."""
import numpy as np
import pytest

import workloads
from parity_util import log, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _check(ws, lse, o, do, tag):
    rows = lse.size
    l2 = ws[:rows].astype(np.float64)
    dl = ws[rows:2 * rows].astype(np.float64)
    ref_l2 = lse.astype(np.float64) * LOG2E
    prod = o.astype(np.float64) * do.astype(np.float64)
    ref_dl = prod.sum(-1)
    bound = 1e-5 * np.abs(prod).sum(-1) + 1e-7
    fin = np.isfinite(ref_l2)
    assert np.array_equal(np.isfinite(l2), fin), f"{tag}: -inf rows differ"
    assert np.all(l2[~fin] == ref_l2[~fin])
    el = float(np.max(np.abs(l2[fin] - ref_l2[fin]) / np.maximum(np.abs(ref_l2[fin]), 1.0))) if fin.any() else 0.0
    ed = float(np.max(np.abs(dl - ref_dl) - bound))
    log(f"  {tag}: rows {rows} max rel |dLSE2| {el:.2e}, max |d delta| - bound {ed:.2e}")
    assert el <= 2e-7, tag
    assert ed <= 0.0, tag


DENSE = [(dt, D) for dt in ("bf16", "fp16", "fp32") for D in (32, 64, 128, 256) if not (dt == "fp32" and D == 256)]


@pytest.mark.parametrize("dt,D", DENSE)
@pytest.mark.parametrize("causal", [False, True])
def test_backward_statistics_dense(dt, D, causal):
    import exact_tiled_attention_15_amd as fa

    w = workloads.Workload(f"stats_{dt}_d{D}", 2, 3, 520, 300, D, dt, causal, 700 + D)
    log(f"case statistics {w.name} causal={causal} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk}")
    q, k, v = to_gpu(workloads.make_inputs(w))
    o, lse = fa.forward(q, k, v, causal)
    do = workloads.make_dout(w).to(q.device)
    ws = torch.full((2 * w.B * w.H * w.Nq,), float("nan"), dtype=torch.float32, device=q.device)
    fa.backward(q, k, v, o, lse, do, causal, workspace=ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().reshape(-1, D)
    _check(ws.cpu().numpy(), lse.cpu().numpy().reshape(-1), f(o), f(do), w.name)


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
def test_backward_statistics_dense_full_grid(dt, causal):
    import exact_tiled_attention_15_amd as fa

    w = workloads.Workload(f"stats_{dt}_d128_h128", 1, 128, 520, 300, 128, dt, causal, 1700)
    log(f"case statistics {w.name} causal={causal} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk}")
    q, k, v = to_gpu(workloads.make_inputs(w))
    o, lse = fa.forward(q, k, v, causal)
    do = workloads.make_dout(w).to(q.device)
    ws = torch.full((2 * w.B * w.H * w.Nq,), float("nan"), dtype=torch.float32, device=q.device)
    fa.backward(q, k, v, o, lse, do, causal, workspace=ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().reshape(-1, 128)
    _check(ws.cpu().numpy(), lse.cpu().numpy().reshape(-1), f(o), f(do), w.name)


@pytest.mark.parametrize("dt,D,H", [("bf16", 128, 2), ("bf16", 128, 64), ("fp16", 64, 2), ("bf16", 256, 2),
                                    ("fp32", 64, 2)])
def test_backward_statistics_varlen(dt, D, H):
    import exact_tiled_attention_15_amd as fa

    lens_q, lens_k = [40, 0, 300, 3, 257], [0, 50, 200, 600, 129]
    w = workloads.VarlenWorkload("stats_v", H, D, dt, True, 900 + D, tuple(lens_q), tuple(lens_k))
    log(f"case statistics varlen {dt} D={D} H={H} lens_q={lens_q} lens_k={lens_k}")
    q, k, v, cu_q, cu_k = (t.to("cuda:0") for t in workloads.make_varlen_inputs(w))
    o, lse = fa.forward_varlen(q, k, v, cu_q, cu_k, max(lens_q), True)
    do = torch.randn(q.shape, generator=torch.Generator().manual_seed(5), dtype=torch.float32).to(q.dtype).to(q.device)
    ws = torch.full((2 * q.shape[0] * q.shape[1],), float("nan"), dtype=torch.float32, device=q.device)
    fa.backward_varlen(q, k, v, o, lse, do, cu_q, cu_k, max(lens_q), max(lens_k), True, workspace=ws)
    torch.cuda.synchronize()
    f = lambda t: t.float().cpu().numpy().reshape(-1, D)
    _check(ws.cpu().numpy(), lse.cpu().numpy().reshape(-1), f(o), f(do), f"varlen {dt} D={D} H={H}")
