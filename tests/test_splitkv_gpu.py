"""GPU parity of the split-KV forward (fa_fwd_splitkv): the merged result
against the float64 oracle (the plain definition: splitting the keys must not
change it) at the forward's tolerances, and the per-range fp32 partials in
the workspace against the oracle's partial over the same key range."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL, compare_full, compare_sampled, log, sample_rows, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

CASES = []
for i, (dt, D, causal, Nq, Nk) in enumerate([
        (dt, D, causal, Nq, Nk)
        for dt in ("bf16", "fp16")
        for D in (32, 64, 128)
        for causal in (False, True)
        for (Nq, Nk) in ((1, 4097), (16, 3000), (33, 700), (300, 1500))]):
    CASES.append((dt, D, causal, Nq, Nk, (0, 3, 7, 40)[i % 4]))
CASES += [("bf16", 256, False, 1, 5000, 0), ("fp16", 256, True, 40, 900, 3)]
# fp32 inputs (the fp32 kernel in split mode, fp32 output from the merge)
for i, (D, causal, Nq, Nk) in enumerate([(D, causal, Nq, Nk) for D in (32, 64, 128) for causal in (False, True)
                                          for (Nq, Nk) in ((1, 4097), (33, 700), (300, 1500))]):
    CASES.append(("fp32", D, causal, Nq, Nk, (0, 3, 7)[i % 3]))


def _run(w, splits, scale=None):
    import exact_tiled_attention_15_amd as fa

    cpu = workloads.make_inputs(w)
    q, k, v = to_gpu(cpu)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.H, w.Nq), float("nan"), device=q.device)
    need = fa.fa_fwd_splitkv_workspace_size(w.B, w.H, w.Nq, w.Nk, w.D, splits)
    ws = torch.full((max(need, 16) // 4,), float("nan"), device=q.device)
    fa.forward_splitkv(q, k, v, w.causal, num_splits=splits, softmax_scale=scale, out=o, lse=lse, workspace=ws)
    torch.cuda.synchronize()
    return cpu, (q, k, v), o, lse, ws, need


@pytest.mark.parametrize("dt,D,causal,Nq,Nk,splits", CASES)
def test_splitkv_parity(dt, D, causal, Nq, Nk, splits):
    w = workloads.Workload(f"split_{dt}_d{D}_{'c' if causal else 'n'}_{Nq}x{Nk}_s{splits}", 2, 2, Nq, Nk, D, dt,
                           causal, 800 + Nq + Nk + D)
    log(f"case {w.name}")
    cpu, _, o, lse, _, _ = _run(w, splits)
    compare_full(w, cpu, o, lse, "splitkv")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_partials(causal, dt):
    # every range's fp32 partial (O_s, LSE_s), empty causal ranges included
    # 500 query rows: under the causal mask range 1 is seen in full by rows
    # >= 383, ranges 2 and 3 in part or not at all
    w = workloads.Workload(f"split_partials_{dt}_{'c' if causal else 'n'}", 1, 2, 500, 700, 64, dt, causal, 91)
    splits = 5  # 700 keys -> ranges of 192 keys: [0,192) [192,384) [384,576) [576,700)
    cpu, _, o, lse, ws, need = _run(w, splits)
    n, length = 4, 192
    rows = w.B * w.H * w.Nq
    assert need == n * rows * (w.D + 1) * 4
    wsn = ws.cpu().double().numpy()
    Po = wsn[:n * rows * w.D].reshape(n, w.B, w.H, w.Nq, w.D)
    Pl = wsn[n * rows * w.D:n * rows * (w.D + 1)].reshape(n, w.B, w.H, w.Nq)
    for s in range(n):
        k0, k1 = s * length, min((s + 1) * length, w.Nk)
        Or, Lr = oracle.attention_partial(*cpu, causal, k0, k1)
        empty = np.isinf(Lr)
        assert np.array_equal(np.isinf(Pl[s]), empty), f"range {s}: empty rows differ"
        assert np.all(Po[s][empty] == 0.0)
        eo = float(np.max(np.abs(Po[s] - Or)))
        el = float(np.max(np.abs(Pl[s][~empty] - Lr[~empty]))) if (~empty).any() else 0.0
        log(f"  range {s} [{k0},{k1}): max|dO_s|={eo:.2e} max|dLSE_s|={el:.2e} empty rows {int(empty.sum())}")
        assert eo <= TOL[dt][0] and el <= TOL[dt][1]
    compare_full(w, cpu, o, lse, "partials-merged")


def test_splitkv_matches_forward_closely():
    # same kernel per range, different summation grouping: close to fa_fwd
    import exact_tiled_attention_15_amd as fa

    w = workloads.Workload("split_vs_fwd", 2, 4, 8, 5000, 128, "bf16", False, 5)
    cpu, (q, k, v), o, lse, _, _ = _run(w, 0)
    o2, l2 = fa.forward(q, k, v, False)
    assert float((o.float() - o2.float()).abs().max()) <= 2 * TOL["bf16"][0]
    assert float((lse - l2).abs().max()) <= 2 * TOL["bf16"][1]


def test_splitkv_explicit_scale_and_single_range():
    w = workloads.Workload("split_scaled", 1, 3, 5, 900, 64, "fp16", True, 6)
    cpu, _, o, lse, _, need = _run(w, 4, scale=0.3)
    compare_full(w, cpu, o, lse, "split-scaled", scale=0.3)
    # fewer keys than one tile: one range, the plain forward, no workspace
    w = workloads.Workload("split_one", 1, 2, 3, 50, 128, "bf16", False, 7)
    cpu, _, o, lse, _, need = _run(w, 0)
    assert need == 0
    compare_full(w, cpu, o, lse, "split-one")


@pytest.mark.parametrize("name", ["d1_bf16_decode_b8h32q1k32768d128", "d2_bf16_decode_b1h32q16k65536d128"])
def test_splitkv_decode_full_size_sampled(name):
    w = workloads.WORKLOADS[name]
    log(f"case {w.name} (sampled rows)")
    cpu, _, o, lse, _, _ = _run(w, 0)
    compare_sampled(w, cpu, o, lse, sample_rows(w, n_heads=6, n_rand=8), "decode")
