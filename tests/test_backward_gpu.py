"""GPU parity of the backward pass: fa_bwd (through the C ABI) against the
float64 backward oracle on the same seeded inputs.  The GPU backward takes
the GPU forward's O and LSE, as a training step would.

Tolerance (16-bit inputs): the gradients have no fixed scale (dV entries shrink like 1/N
for spread-out softmax rows), so the error of each gradient tensor is taken
relative to its largest magnitude: max|G_gpu - G| <= 2e-2 * max|G|, the
forward's 16-bit bound on O (whose entries are O(1)) applied to the
gradient's own scale, plus an absolute 1e-4 for gradients that vanish
exactly (a row with a single key has dQ = dK = 0 up to rounding).  Its budget: P and dS enter the MFMAs rounded to 16
bits (relative 2^-9 for bf16), delta comes from the 16-bit O, and the
results are rounded to 16 bits.  fp32 inputs: nothing is rounded below
fp32 and every product accumulates in fp32 (relative error of order
2^-24 sqrt(N) per dot product, ~1e-6 here), and the forward's O and LSE it
starts from are within 1e-4 / 1e-5 of exact; 1e-4 of max|G| (plus 1e-6
absolute) bounds the result with room."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import log, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_TOL = 2e-2
ABS_FLOOR = 1e-4
REL_TOL_FP32 = 1e-4
ABS_FLOOR_FP32 = 1e-6


def _bound(m, dtype="bf16"):
    if dtype == "fp32":
        return REL_TOL_FP32 * m + ABS_FLOOR_FP32
    return REL_TOL * m + ABS_FLOOR


def _run(w, scale=None, cpu=None, dout=None):
    import exact_tiled_attention_15_amd as fa

    cpu = cpu if cpu is not None else workloads.make_inputs(w)
    dout = dout if dout is not None else workloads.make_dout(w)
    q, k, v = to_gpu(cpu)
    do = dout.to("cuda:0")
    o, lse = fa.forward(q, k, v, w.causal, softmax_scale=scale)
    grads = [torch.full_like(t, float("nan")) for t in (q, k, v)]
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, w.causal, softmax_scale=scale, dq=grads[0], dk=grads[1],
                             dv=grads[2])
    torch.cuda.synchronize()
    return cpu, dout, (dq, dk, dv)


def _compare(w, cpu, dout, grads, scale=None, tag=""):
    ref = oracle.attention_backward(*cpu, dout, w.causal, scale=scale)
    errs = []
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        g = g.float().cpu().double().numpy()
        assert np.isfinite(g).all(), f"{tag} {name}: non-finite values"
        e = float(np.max(np.abs(g - r)))
        m = float(np.max(np.abs(r)))
        errs.append((name, e, m))
        assert e <= _bound(m, w.dtype), f"{tag} {name}: max err {e:.3e} > bound {_bound(m, w.dtype):.3e}"
    log(f"  {tag} {w.name}: " + " ".join(f"{n} err {e:.2e} max {m:.2e}" for n, e, m in errs))


GRID = [(dt, D, causal, Nq, Nk)
        for dt in ("bf16", "fp16", "fp32")
        for D in (32, 64, 128, 256) if not (dt == "fp32" and D == 256)
        for causal in (False, True)
        for (Nq, Nk) in ((300, 300), (257, 517), (130, 70))]


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 3, 300, 700), (1, 256, 130, 300), (1, 128, 100, 300),
                                       (1, 128, 300, 100)])
def test_backward_fp32_grid_sizes(D, causal, B, H, Nq, Nk):
    # Each fp32 backward kernel picks its workgroup shape from its own grid:
    # with at most one 128-row workgroup per CU (B*H*ceil(N/128) <= 256, N =
    # Nq for dQ, Nk for dK/dV) it runs 32-row workgroups whose four waves
    # split the streamed keys (dQ) or queries (dK/dV, D <= 64) and sum their
    # partial gradients at the end.  The shapes cover: both split, neither
    # split, only dQ split, only dK/dV split; with ragged tails.
    w = workloads.Workload(f"bwd32grid_d{D}_{'c' if causal else 'n'}_h{H}_{Nq}x{Nk}", B, H, Nq, Nk, D, "fp32",
                           causal, 900 + D + Nq + Nk)
    log(f"case {w.name}")
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag="fp32-grid")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 128, 520, 300), (1, 64, 300, 520)])
def test_backward_16bit_dq_grid_sizes(dt, causal, B, H, Nq, Nk):
    # At D = 128 the dQ kernel depends on the grid: with at least as many
    # 256-row workgroups as CUs (B*H*ceil(Nq/256) = 384 here) the 256-row
    # kernel that computes the row statistics itself, otherwise (128) the
    # 128-row role-split kernel after the statistics kernel.  Ragged tails.
    w = workloads.Workload(f"bwd16grid_{dt}_{'c' if causal else 'n'}_h{H}_{Nq}x{Nk}", B, H, Nq, Nk, 128, dt, causal,
                           1300 + H + Nq)
    log(f"case {w.name}")
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag="16bit-grid")


@pytest.mark.parametrize("dt,D,causal,Nq,Nk", GRID)
def test_backward_parity_grid(dt, D, causal, Nq, Nk):
    w = workloads.Workload(f"bwd_{dt}_d{D}_{'c' if causal else 'n'}_{Nq}x{Nk}", 2, 3, Nq, Nk, D, dt, causal,
                           300 + Nq + Nk + D)
    log(f"case {w.name}")
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag="grid")


@pytest.mark.parametrize("dt,D,causal,scale", [("bf16", 128, True, 0.05), ("fp16", 64, False, 0.4),
                                               ("bf16", 32, True, 1.0), ("fp16", 256, True, 0.3),
                                               ("fp32", 128, True, 0.2)])
def test_backward_explicit_scale(dt, D, causal, scale):
    w = workloads.Workload(f"bwd_scaled_{dt}_d{D}", 1, 2, 200, 333, D, dt, causal, 71 + D)
    log(f"case {w.name} scale={scale}")
    cpu, dout, grads = _run(w, scale=scale)
    _compare(w, cpu, dout, grads, scale=scale, tag="scaled")


EDGE = [("bf16", Nq, Nk, c) for (Nq, Nk, c) in ((1, 1, True), (1, 300, False), (5, 200, True), (200, 5, True),
                                                 (64, 64, False), (65, 129, True), (0, 70, False))]
EDGE += [("fp32", Nq, Nk, c) for (Nq, Nk, c) in ((1, 1, True), (5, 200, True), (200, 5, True), (0, 70, False))]


@pytest.mark.parametrize("dt,Nq,Nk,causal", EDGE)
def test_backward_edge_shapes(dt, Nq, Nk, causal):
    w = workloads.Workload(f"bwd_edge_{dt}_{Nq}x{Nk}", 1, 2, Nq, Nk, 64, dt, causal, Nq * 3 + Nk)
    log(f"case {w.name} causal={causal}")
    if Nq == 0:
        import exact_tiled_attention_15_amd as fa

        cpu = workloads.make_inputs(w)
        q, k, v = to_gpu(cpu)
        o = torch.empty_like(q)
        lse = torch.empty((1, 2, 0), device="cuda:0")
        dk = torch.full_like(k, float("nan"))
        dv = torch.full_like(v, float("nan"))
        fa.backward(q, k, v, o, lse, torch.empty_like(q), causal, dk=dk, dv=dv)
        torch.cuda.synchronize()
        assert float(dk.abs().max()) == 0.0 and float(dv.abs().max()) == 0.0
        return
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag="edge")


# D = 128 and 256 run the two-wave-per-SIMD dK/dV kernel (a P wave and a dS
# wave per 32-key group): shapes with fewer keys than one 128-key block, a
# partial last key group, tiny and ragged query tails, both mask modes.
EDGE2 = [(dt, D, Nq, Nk, c) for dt in ("bf16", "fp16") for D in (128, 256)
         for (Nq, Nk, c) in ((1, 1, True), (1, 33, False), (5, 200, True), (200, 5, True), (64, 64, False),
                             (65, 129, True), (300, 161, False), (130, 97, True), (33, 300, True))]


@pytest.mark.parametrize("dt,D,Nq,Nk,causal", EDGE2)
def test_backward_edge_shapes_two_role(dt, D, Nq, Nk, causal):
    # the two-role dK/dV kernel (D = 128: 64-row Q/dO tiles; D = 256: 32-row
    # tiles): fewer keys than one 128-key block, a partial last key group,
    # tiny and ragged query tails (33 rows: one row past a 32-row tile)
    w = workloads.Workload(f"bwd_edge{D}_{dt}_{Nq}x{Nk}", 1, 3, Nq, Nk, D, dt, causal, Nq * 5 + Nk + D)
    log(f"case {w.name} causal={causal}")
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag=f"edge{D}")


@pytest.mark.parametrize("name", ["c1_fp32_causal_b2h4n128d64", "c2_fp32_b1h8n1024d64"])
def test_backward_fp32_workloads(name):
    # the fp32 workloads at their full sizes, every element compared
    w = workloads.WORKLOADS[name]
    log(f"case {w.name} (backward)")
    cpu, dout, grads = _run(w)
    _compare(w, cpu, dout, grads, tag="fp32")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_backward_unseen_keys_are_zero(dt):
    # causal, Nk > Nq: keys past the last query get exactly zero gradients
    w = workloads.Workload(f"bwd_unseen_{dt}", 1, 2, 100, 400, 128, dt, True, 17)
    cpu, dout, (dq, dk, dv) = _run(w)
    assert float(dk[:, :, 100:].abs().max()) == 0.0
    assert float(dv[:, :, 100:].abs().max()) == 0.0
    _compare(w, cpu, dout, (dq, dk, dv), tag="unseen")


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_backward_deterministic(dt):
    w = workloads.Workload(f"bwd_det_{dt}", 1, 4, 700, 700, 128, dt, True, 23)
    cpu, dout, g1 = _run(w)
    _, _, g2 = _run(w, cpu=cpu, dout=dout)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b), "run-to-run backward results differ"


@pytest.mark.parametrize("name", ["c3_bf16_causal_b4h16n4096d128", "c5_fp16_cross_b8h32q512k8192d64",
                                  "x1_bf16_causal_b4h8n4096d256"])
def test_backward_full_size_sampled_heads(name):
    # the measured shapes, checked on whole (b, h) heads the oracle can afford
    w = workloads.WORKLOADS[name]
    log(f"case {w.name} (backward, sampled heads)")
    cpu, dout, grads = _run(w)
    BH = w.B * w.H
    for bh in (0, BH - 1):
        b, h = divmod(bh, w.H)
        sub = tuple(t[b:b + 1, h:h + 1] for t in cpu)
        ref = oracle.attention_backward(*sub, dout[b:b + 1, h:h + 1], w.causal)
        for name_, g, r in zip(("dQ", "dK", "dV"), grads, ref):
            gg = g[b:b + 1, h:h + 1].float().cpu().double().numpy()
            assert np.isfinite(gg).all()
            e = float(np.max(np.abs(gg - r)))
            m = float(np.max(np.abs(r)))
            log(f"  head {bh} {name_}: err {e:.2e} / max {m:.2e}")
            assert e <= _bound(m, w.dtype)
