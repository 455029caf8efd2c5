"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
identical seeded inputs, element by element at oracle-friendly sizes and on
sampled rows at the full workload sizes."""
import numpy as np
import pytest

import workloads
from parity_util import TOL, compare_full, compare_sampled, log, run_gpu, sample_rows, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _case(w, seed=None):
    log(f"case {w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} D={w.D} {w.dtype} causal={w.causal}")
    cpu = workloads.make_inputs(w, seed)
    return cpu, to_gpu(cpu)


@pytest.mark.parametrize("name", ["c1_fp32_causal_b2h4n128d64", "c2_fp32_b1h8n1024d64",
                                  "c1t_fp32_causal_b1h2q77k131d64", "c1t_fp32_b1h2q77k131d64",
                                  "c3t_bf16_causal_b1h3n1000d128"])
def test_parity_full(name):
    w = W[name]
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "full")


def test_parity_p1_worked_example_inputs():
    # the first page's own Step 2 inputs (legacy seed 0, randn), causal, fp32
    w = W["c1_fp32_causal_b2h4n128d64"]
    cpu = workloads.make_p1_legacy_inputs()
    o, l = run_gpu(*to_gpu(cpu), True)
    compare_full(w, cpu, o, l, "p1-inputs")


SMALL = [(dt, D, causal, Nq, Nk)
         for dt in ("bf16", "fp16", "fp32")
         for D in (32, 64, 128)
         for causal in (False, True)
         for (Nq, Nk) in ((300, 300), (257, 517), (130, 70))]


@pytest.mark.parametrize("dt,D,causal,Nq,Nk", SMALL)
def test_parity_small_grid(dt, D, causal, Nq, Nk):
    w = workloads.Workload(f"grid_{dt}_d{D}_{'c' if causal else 'n'}_{Nq}x{Nk}", 2, 3, Nq, Nk, D, dt,
                           causal, 77 + Nq + D)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "grid")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 3, 300, 700), (2, 2, 1, 129), (1, 256, 130, 300)])
def test_parity_fp32_grid_sizes(D, causal, B, H, Nq, Nk):
    # The fp32 forward picks its workgroup shape from the grid: with at most
    # as many 128-row workgroups as the 256 CUs (B*H*ceil(Nq/128) <= 256: the
    # first two shapes) 32-row workgroups split each 128-key tile over their
    # four waves and merge the waves' partial results at the end; otherwise
    # (the third shape, 512 workgroups) each wave owns 32 rows of a 128-row
    # tile.  Both with ragged Q and K tails.
    w = workloads.Workload(f"fp32grid_d{D}_{'c' if causal else 'n'}_b{B}h{H}_{Nq}x{Nk}", B, H, Nq, Nk, D, "fp32",
                           causal, 3200 + D + Nq)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "fp32-grid")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("B,H,Nq,Nk", [(1, 3, 300, 700), (1, 256, 130, 300), (1, 2, 40, 300), (1, 4, 129, 33),
                                       (1, 2, 300, 100), (1, 3, 1, 17)])
def test_parity_16bit_grid_sizes(dt, D, causal, B, H, Nq, Nk):
    # The 16-bit forward picks its workgroup from the grid: with fewer
    # 256-row (8-wave) workgroups than the 256 CUs (B*H*ceil(Nq/256) < 256,
    # every shape but the second) it runs 128-row workgroups, of score and
    # PV waves at D >= 64 and of 4 waves with pipelined steps at D = 32; the
    # second shape (256 workgroups) runs 256-row ones (16 score and PV waves
    # at D = 128, 8 waves below).  All compared
    # element by element, with ragged Q and K tails; Nq = 40 leaves row
    # groups without rows, Nk = 33 and 17 a ragged or lone partial key tile,
    # 300 x 100 (causal) rows that see every key.
    w = workloads.Workload(f"g16_{dt}_d{D}_{'c' if causal else 'n'}_h{H}_{Nq}x{Nk}", B, H, Nq, Nk, D, dt, causal,
                           1600 + D + Nq)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "16bit-grid")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(40, 17), (257, 33), (300, 100)])
def test_parity_d128_full_grid_edges(dt, causal, Nq, Nk):
    # D = 128 on a grid that fills the CUs (300 heads): the 16-wave role
    # split with row groups that hold no row (Nq = 40: six of eight), a lone
    # or ragged partial key tile, a one-row second Q tile (257), and causal
    # rows that see every key (300 x 100).
    w = workloads.Workload(f"rs16_{dt}_{'c' if causal else 'n'}_{Nq}x{Nk}", 1, 300, Nq, Nk, 128, dt, causal,
                           9100 + Nq + Nk)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "rs16")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_parity_8wave_several_q_tiles(dt, D, causal):
    # The 256-row workgroups (16-wave role split at D = 128, 8-wave fa_fwd_16
    # below) at a grid of more workgroups than CUs (128 heads x 3 Q tiles =
    # 384), with several Q tiles per head (causal
    # diagonals at q0 > 0, running maxima rescaled mid-stream), a ragged Q
    # tile (520 = 2 x 256 + 8 rows) and a ragged key tail (700 = 10 x 64 +
    # 60), every element compared.
    w = workloads.Workload(f"w8_{dt}_d{D}_{'c' if causal else 'n'}_h128_520x700", 1, 128, 520, 700, D, dt,
                           causal, 8800 + D)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "8wave")


@pytest.mark.parametrize("dt", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(300, 300), (257, 517), (130, 70), (1, 200), (40, 300), (129, 33),
                                   (300, 100), (64, 17)])
def test_parity_d256(dt, causal, Nq, Nk):
    # head dimension 256: 128-row workgroups of score and PV waves (one pair
    # per 32 rows), 32-key tiles.  Nq = 40 leaves two row groups with no row
    # at all, 129 a workgroup with one row; Nk = 33 and 17 give a ragged or
    # lone partial key tile; 300 x 100 under the causal mask has rows that see
    # every key.
    w = workloads.Workload(f"d256_{dt}_{'c' if causal else 'n'}_{Nq}x{Nk}", 2, 2, Nq, Nk, 256, dt, causal,
                           2560 + Nq + Nk)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "d256")


@pytest.mark.parametrize("dt,causal", [("bf16", True), ("fp16", False)])
def test_parity_d256_many_workgroups(dt, causal):
    # More 128-row workgroups than CUs (96 heads x 3 = 288): CUs run
    # workgroups back to back, every element compared.
    w = workloads.Workload(f"d256_many_{dt}", 1, 96, 300, 333, 256, dt, causal, 2600)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_full(w, cpu, o, l, "d256-many")


def test_parity_d256_scaled_and_moves():
    w = workloads.Workload("d256_scaled", 1, 2, 333, 401, 256, "bf16", True, 256)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, True, softmax_scale=0.04)
    compare_full(w, cpu, o, l, "d256-scaled", scale=0.04)


@pytest.mark.parametrize("H", [2, 128])
@pytest.mark.parametrize("dt,D,causal", [("bf16", 128, True), ("bf16", 128, False), ("fp16", 64, True),
                                         ("fp16", 128, False), ("fp32", 64, True), ("bf16", 256, True)])
def test_parity_reference_moves(dt, D, causal, H):
    # Keys whose norm grows along the sequence (K row j scaled by
    # 1 + a j/Nk, Q by a): each row's running max climbs tile after tile, so
    # the softmax reference moves mid-stream (about one move per row for
    # a = 3) and every rescale path of the kernel (l and O, with PV work in
    # flight) is exercised.  fp32 takes a = 2 (|LSE| up to ~22 rather than
    # ~44): its absolute LSE tolerance of 1e-5 is a few fp32 ulps of such
    # values, below what the rounding of larger scores allows.  H = 2 runs
    # the small-grid workgroup forms (role-split 16-bit, key-split fp32),
    # H = 128 the large-grid ones (8-wave 16-bit at D <= 128, 128-row fp32).
    w = workloads.Workload(f"moves_{dt}_d{D}_{'c' if causal else 'n'}_h{H}", 1, H, 700, 700, D, dt, causal,
                           4242 + D)
    q64, k64, v64 = workloads.draw_float64(w)
    a = 2.0 if dt == "fp32" else 3.0
    ramp = 1.0 + a * np.arange(w.Nk, dtype=np.float64) / w.Nk
    q64 = q64 * a
    k64 = k64 * ramp[None, None, :, None]
    cpu = tuple(workloads.round_to_dtype(x, dt) for x in (q64, k64, v64))
    log(f"case {w.name} (growing key norms)")
    o, l = run_gpu(*to_gpu(cpu), causal)
    compare_full(w, cpu, o, l, "moves")


@pytest.mark.parametrize("dt,D,causal,scale", [
    ("bf16", 128, True, 0.03), ("bf16", 64, False, 0.5), ("fp16", 32, True, 1.0),
    ("fp16", 128, False, 0.2), ("fp32", 32, False, 0.4), ("fp32", 128, True, 0.05),
    ("bf16", 32, False, 1.0 / 32**0.5)])
def test_parity_explicit_scale(dt, D, causal, scale):
    # fa_fwd_scaled: s = scale * q.k, against the oracle at the same scale
    # (larger scales give peakier rows, small ones nearly uniform weights).
    w = workloads.Workload(f"scaled_{dt}_d{D}_{'c' if causal else 'n'}_{scale:.3g}", 2, 2, 333, 401, D, dt,
                           causal, 5150 + D)
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal, softmax_scale=scale)
    compare_full(w, cpu, o, l, "scaled", scale=scale)


def test_default_scale_matches_explicit():
    # fa_fwd and fa_fwd_scaled(1/sqrt(D)) run the same kernel with the same
    # fp32 factor: identical bits.
    for dt, D in (("bf16", 128), ("fp16", 32), ("fp32", 64)):
        w = workloads.Workload(f"dflt_{dt}_d{D}", 1, 2, 200, 260, D, dt, True, 61 + D)
        cpu, gpu = _case(w)
        o1, l1 = run_gpu(*gpu, True)
        o2, l2 = run_gpu(*gpu, True, softmax_scale=1.0 / D**0.5)
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["c3_bf16_causal_b4h16n4096d128",
                                  "c4_bf16_causal_b1h32n16384d128_q4",
                                  "c5_fp16_cross_b8h32q512k8192d64",
                                  "x1_bf16_causal_b4h8n4096d256",
                                  "c5t_fp16_cross_b8h32q511k8191d64"])
def test_parity_full_size_sampled(name):
    w = W[name]
    cpu, gpu = _case(w)
    o, l = run_gpu(*gpu, w.causal)
    compare_sampled(w, cpu, o, l, sample_rows(w), "sampled")
    # a property that holds at any size: O is a convex combination of V rows
    vmax = gpu[2].float().abs().amax(dim=(2, 3))
    assert bool((o.float().abs().amax(dim=(2, 3)) <= vmax + TOL[w.dtype][0]).all())


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 64), ("fp32", 64), ("bf16", 32), ("fp32", 32)])
def test_edge_shapes(dt, D):
    for (Nq, Nk, causal) in ((1, 1, False), (1, 1, True), (1, 4099, False), (3, 1, True),
                             (200, 5, True), (5, 200, True), (129, 129, True), (64, 64, False)):
        w = workloads.Workload(f"edge_{dt}_{Nq}x{Nk}", 1, 2, Nq, Nk, D, dt, causal, Nq * 7 + Nk)
        cpu, gpu = _case(w)
        o, l = run_gpu(*gpu, causal)
        compare_full(w, cpu, o, l, "edge")


def test_empty_batch_is_noop():
    import exact_tiled_attention_15_amd as fa

    q = torch.empty(0, 2, 16, 64, device="cuda:0", dtype=torch.bfloat16)
    o, l = fa.forward(q, q, q, True)
    assert o.shape == (0, 2, 16, 64) and l.shape == (0, 2, 16)


@pytest.mark.parametrize("name", ["c3t_bf16_causal_b1h3n1000d128", "c2_fp32_b1h8n1024d64"])
def test_deterministic(name):
    w = W[name]
    _, gpu = _case(w)
    o1, l1 = run_gpu(*gpu, w.causal)
    o2, l2 = run_gpu(*gpu, w.causal)
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "run-to-run results differ"


@pytest.mark.parametrize("dt", ["bf16", "fp16", "fp32"])
def test_gpu_invariants(dt):
    w = workloads.Workload("inv", 1, 2, 300, 300, 128 if dt != "fp32" else 64, dt, True, 9)
    cpu, gpu = _case(w)
    q, k, v = gpu
    # causal row 0 sees only key 0: O = V[0] exactly (weight 1), LSE = s00
    o, l = run_gpu(q, k, v, True)
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) / np.sqrt(w.D)
    assert float((l[:, :, 0].double() - s00).abs().max()) <= TOL[dt][1]
    # constant V -> constant O
    c = torch.linspace(-2, 3, w.D, device=q.device).to(q.dtype)
    vc = c.expand_as(v).contiguous()
    o, _ = run_gpu(q, k, vc, False)
    assert float((o.float() - c.float()).abs().max()) <= TOL[dt][0]


@pytest.mark.parametrize("path", ["fwd", "splitkv"])
def test_max_size_closed_forms(path):
    # Nk just below the 32-bit per-head offset limit ((Nk + 256) D 2 < 2^31 at
    # D = 128): the oracle would need tens of GB of float64, so use the closed
    # forms that hold at any size: Q = 0 gives uniform weights, O = mean of V
    # over the keys and LSE = ln Nk.
    import exact_tiled_attention_15_amd as fa

    Nk = (2**31 - 1) // 256 - 256 - 1000
    Nq = 100 if path == "fwd" else 8
    D = 128
    log(f"case max-size {path}: Nq={Nq} Nk={Nk} D={D} bf16, Q = 0")
    gen = torch.Generator(device="cuda:0").manual_seed(31)
    q = torch.zeros(1, 1, Nq, D, device="cuda:0", dtype=torch.bfloat16)
    k = torch.randn(1, 1, Nk, D, device="cuda:0", dtype=torch.bfloat16, generator=gen)
    v = torch.randn(1, 1, Nk, D, device="cuda:0", dtype=torch.bfloat16, generator=gen)
    if path == "fwd":
        o, l = fa.forward(q, k, v, False)
    else:
        o, l = fa.forward_splitkv(q, k, v, False)
    torch.cuda.synchronize()
    mean = v[0, 0].double().mean(dim=0)
    eo = float((o[0, 0].double() - mean).abs().max())
    el = float((l.double() - np.log(Nk)).abs().max())
    log(f"  max|O - mean V|={eo:.3e} max|LSE - ln Nk|={el:.3e}")
    assert bool(torch.isfinite(o).all())
    assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1]
    del k, v
    torch.cuda.empty_cache()
