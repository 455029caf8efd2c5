"""GPU parity of the packed variable-length forward (fa_fwd_varlen) against
the float64 varlen oracle: every row of every sequence, including empty
sequences, sequences without keys (O = 0, LSE = -inf) and lengths around the
64-key and 256-row tile edges."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import TOL, log

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _run(q, k, v, cu_q, cu_k, causal, scale=None, max_q=None):
    import exact_tiled_attention_15_amd as fa

    dev = "cuda:0"
    qg, kg, vg = (t.to(dev).contiguous() for t in (q, k, v))
    cq, ck = cu_q.to(dev), cu_k.to(dev)
    max_q = int((cu_q[1:] - cu_q[:-1]).max()) if max_q is None else max_q
    o = torch.full_like(qg, float("nan"))
    lse = torch.full(qg.shape[:2], float("nan"), device=dev)
    fa.forward_varlen(qg, kg, vg, cq, ck, max_q, causal, softmax_scale=scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return o, lse


def _compare(dt, inputs, o, lse, causal, tag, scale=None):
    q, k, v, cu_q, cu_k = inputs
    O, L = oracle.attention_varlen(q, k, v, cu_q.numpy(), cu_k.numpy(), causal, scale=scale)
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    assert not np.isnan(og).any() and not np.isnan(lg).any(), f"{tag}: rows left unwritten"
    fin = np.isfinite(L)
    assert np.array_equal(np.isfinite(lg), fin), f"{tag}: -inf rows differ"
    assert np.all(og[~fin] == 0.0)
    eo = float(np.max(np.abs(og - O)))
    el = float(np.max(np.abs(lg[fin] - L[fin]))) if fin.any() else 0.0
    to, tl = TOL[dt]
    log(f"  {tag}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= to and el <= tl


def _inputs(dt, H, D, lens_q, lens_k, seed):
    w = workloads.VarlenWorkload("t", H, D, dt, False, seed, tuple(lens_q), tuple(lens_k))
    return workloads.make_varlen_inputs(w)


LENS = [
    ([1, 64, 65, 255, 256, 257, 700], [1, 64, 65, 255, 256, 257, 700]),      # self-attention, tile edges
    ([0, 300, 5, 0, 129], [10, 200, 600, 7, 129]),                          # empty query sets, Nq != Nk
    ([40, 3, 90], [0, 50, 0]),                                              # sequences without keys
]


GRID = [(dt, D) for dt in ("bf16", "fp16", "fp32") for D in (32, 64, 128, 256) if not (dt == "fp32" and D == 256)]


@pytest.mark.parametrize("dt,D", GRID)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("li", range(len(LENS)))
def test_varlen_parity(dt, D, causal, li):
    lens_q, lens_k = LENS[li]
    log(f"case varlen {dt} D={D} causal={causal} lens_q={lens_q} lens_k={lens_k}")
    inputs = _inputs(dt, 3, D, lens_q, lens_k, 100 + li + D)
    o, lse = _run(*inputs, causal)
    _compare(dt, inputs, o, lse, causal, f"varlen-{li}")


def test_varlen_explicit_scale_and_large_max():
    # an over-estimated max_seqlen_q only adds workgroups that exit
    inputs = _inputs("bf16", 2, 64, [33, 250], [77, 250], 7)
    o, lse = _run(*inputs, True, scale=0.2, max_q=283)
    _compare("bf16", inputs, o, lse, True, "varlen-scaled", scale=0.2)


@pytest.mark.parametrize("dt,H", [("bf16", 4), ("bf16", 96), ("fp32", 32)])
def test_varlen_equals_dense_for_equal_lengths(dt, H):
    # Equal lengths: bit for bit the dense forward's result.  The varlen
    # 16-bit kernel always runs 8-wave workgroups of 256 rows; the dense one
    # runs them too with H = 96 (3*96*ceil(300/256) = 576 workgroups, the
    # same tiles), and its role-split 128-row form (score and PV waves) on the
    # small grid of H = 4 (24 workgroups of 256 rows, fewer than the CUs):
    # the same arithmetic in the same order, so the same bits.  fp32 takes
    # enough heads (3*32*ceil(300/128) = 288 workgroups of 128 rows) that the
    # dense forward keeps its 128-row tiles: on grids of at most one
    # workgroup per CU it splits keys over the waves instead (another
    # addition order, equal only within the tolerance).
    import exact_tiled_attention_15_amd as fa

    B, N, D = 3, 300, 128
    inputs = _inputs(dt, H, D, [N] * B, [N] * B, 11)
    q, k, v = inputs[:3]
    o, lse = _run(*inputs, True)
    dense = [t.reshape(H, B, N, D).permute(1, 0, 2, 3).contiguous().cuda() for t in (q, k, v)]
    od, ld = fa.forward(*dense, True)
    od = od.permute(1, 0, 2, 3).reshape(H, B * N, D)
    ld = ld.permute(1, 0, 2).reshape(H, B * N)
    assert torch.equal(o, od) and torch.equal(lse, ld)


def test_varlen_full_size_sampled():
    w = workloads.VARLEN_WORKLOADS["v1_bf16_causal_varlen_b16h16d128"]
    log(f"case {w.name} (sampled rows)")
    q, k, v, cu_q, cu_k = workloads.make_varlen_inputs(w)
    o, lse = _run(q, k, v, cu_q, cu_k, w.causal)
    r = np.random.default_rng(5)
    for b in sorted(set([0, w.B - 1] + list(r.integers(0, w.B, 3)))):
        q0, q1, k0, k1 = (int(x) for x in (cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]))
        rows = sorted(set([0, q1 - q0 - 1, (q1 - q0) // 2] + list(r.integers(0, q1 - q0, 6))))
        for h in (0, w.H - 1):
            sel = [(0, 0, i) for i in rows]
            O, L = oracle.attention_rows(q[h][None, None, q0:q1], k[h][None, None, k0:k1],
                                         v[h][None, None, k0:k1], w.causal, sel)
            og = o[h, q0:q1][rows].float().cpu().double().numpy()
            lg = lse[h, q0:q1][rows].cpu().double().numpy()
            eo, el = float(np.max(np.abs(og - O))), float(np.max(np.abs(lg - L)))
            assert eo <= TOL["bf16"][0] and el <= TOL["bf16"][1], (b, h, eo, el)
    log("  sampled rows within tolerance")


# ---------------------------------------------------------------------------
# Backward over packed sequences (fa_bwd_varlen)
# ---------------------------------------------------------------------------
# Tolerance as the dense backward's (tests/test_backward_gpu.py): each
# gradient tensor within REL of its own largest magnitude, plus a floor.
BWD_TOL = {"bf16": (2e-2, 1e-4), "fp16": (2e-2, 1e-4), "fp32": (1e-4, 1e-6)}


def _dout(dt, like, seed):
    r = np.random.default_rng(seed)
    return torch.from_numpy(r.standard_normal(tuple(like.shape)).astype(np.float32)).to(like.dtype)


def _run_bwd(inputs, causal, dout, scale=None):
    import exact_tiled_attention_15_amd as fa

    q, k, v, cu_q, cu_k = inputs
    o, lse = _run(q, k, v, cu_q, cu_k, causal, scale=scale)
    dev = o.device
    qg, kg, vg = (t.to(dev).contiguous() for t in (q, k, v))
    cq, ck = cu_q.to(dev), cu_k.to(dev)
    max_q = int((cu_q[1:] - cu_q[:-1]).max())
    max_k = int((cu_k[1:] - cu_k[:-1]).max())
    grads = [torch.full_like(t, float("nan")) for t in (qg, kg, vg)]
    fa.backward_varlen(qg, kg, vg, o, lse, dout.to(dev), cq, ck, max_q, max_k, causal, softmax_scale=scale,
                       dq=grads[0], dk=grads[1], dv=grads[2])
    torch.cuda.synchronize()
    return grads


def _compare_bwd(dt, inputs, dout, grads, causal, tag, scale=None):
    q, k, v, cu_q, cu_k = inputs
    ref = oracle.attention_varlen_backward(q, k, v, dout, cu_q.numpy(), cu_k.numpy(), causal, scale=scale)
    rel, floor = BWD_TOL[dt]
    msg = []
    for name, g, r in zip(("dQ", "dK", "dV"), grads, ref):
        g = g.float().cpu().double().numpy()
        assert np.isfinite(g).all(), f"{tag} {name}: rows left unwritten or non-finite"
        e = float(np.max(np.abs(g - r))) if r.size else 0.0
        m = float(np.max(np.abs(r))) if r.size else 0.0
        msg.append(f"{name} err {e:.2e} max {m:.2e}")
        assert e <= rel * m + floor, f"{tag} {name}: {e:.3e} > {rel} * {m:.3e} + {floor}"
    log(f"  {tag}: " + " ".join(msg))


@pytest.mark.parametrize("dt,D", GRID)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("li", range(len(LENS)))
def test_varlen_backward_parity(dt, D, causal, li):
    lens_q, lens_k = LENS[li]
    log(f"case varlen backward {dt} D={D} causal={causal} lens_q={lens_q} lens_k={lens_k}")
    inputs = _inputs(dt, 2, D, lens_q, lens_k, 200 + li + D)
    dout = _dout(dt, inputs[0], 300 + li + D)
    grads = _run_bwd(inputs, causal, dout)
    _compare_bwd(dt, inputs, dout, grads, causal, f"varlen-bwd-{li}")


def test_varlen_backward_explicit_scale():
    inputs = _inputs("fp16", 2, 128, [33, 250, 1], [77, 250, 9], 17)
    dout = _dout("fp16", inputs[0], 18)
    grads = _run_bwd(inputs, True, dout, scale=0.2)
    _compare_bwd("fp16", inputs, dout, grads, True, "varlen-bwd-scaled", scale=0.2)


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_varlen_backward_equals_dense_for_equal_lengths(dt):
    # equal lengths: the same tiles as the dense backward, bit for bit (fp32
    # with 32 heads, so that the dense kernels keep their 128-row tiles, as
    # in the forward test above)
    import exact_tiled_attention_15_amd as fa

    B, H, N, D = 3, 4 if dt != "fp32" else 32, 300, 128
    inputs = _inputs(dt, H, D, [N] * B, [N] * B, 21)
    dout = _dout(dt, inputs[0], 22)
    grads = _run_bwd(inputs, True, dout)
    q, k, v = inputs[:3]
    dense = [t.reshape(H, B, N, D).permute(1, 0, 2, 3).contiguous().cuda() for t in (q, k, v, dout)]
    o, lse = fa.forward(*dense[:3], True)
    gd = fa.backward(*dense[:3], o, lse, dense[3], True)
    for g, d in zip(grads, gd):
        assert torch.equal(g, d.permute(1, 0, 2, 3).reshape(H, B * N, D))
