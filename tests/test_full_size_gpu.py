"""Whole-tensor parity at the measured workloads' own sizes: every element of
O and LSE (and of dQ, dK, dV for the backward) compared with the float64
oracle on the same seeded inputs, as the pages' own sanity check compares the
whole output ("Building a FlashAttention-2 Forward Kernel in Pure NumPy",
Step 5).  The oracle runs head by head on the host (seconds to a minute)."""
import numpy as np
import pytest

import oracle
import workloads
from parity_util import _oracle_pool, compare_whole, log, run_gpu, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


@pytest.mark.parametrize("name", ["c3_bf16_causal_b4h16n4096d128",
                                  "c4_bf16_causal_b1h32n16384d128_q4",
                                  "c5_fp16_cross_b8h32q512k8192d64",
                                  "c5t_fp16_cross_b8h32q511k8191d64",
                                  "x1_bf16_causal_b4h8n4096d256"])
def test_forward_whole_tensors(name):
    w = W[name]
    log(f"case {w.name} whole tensors B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} D={w.D} {w.dtype} causal={w.causal}")
    cpu = workloads.make_inputs(w)
    o, l = run_gpu(*to_gpu(cpu), w.causal)
    compare_whole(w, cpu, o, l, "whole")


@pytest.mark.parametrize("name", ["d1_bf16_decode_b8h32q1k32768d128", "d2_bf16_decode_b1h32q16k65536d128"])
def test_splitkv_decode_whole_tensors(name):
    import exact_tiled_attention_15_amd as fa

    w = W[name]
    log(f"case {w.name} whole tensors (split-KV, automatic ranges)")
    cpu = workloads.make_inputs(w)
    q, k, v = to_gpu(cpu)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), device=q.device)
    fa.forward_splitkv(q, k, v, w.causal, 0, out=out, lse=lse)
    torch.cuda.synchronize()
    del k, v
    compare_whole(w, cpu, out, lse, "decode-whole")


def test_varlen_every_row():
    import exact_tiled_attention_15_amd as fa

    w = workloads.VARLEN_WORKLOADS["v1_bf16_causal_varlen_b16h16d128"]
    log(f"case {w.name} every row ({sum(w.lens_q)} tokens x {w.H} heads)")
    q, k, v, cu_q, cu_k = workloads.make_varlen_inputs(w)
    g = [t.to("cuda:0") for t in (q, k, v, cu_q, cu_k)]
    o = torch.full_like(g[0], float("nan"))
    lse = torch.full(g[0].shape[:2], float("nan"), device=g[0].device)
    fa.forward_varlen(*g, max(w.lens_q), w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    og = o.float().cpu().double().numpy()
    lg = lse.cpu().double().numpy()
    assert np.isfinite(og).all() and np.isfinite(lg).all()
    eo = el = 0.0
    for b in range(w.B):
        q0, q1, k0, k1 = (int(x) for x in (cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]))
        O, L = oracle.attention_varlen(q[:, q0:q1], k[:, k0:k1], v[:, k0:k1], [0, q1 - q0], [0, k1 - k0], w.causal)
        eo = max(eo, float(np.max(np.abs(og[:, q0:q1] - O))))
        el = max(el, float(np.max(np.abs(lg[:, q0:q1] - L))))
    log(f"  varlen-whole {w.name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}")
    assert eo <= 2e-2 and el <= 1e-3


def test_backward_whole_tensors_c5():
    import exact_tiled_attention_15_amd as fa

    w = W["c5_fp16_cross_b8h32q512k8192d64"]
    log(f"case {w.name} backward, whole tensors")
    cpu = workloads.make_inputs(w)
    dout = workloads.make_dout(w)
    q, k, v = to_gpu(cpu)
    o, lse = fa.forward(q, k, v, w.causal)
    grads = fa.backward(q, k, v, o, lse, dout.to("cuda:0"), w.causal)
    torch.cuda.synchronize()
    gc = [g.float().cpu() for g in grads]

    def head(bh):
        b, h = divmod(bh, w.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        ref = oracle.attention_backward(*(t[sl] for t in cpu), dout[sl], w.causal)
        out = []
        for g, r in zip(gc, ref):
            gg = g[sl].double().numpy()
            assert np.isfinite(gg).all()
            out.append((float(np.max(np.abs(gg - r))), float(np.max(np.abs(r)))))
        return out

    pool, limits = _oracle_pool()
    with pool, limits:
        per_head = list(pool.map(head, range(w.B * w.H)))
    for i, n in enumerate(("dQ", "dK", "dV")):
        err = max(x[i][0] for x in per_head)
        mx = max(x[i][1] for x in per_head)
        log(f"  bwd-whole {w.name} {n}: max err {err:.3e} (max |{n}| {mx:.3e})")
        assert err <= 2e-2 * mx + 1e-4
