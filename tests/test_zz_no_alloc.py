"""fa_fwd_splitkv_static (split-KV with the library's static device scratch,
no allocation) against fa_fwd_splitkv (caller workspace), through the C ABI:
the same kernels and key ranges, so the same bits.  Two calls in a row, the
second with a smaller input, so the second runs on scratch that still holds
the first call's partials."""
import pytest

import workloads
from parity_util import TOL, compare_full, log, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _with_workspace(fa, q, k, v, causal, splits):
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    need = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, splits)
    assert need > 0, "the case must run as several key ranges"
    ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=q.device)
    rc = fa.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), ws.data_ptr(),
                           need, B, H, Nq, Nk, D, fa.FA_DEFAULT_SCALE, splits, int(causal), fa._dtype_code(q),
                           torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_status_str(rc)
    return o, lse, need


def _static(fa, q, k, v, causal, splits):
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), device=q.device)
    rc = fa.fa_fwd_splitkv_static(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                                  Nk, D, fa.FA_DEFAULT_SCALE, splits, int(causal), fa._dtype_code(q),
                                  torch.cuda.current_stream().cuda_stream)
    assert rc == fa.FA_OK, fa.fa_status_str(rc)
    return o, lse


@pytest.mark.parametrize("dt", ["bf16", "fp32"])
def test_static_scratch_matches_workspace_twice(dt):
    import exact_tiled_attention_15_amd as fa

    cases = [
        # decoding shape with automatic ranges (16 rows against 20000 keys),
        # then a smaller, causal one with an explicit range count
        workloads.Workload(f"static_a_{dt}", 1, 32, 16, 20000, 128, dt, False, 91),
        workloads.Workload(f"static_b_{dt}", 1, 4, 5, 900, 64, dt, True, 92),
    ]
    for w, splits in zip(cases, (0, 5)):
        log(f"case {w.name} B={w.B} H={w.H} Nq={w.Nq} Nk={w.Nk} D={w.D} splits={splits}")
        cpu = workloads.make_inputs(w)
        q, k, v = to_gpu(cpu)
        o1, l1, need = _with_workspace(fa, q, k, v, w.causal, splits)
        assert need <= fa.FA_STATIC_SCRATCH_BYTES
        o2, l2 = _static(fa, q, k, v, w.causal, splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "static-scratch result differs from the workspace one"
        compare_full(w, cpu, o2, l2, "static")
