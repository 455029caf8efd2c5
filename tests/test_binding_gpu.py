"""The Python binding's argument checks on the GPU: every tensor reaches the
kernels as a raw device address, so a tensor on the wrong device, of the
wrong dtype or shape, or not contiguous must raise before the C call (these
tests launch no kernel).  Also: FA_DEFAULT_SCALE selects exactly 1/sqrt(D)
in every entry point that takes a scale."""
import numpy as np
import pytest

import workloads
from parity_util import log, to_gpu

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _qkv(B=1, H=2, Nq=64, Nk=96, D=64, dtype=torch.bfloat16):
    g = torch.Generator(device=DEV).manual_seed(5)
    q = torch.randn(B, H, Nq, D, device=DEV, dtype=dtype, generator=g)
    k = torch.randn(B, H, Nk, D, device=DEV, dtype=dtype, generator=g)
    v = torch.randn(B, H, Nk, D, device=DEV, dtype=dtype, generator=g)
    return q, k, v


def test_forward_rejects_bad_tensors():
    import exact_tiled_attention_15_amd as fa

    q, k, v = _qkv()
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, k, v, out=torch.empty(q.shape, dtype=q.dtype))  # host out
    with pytest.raises(ValueError, match="GPU"):
        fa.forward(q, k, v, lse=torch.empty(q.shape[:3]))  # host lse
    with pytest.raises(TypeError):
        fa.forward(q, k.float(), v)  # k of another dtype
    with pytest.raises(TypeError):
        fa.forward(q, k, v, out=torch.empty_like(q, dtype=torch.float16))
    with pytest.raises(ValueError, match="shape"):
        fa.forward(q, k, v, lse=torch.empty(1, 2, 63, device=DEV))
    with pytest.raises(ValueError, match="contiguous"):
        fa.forward(q, k.transpose(2, 3).contiguous().transpose(2, 3), v)
    with pytest.raises(ValueError, match="shape"):
        fa.forward(q, k, v[:, :, :95].contiguous())


def test_splitkv_rejects_bad_tensors():
    import exact_tiled_attention_15_amd as fa

    q, k, v = _qkv(Nq=4, Nk=2048)
    with pytest.raises(TypeError):
        fa.forward_splitkv(q.float(), k, v)  # fp32 q with bf16 k, v
    with pytest.raises(TypeError):
        fa.forward_splitkv(q, k, v.half())
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_splitkv(q, k, v, out=torch.empty(q.shape, dtype=q.dtype))
    with pytest.raises(ValueError, match="shape"):
        fa.forward_splitkv(q, k, v, lse=torch.empty(1, 2, 5, device=DEV))
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_splitkv(q, k, v, workspace=torch.empty(1 << 20, dtype=torch.uint8))


def test_backward_rejects_bad_tensors():
    import exact_tiled_attention_15_amd as fa

    q, k, v = _qkv()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], device=DEV)
    do = torch.empty_like(q)
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(q, k, v, o, lse, do, dq=torch.empty(q.shape, dtype=q.dtype))
    with pytest.raises(ValueError, match="GPU"):
        fa.backward(q, k, v, o, lse, do, workspace=torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(TypeError):
        fa.backward(q, k, v, o, lse, do, dk=torch.empty_like(k, dtype=torch.float32))
    with pytest.raises(ValueError, match="shape"):
        fa.backward(q, k, v, o, lse, do, dv=torch.empty_like(q))
    with pytest.raises(TypeError):
        fa.backward(q, k, v, o, lse.double(), do)


def test_varlen_rejects_bad_tensors():
    import exact_tiled_attention_15_amd as fa

    q = torch.randn(2, 100, 64, device=DEV, dtype=torch.bfloat16)
    k = torch.randn(2, 120, 64, device=DEV, dtype=torch.bfloat16)
    cu_q = torch.tensor([0, 40, 100], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, 50, 120], dtype=torch.int32, device=DEV)
    with pytest.raises(TypeError):
        fa.forward_varlen(q, k, k, cu_q.long(), cu_k, 60)
    with pytest.raises(ValueError, match="GPU"):
        fa.forward_varlen(q, k, k, cu_q.cpu(), cu_k, 60)
    with pytest.raises(ValueError, match="shape"):
        fa.forward_varlen(q, k, k, cu_q, cu_k[:2].contiguous(), 60)
    with pytest.raises(ValueError, match="shape"):
        fa.forward_varlen(q, k, k, cu_q, cu_k, 60, out=torch.empty(2, 99, 64, device=DEV, dtype=q.dtype))
    with pytest.raises(TypeError):
        fa.forward_varlen(q, k.half(), k, cu_q, cu_k, 60)
    o = torch.empty_like(q)
    lse = torch.empty(2, 100, device=DEV)
    with pytest.raises(ValueError, match="GPU"):
        fa.backward_varlen(q, k, k, o, lse, o, cu_q, cu_k, 60, 70, dq=torch.empty(q.shape, dtype=q.dtype))


@pytest.mark.parametrize("dt,D", [("bf16", 128), ("fp16", 32), ("fp32", 64), ("bf16", 256)])
def test_default_scale_is_one_over_sqrt_d_everywhere(dt, D):
    # FA_DEFAULT_SCALE (0) and an explicit 1/sqrt(D) run the same kernels with
    # the same fp32 factor: identical bits, for every entry point with a scale.
    import exact_tiled_attention_15_amd as fa

    w = workloads.Workload(f"dflt_{dt}_d{D}", 1, 2, 200, 260, D, dt, True, 61 + D)
    log(f"case default scale {w.name}")
    q, k, v = to_gpu(workloads.make_inputs(w))
    s = 1.0 / D**0.5
    o0, l0 = fa.forward(q, k, v, True)  # fa_fwd
    o1, l1 = fa.forward(q, k, v, True, softmax_scale=fa.FA_DEFAULT_SCALE)  # fa_fwd_scaled(0)
    o2, l2 = fa.forward(q, k, v, True, softmax_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(o0, o2) and torch.equal(l0, l2)
    o3, l3 = fa.forward_splitkv(q, k, v, True, num_splits=3)
    o4, l4 = fa.forward_splitkv(q, k, v, True, num_splits=3, softmax_scale=s)
    torch.cuda.synchronize()
    assert torch.equal(o3, o4) and torch.equal(l3, l4)
    g = [fa.backward(q, k, v, o0, l0, o0, True, softmax_scale=sc) for sc in (None, s)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(*g))
    # varlen: one sequence per head-major block
    qv, kv, vv = (t[0].contiguous() for t in (q, k, v))
    cu_q = torch.tensor([0, 120, 200], dtype=torch.int32, device=DEV)
    cu_k = torch.tensor([0, 130, 260], dtype=torch.int32, device=DEV)
    r = [fa.forward_varlen(qv, kv, vv, cu_q, cu_k, 120, True, softmax_scale=sc) for sc in (None, s)]
    torch.cuda.synchronize()
    assert torch.equal(r[0][0], r[1][0]) and torch.equal(r[0][1], r[1][1])
    gv = [fa.backward_varlen(qv, kv, vv, r[0][0], r[0][1], r[0][0], cu_q, cu_k, 120, 130, True, softmax_scale=sc)
          for sc in (None, s)]
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(*gv))
