"""The float64 backward oracle against finite differences of the brute-force
forward, torch.autograd, invariants and closed forms; and planted mistakes
in copies of its definition, each of which must fail one of those pins."""
import math

import numpy as np
import pytest

import oracle
import pins_backward as pb


def _impl(q, k, v, do, causal, scale):
    return oracle.attention_backward(q, k, v, do, causal, scale=scale)


def _impl_chunked(q, k, v, do, causal, scale):
    return oracle.attention_backward(q, k, v, do, causal, scale=scale, row_chunk=2)


@pytest.mark.parametrize("check", pb.ALL_CHECKS, ids=lambda f: f.__name__)
def test_backward_oracle_pinned(check):
    check(_impl)


@pytest.mark.parametrize("check", [pb.check_torch_autograd, pb.check_invariants],
                         ids=lambda f: f.__name__)
def test_backward_oracle_row_chunking(check):
    check(_impl_chunked)


def test_backward_rejects_bad_shapes():
    z = np.zeros((1, 1, 3, 4))
    with pytest.raises(ValueError):
        oracle.attention_backward(z, z, z, np.zeros((1, 1, 2, 4)), False)


def _mutant(q, k, v, do, causal, scale, *, delta=True, dq_scale=True, dk_scale=True, strict=False,
            delta_axis=1, dv_from_ds=False):
    B, H, Nq, D = q.shape
    sc = 1.0 / math.sqrt(D) if scale is None else scale
    dQ, dK, dV = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            s = q[b, h] @ k[b, h].T * sc
            if causal:
                keep = (np.arange(k.shape[2])[None, :] < np.arange(Nq)[:, None]) if strict else \
                       (np.arange(k.shape[2])[None, :] <= np.arange(Nq)[:, None])
                s = np.where(keep, s, -np.inf)
            with np.errstate(invalid="ignore"):
                p = np.exp(s - s.max(1, keepdims=True))
                p = np.nan_to_num(p / p.sum(1, keepdims=True))
            dp = do[b, h] @ v[b, h].T
            ds = p * (dp - (p * dp).sum(delta_axis, keepdims=True)) if delta else p * dp
            dV[b, h] = ds.T @ do[b, h] if dv_from_ds else p.T @ do[b, h]
            dQ[b, h] = (sc if dq_scale else 1.0) * ds @ k[b, h]
            dK[b, h] = (sc if dk_scale else 1.0) * ds.T @ q[b, h]
    return dQ, dK, dV


MUTANTS = {
    "no_delta_term": dict(delta=False),
    "dq_unscaled": dict(dq_scale=False),
    "dk_unscaled": dict(dk_scale=False),
    "strict_causal_mask": dict(strict=True),
    "delta_over_queries": dict(delta_axis=0),
    "dv_from_ds": dict(dv_from_ds=True),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_backward_planted_mistake_is_caught(name):
    kw = MUTANTS[name]
    impl = lambda q, k, v, do, c, s: _mutant(q, k, v, do, c, s, **kw)
    caught = []
    for check in pb.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_backward_unmutated_definition_passes():
    for check in pb.ALL_CHECKS:
        check(lambda q, k, v, do, c, s: _mutant(q, k, v, do, c, s))


# ---------------------------------------------------------------------------
# Packed variable-length sequences: oracle.attention_varlen_backward
# ---------------------------------------------------------------------------
def _varlen_fd(q, k, v, do, cu_q, cu_k, causal, scale, eps=1e-5):
    """Central finite differences of sum(dO * O) through the varlen forward
    oracle (a separate definition: per-sequence slices of the forward)."""
    def f():
        O, _ = oracle.attention_varlen(q, k, v, cu_q, cu_k, causal, scale=scale)
        return float(np.sum(O * do))

    grads = []
    for x in (q, k, v):
        g = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            old = x[i]
            x[i] = old + eps
            fp = f()
            x[i] = old - eps
            fm = f()
            x[i] = old
            g[i] = (fp - fm) / (2 * eps)
        grads.append(g)
    return grads


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_backward_oracle_finite_differences(causal):
    # sequence 1 has keys but no queries, sequence 2 queries but no keys
    lens_q, lens_k = [2, 0, 3, 4], [3, 2, 0, 2]
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int64)
    r = np.random.default_rng(31)
    H, D = 2, 3
    q = r.standard_normal((H, cu_q[-1], D))
    k = r.standard_normal((H, cu_k[-1], D))
    v = r.standard_normal((H, cu_k[-1], D))
    do = r.standard_normal((H, cu_q[-1], D))
    for scale in (None, 0.7):
        got = oracle.attention_varlen_backward(q, k, v, do, cu_q, cu_k, causal, scale=scale)
        ref = _varlen_fd(q, k, v, do, cu_q, cu_k, causal, scale)
        for name, a, b in zip(("dQ", "dK", "dV"), got, ref):
            assert np.max(np.abs(a - b)) <= 1e-7, (name, scale, float(np.max(np.abs(a - b))))
    dQ, dK, dV = oracle.attention_varlen_backward(q, k, v, do, cu_q, cu_k, causal)
    assert np.all(dQ[:, cu_q[2]:cu_q[3]] == 0.0)  # queries without keys
    assert np.all(dK[:, cu_k[1]:cu_k[2]] == 0.0) and np.all(dV[:, cu_k[1]:cu_k[2]] == 0.0)  # keys without queries


def test_varlen_backward_oracle_equal_lengths_match_dense():
    # B equal-length sequences packed head-major are the dense batch
    r = np.random.default_rng(32)
    B, H, N, D = 3, 2, 17, 8
    q, k, v, do = (r.standard_normal((B, H, N, D)) for _ in range(4))
    pack = lambda t: t.transpose(1, 0, 2, 3).reshape(H, B * N, D)
    cu = np.arange(B + 1) * N
    for causal in (False, True):
        dense = oracle.attention_backward(q, k, v, do, causal)
        packed = oracle.attention_varlen_backward(pack(q), pack(k), pack(v), pack(do), cu, cu, causal)
        for a, b in zip(packed, dense):
            assert np.array_equal(a, pack(b))
