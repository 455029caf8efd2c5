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
