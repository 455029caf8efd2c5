"""Planted mistakes: copies of the oracle's definition with one plausible
error each.  Every one must fail at least one pin in tests/pins.py; this is
what makes the pins a real check of the oracle rather than a restatement."""
import math

import numpy as np
import pytest

import pins


def _definition(q, k, v, causal, *, scale_fn=lambda D: 1.0 / math.sqrt(D), keep=None,
                normalize=True, lse_fn=None, v_fn=None, swap_qk=False, eps=0.0):
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if swap_qk:
        n = min(Nq, Nk)
        s = np.einsum("bhjd,bhid->bhij", k[:, :, :Nq] if Nk >= Nq else np.pad(k, ((0, 0), (0, 0), (0, Nq - Nk), (0, 0))),
                      q[:, :, :Nk] if Nq >= Nk else np.pad(q, ((0, 0), (0, 0), (0, Nk - Nq), (0, 0))))
        s = s[:, :, :Nq, :Nk] * scale_fn(D)
    else:
        s = np.einsum("bhid,bhjd->bhij", q, k) * scale_fn(D)
    if causal:
        keep = keep or (lambda i, j, Nq, Nk: j <= i)
        ii, jj = np.meshgrid(np.arange(Nq), np.arange(Nk), indexing="ij")
        s = np.where(keep(ii, jj, Nq, Nk), s, -np.inf)
    m = s.max(-1)
    e = np.exp(s - m[..., None])
    l = e.sum(-1) + eps
    vv = v_fn(v) if v_fn else v
    o = np.matmul(e, vv)
    if normalize:
        o = o / l[..., None]
    lse = lse_fn(m, l) if lse_fn else m + np.log(l)
    return o, lse


def _p3_tiled_no_rescale(q, k, v, causal, br=32, bc=16):
    # the third page's loop: per-tile max, no correction of earlier tiles
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    O = np.zeros_like(q)
    L = np.zeros(q.shape[:3])
    for i0 in range(0, Nq, br):
        qi = q[:, :, i0:i0 + br]
        acc = np.zeros_like(qi)
        tot = np.zeros(qi.shape[:3])
        run = np.full(qi.shape[:3], -np.inf)
        for j0 in range(0, Nk, bc):
            t = np.einsum("bhid,bhjd->bhij", qi, k[:, :, j0:j0 + bc]) / math.sqrt(D)
            if causal:
                ii = np.arange(i0, i0 + qi.shape[2])[:, None]
                jj = np.arange(j0, j0 + t.shape[3])[None, :]
                t = np.where(jj <= ii, t, -np.inf)
            tm = t.max(-1)
            run = np.maximum(run, tm)
            with np.errstate(invalid="ignore"):
                e = np.exp(t - tm[..., None])
            e = np.nan_to_num(e)
            tot = tot + e.sum(-1)
            acc = acc + np.matmul(e, v[:, :, j0:j0 + bc])
        O[:, :, i0:i0 + br] = acc / tot[..., None]
        L[:, :, i0:i0 + br] = run + np.log(tot)
    return O, L


MUTANTS = {
    "scale_1_over_d": lambda q, k, v, c: _definition(q, k, v, c, scale_fn=lambda D: 1.0 / D),
    "no_scale": lambda q, k, v, c: _definition(q, k, v, c, scale_fn=lambda D: 1.0),
    "strict_lower_mask": lambda q, k, v, c: _definition(q, k, v, c, keep=lambda i, j, a, b: j < i),
    "bottom_right_mask": lambda q, k, v, c: _definition(q, k, v, c, keep=lambda i, j, a, b: j <= i + (b - a)),
    "mask_off_by_one": lambda q, k, v, c: _definition(q, k, v, c, keep=lambda i, j, a, b: j <= i + 1),
    "mask_ignored": lambda q, k, v, c: _definition(q, k, v, False),
    "no_normalization": lambda q, k, v, c: _definition(q, k, v, c, normalize=False),
    "lse_without_max": lambda q, k, v, c: _definition(q, k, v, c, lse_fn=lambda m, l: np.log(l)),
    "lse_log2": lambda q, k, v, c: _definition(q, k, v, c, lse_fn=lambda m, l: (m + np.log(l)) / math.log(2)),
    "v_keys_reversed": lambda q, k, v, c: _definition(q, k, v, c, v_fn=lambda v: v[:, :, ::-1]),
    "v_last_key_dropped": lambda q, k, v, c: _definition(q, k, v, c, v_fn=lambda v: np.concatenate([v[:, :, :-1], 0 * v[:, :, -1:]], 2)),
    "q_k_roles_swapped": lambda q, k, v, c: _definition(q, k, v, c, swap_qk=True),
    "denominator_epsilon": lambda q, k, v, c: _definition(q, k, v, c, eps=1e-6),
    "p3_tiled_no_rescale": _p3_tiled_no_rescale,
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name):
    impl = MUTANTS[name]
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            with np.errstate(all="ignore"):
                check(impl)
        except (AssertionError, ValueError, IndexError) as e:
            caught.append(check.__name__)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_definition_passes():
    impl = lambda q, k, v, c: _definition(q, k, v, c)
    for check in pins.ALL_CHECKS:
        check(impl)


def test_ignored_explicit_scale_is_caught():
    # an implementation that drops the explicit scale (always 1/sqrt(D))
    impl = lambda q, k, v, c, scale: _definition(q, k, v, c)
    with pytest.raises(AssertionError):
        pins.check_explicit_scale(impl)
    # applying the scale to the exponent base instead of the scores
    impl2 = lambda q, k, v, c, scale: _definition(q, k, v, c, scale_fn=lambda D: scale / math.sqrt(D))
    with pytest.raises(AssertionError):
        pins.check_explicit_scale(impl2)
    pins.check_explicit_scale(lambda q, k, v, c, scale: _definition(q, k, v, c, scale_fn=lambda D: scale))
