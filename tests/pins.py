"""Checks that pin an attention implementation to the mathematics.

Each check takes an implementation ``impl(q, k, v, causal) -> (O, LSE)`` on
float64 arrays shaped (B, H, Nq, D) / (B, H, Nk, D) and raises
AssertionError when it disagrees with something the pages or the
mathematics fix independently of that implementation:

* a brute-force per-element loop (math.fsum / math.exp) on tiny shapes;
* hand-derived worked examples with closed forms (tests/golden);
* scipy.special.logsumexp of the row scores (the routine the FlashAttention-2
  NumPy page names for the log-sum-exp);
* invariants: rows of the softmax sum to 1, constant V gives constant O,
  causal row 0 gives O = V[0], linearity in V, key permutation invariance,
  causal equals non-causal on the last row;
* closed forms: Q = 0 gives uniform weights (LSE = ln |A_i|, O = mean of V
  over the kept keys);
* the peaky limit: one dominant key gives O -> V[argmax];
* an independent float64 online-softmax tiled implementation at many tile
  sizes (tests/online_reference.py).

The same checks run against deliberately broken implementations in
test_pin_power.py, to show that each plausible mistake fails one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B, H, Nq, Nk, D):
    r = _rng(seed)
    return (r.standard_normal((B, H, Nq, D)), r.standard_normal((B, H, Nk, D)),
            r.standard_normal((B, H, Nk, D)))


def brute_force(q, k, v, causal, scale=None):
    """Per-element loop straight from the definition, with exact sums."""
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    O = np.zeros((B, H, Nq, D))
    L = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if (not causal) or j <= i]
                s = [scale * math.fsum(q[b, h, i, d] * k[b, h, j, d] for d in range(D)) for j in keys]
                mx = max(s)
                w = [math.exp(x - mx) for x in s]
                tot = math.fsum(w)
                L[b, h, i] = mx + math.log(tot)
                for d in range(D):
                    O[b, h, i, d] = math.fsum(wj * v[b, h, j, d] for wj, j in zip(w, keys)) / tot
    return O, L


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def check_brute_force(impl):
    for causal in (False, True):
        for Nq in (1, 2, 3, 5, 9):
            for Nk in (1, 2, 3, 5, 9):
                for D in (1, 4, 8):
                    q, k, v = _inputs(1000 + 100 * Nq + 10 * Nk + D, 1, 2, Nq, Nk, D)
                    O, L = impl(q, k, v, causal)
                    Ob, Lb = brute_force(q, k, v, causal)
                    tag = f"brute Nq={Nq} Nk={Nk} D={D} causal={causal}"
                    _close(O, Ob, 1e-12, tag + " O")
                    _close(L, Lb, 1e-12, tag + " LSE")


def check_explicit_scale(impl_scaled):
    """``impl_scaled(q, k, v, causal, scale)``: an explicit softmax scale
    multiplies q.k (brute force), which is the same as scaling Q by
    scale * sqrt(D) at the default scale."""
    for causal in (False, True):
        for (Nq, Nk, D) in ((3, 5, 4), (9, 2, 8), (5, 9, 1)):
            q, k, v = _inputs(3000 + Nq + Nk + D, 1, 2, Nq, Nk, D)
            for scale in (0.05, 0.7, 2.0):
                O, L = impl_scaled(q, k, v, causal, scale)
                Ob, Lb = brute_force(q, k, v, causal, scale)
                tag = f"scale={scale} Nq={Nq} Nk={Nk} D={D} causal={causal}"
                _close(O, Ob, 1e-12, tag + " O")
                _close(L, Lb, 1e-12, tag + " LSE")
        q, k, v = _inputs(3100, 2, 2, 17, 23, 16)
        t = 0.37
        O1, L1 = impl_scaled(q, k, v, causal, t / math.sqrt(16))
        O2, L2 = impl_scaled(q * t, k, v, causal, 1.0 / math.sqrt(16))
        _close(O1, O2, 1e-12, "scale t/sqrt(D) == Q scaled by t: O")
        _close(L1, L2, 1e-12, "scale t/sqrt(D) == Q scaled by t: LSE")


def check_golden(impl):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        q = np.array(c["q"], float)[None, None]
        k = np.array(c["k"], float)[None, None]
        v = np.array(c["v"], float)[None, None]
        O, L = impl(q, k, v, c["causal"])
        _close(O[0, 0], np.array(c["O"]), 1e-12, c["name"] + " O")
        _close(L[0, 0], np.array(c["LSE"]), 1e-12, c["name"] + " LSE")


def _row_scores(q, k, causal):
    D = q.shape[-1]
    s = np.einsum("bhid,bhjd->bhij", q, k) / math.sqrt(D)
    if causal:
        Nq, Nk = q.shape[2], k.shape[2]
        keep = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
        s = np.where(keep, s, -np.inf)
    return s


def check_logsumexp_scipy(impl):
    from scipy.special import logsumexp, softmax

    for causal in (False, True):
        for (Nq, Nk, D) in ((33, 47, 16), (64, 64, 32), (17, 100, 64)):
            q, k, v = _inputs(7 + Nq + Nk + D, 2, 2, Nq, Nk, D)
            O, L = impl(q, k, v, causal)
            s = _row_scores(q, k, causal)
            _close(L, logsumexp(s, axis=-1), 1e-12, "scipy logsumexp")
            w = softmax(s, axis=-1)
            _close(O, np.matmul(w, v), 1e-12, "scipy softmax weights @ V")
            # rows of exp(s - LSE) sum to one
            _close(np.exp(s - L[..., None]).sum(-1), np.ones_like(L), 1e-12, "softmax rows sum to 1")


def check_zero_q(impl):
    for causal in (False, True):
        for (Nq, Nk, D) in ((7, 7, 8), (5, 11, 4), (40, 40, 64)):
            _, k, v = _inputs(31 + Nq + Nk, 1, 2, Nq, Nk, D)
            q = np.zeros((1, 2, Nq, D))
            O, L = impl(q, k, v, causal)
            n_keys = np.array([(min(i, Nk - 1) + 1) if causal else Nk for i in range(Nq)], float)
            _close(L, np.broadcast_to(np.log(n_keys), L.shape), 1e-12, "Q=0 LSE = ln|A_i|")
            if causal:
                prefix = np.cumsum(v, axis=2) / np.arange(1, Nk + 1)[None, None, :, None]
                want = prefix[:, :, [min(i, Nk - 1) for i in range(Nq)]]
            else:
                want = np.broadcast_to(v.mean(axis=2, keepdims=True), O.shape)
            _close(O, want, 1e-12, "Q=0 O = mean of V over kept keys")


def check_constant_v(impl):
    for causal in (False, True):
        q, k, _ = _inputs(41, 2, 3, 19, 23, 16)
        c = np.linspace(-2.0, 3.0, 16)
        v = np.broadcast_to(c, (2, 3, 23, 16)).copy()
        O, _ = impl(q, k, v, causal)
        _close(O, np.broadcast_to(c, O.shape), 1e-12, "constant V -> constant O")


def check_causal_row0_and_last(impl):
    q, k, v = _inputs(51, 2, 2, 24, 24, 8)
    Oc, Lc = impl(q, k, v, True)
    _close(Oc[:, :, 0], v[:, :, 0], 1e-12, "causal row 0: O = V[0]")
    s00 = np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]) / math.sqrt(8)
    _close(Lc[:, :, 0], s00, 1e-12, "causal row 0: LSE = s00")
    On, Ln = impl(q, k, v, False)
    _close(Oc[:, :, -1], On[:, :, -1], 1e-12, "causal last row == non-causal last row")
    _close(Lc[:, :, -1], Ln[:, :, -1], 1e-12, "causal last row LSE")
    # and the causal result differs from non-causal on earlier rows
    assert np.max(np.abs(Oc[:, :, :-1] - On[:, :, :-1])) > 1e-3, "causal mask had no effect"


def check_linearity_and_permutation(impl):
    q, k, v = _inputs(61, 1, 2, 13, 29, 8)
    O, L = impl(q, k, v, False)
    O2, L2 = impl(q, k, 2.5 * v - 0.75, False)
    _close(O2, 2.5 * O - 0.75, 1e-12, "O(aV+b) = aO+b")
    _close(L2, L, 1e-12, "LSE independent of V")
    perm = _rng(5).permutation(29)
    O3, L3 = impl(q, k[:, :, perm], v[:, :, perm], False)
    _close(O3, O, 1e-12, "key permutation invariance O")
    _close(L3, L, 1e-12, "key permutation invariance LSE")


def check_peaky_limit(impl):
    # one key aligned with the query dominates as the query grows
    D, Nk = 8, 6
    r = _rng(71)
    k = r.standard_normal((1, 1, Nk, D))
    v = r.standard_normal((1, 1, Nk, D))
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0] = k[0, 0, 3] * 200.0
    O, L = impl(q, k, v, False)
    _close(O[0, 0, 0], v[0, 0, 3], 1e-9, "peaky row -> V[argmax]")
    s = (k[0, 0] @ q[0, 0, 0]) / math.sqrt(D)
    _close(L[0, 0, 0], s.max(), 1e-9, "peaky row LSE -> max score")


def check_online_tiled(impl):
    from online_reference import online_tiled_attention

    # the FlashAttention-2 NumPy page's pytest grid (N, d, block) plus odd sizes
    grid = [(N, N, d, br, br) for N in (64, 128, 256) for d in (32, 64) for br in (16, 32)]
    grid += [(77, 131, 64, 1, 3), (77, 131, 64, 16, 64), (77, 131, 64, 64, 131),
             (100, 100, 8, 64, 16), (100, 100, 8, 16, 64), (33, 9, 4, 64, 1)]
    for n, (Nq, Nk, D, br, bc) in enumerate(grid):
        for causal in (False, True):
            q, k, v = _inputs(900 + n, 1, 2, Nq, Nk, D)
            O, L = impl(q, k, v, causal)
            Ot, Lt = online_tiled_attention(q, k, v, causal, br, bc)
            tag = f"online Nq={Nq} Nk={Nk} D={D} Br={br} Bc={bc} causal={causal}"
            _close(O, Ot, 1e-12, tag + " O")
            _close(L, Lt, 1e-12, tag + " LSE")


ALL_CHECKS = [
    check_brute_force,
    check_golden,
    check_logsumexp_scipy,
    check_zero_q,
    check_constant_v,
    check_causal_row0_and_last,
    check_linearity_and_permutation,
    check_peaky_limit,
    check_online_tiled,
]
