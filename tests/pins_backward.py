"""Checks that pin an attention backward implementation to the mathematics.

Each check takes ``impl(q, k, v, do, causal, scale) -> (dQ, dK, dV)`` on
float64 arrays and raises AssertionError when it disagrees with something
fixed independently of that implementation:

* central finite differences of sum(dO * O) through the brute-force forward
  loop of tests/pins.py (pure Python, math.fsum / math.exp), on tiny shapes;
* torch.autograd (float64, CPU) through a plain softmax-attention
  expression, at moderate non-square shapes;
* invariants: shifting every key by one vector leaves every score row's
  softmax unchanged, so the dK rows sum to zero; shifting every value by c
  shifts every O row by c, so the dV rows sum to the dO rows; constant V
  gives dQ = dK = 0; one key gives P = 1 (dV = sum of dO, dQ = dK = 0);
  linearity in dO.
"""
from __future__ import annotations

import math

import numpy as np

import pins


def _inputs(seed, B, H, Nq, Nk, D):
    r = np.random.default_rng(seed)
    return (r.standard_normal((B, H, Nq, D)), r.standard_normal((B, H, Nk, D)),
            r.standard_normal((B, H, Nk, D)), r.standard_normal((B, H, Nq, D)))


def _close(a, b, tol, what):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max abs err {err:.3e} > {tol:.1e}"


def _objective(q, k, v, do, causal, scale):
    O, _ = pins.brute_force(q, k, v, causal, scale)
    return math.fsum((O * do).ravel())


def _fd_grad(x, f, eps):
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
    return g


def check_finite_differences(impl):
    eps = 1e-5
    for causal in (False, True):
        for (Nq, Nk, D) in ((1, 1, 3), (3, 5, 4), (5, 3, 2), (4, 4, 1), (2, 7, 3)):
            for scale in (None, 0.8):
                q, k, v, do = _inputs(500 + 10 * Nq + Nk + D, 1, 2, Nq, Nk, D)
                dQ, dK, dV = impl(q, k, v, do, causal, scale)
                f = lambda: _objective(q, k, v, do, causal, scale)
                tag = f"FD Nq={Nq} Nk={Nk} D={D} causal={causal} scale={scale}"
                _close(dQ, _fd_grad(q, f, eps), 1e-7, tag + " dQ")
                _close(dK, _fd_grad(k, f, eps), 1e-7, tag + " dK")
                _close(dV, _fd_grad(v, f, eps), 1e-7, tag + " dV")


def check_torch_autograd(impl):
    import torch

    for causal in (False, True):
        for (Nq, Nk, D, scale) in ((37, 53, 16, None), (64, 40, 8, 0.3), (129, 129, 32, None)):
            q, k, v, do = _inputs(77 + Nq + Nk, 2, 2, Nq, Nk, D)
            tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
            sc = 1.0 / math.sqrt(D) if scale is None else scale
            s = torch.matmul(tq, tk.transpose(-1, -2)) * sc
            if causal:
                keep = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None]
                s = s.masked_fill(~keep, float("-inf"))
            o = torch.matmul(torch.softmax(s, dim=-1), tv)
            o.backward(torch.tensor(do, dtype=torch.float64))
            dQ, dK, dV = impl(q, k, v, do, causal, scale)
            tag = f"autograd Nq={Nq} Nk={Nk} D={D} causal={causal}"
            _close(dQ, tq.grad.numpy(), 1e-10, tag + " dQ")
            _close(dK, tk.grad.numpy(), 1e-10, tag + " dK")
            _close(dV, tv.grad.numpy(), 1e-10, tag + " dV")


def check_invariants(impl):
    for causal in (False, True):
        q, k, v, do = _inputs(91, 2, 3, 21, 17, 8)
        dQ, dK, dV = impl(q, k, v, do, causal, None)
        _close(dK.sum(axis=2), np.zeros((2, 3, 8)), 1e-10, "sum of dK rows = 0")
        _close(dV.sum(axis=2), do.sum(axis=2), 1e-10, "sum of dV rows = sum of dO rows")
        dQ2, dK2, dV2 = impl(q, k, v, -2.5 * do, causal, None)
        _close(dQ2, -2.5 * dQ, 1e-10, "linear in dO: dQ")
        _close(dK2, -2.5 * dK, 1e-10, "linear in dO: dK")
        _close(dV2, -2.5 * dV, 1e-10, "linear in dO: dV")
        vc = np.broadcast_to(np.linspace(-1, 2, 8), v.shape).copy()
        dQc, dKc, _ = impl(q, k, vc, do, causal, None)
        _close(dQc, np.zeros_like(dQc), 1e-12, "constant V: dQ = 0")
        _close(dKc, np.zeros_like(dKc), 1e-12, "constant V: dK = 0")
        # one key: every weight is 1
        q1, k1, v1, do1 = _inputs(92, 1, 2, 6, 1, 4)
        dQ1, dK1, dV1 = impl(q1, k1, v1, do1, causal, None)
        _close(dV1[:, :, 0], do1.sum(axis=2), 1e-12, "one key: dV = sum of dO")
        _close(dQ1, np.zeros_like(dQ1), 1e-12, "one key: dQ = 0")
        _close(dK1, np.zeros_like(dK1), 1e-12, "one key: dK = 0")


def check_causal_unseen_keys(impl):
    # causal with Nq < Nk: keys j >= Nq are seen by no query
    q, k, v, do = _inputs(93, 1, 2, 5, 9, 4)
    _, dK, dV = impl(q, k, v, do, True, None)
    _close(dK[:, :, 5:], np.zeros((1, 2, 4, 4)), 0.0, "unseen keys: dK = 0")
    _close(dV[:, :, 5:], np.zeros((1, 2, 4, 4)), 0.0, "unseen keys: dV = 0")
    # causal row 0 sees key 0 only: its dO reaches dV[0] with weight 1
    q, k, v, do = _inputs(94, 1, 1, 4, 4, 3)
    do0 = np.zeros_like(do)
    do0[:, :, 0] = do[:, :, 0]
    dQ, dK, dV = impl(q, k, v, do0, True, None)
    _close(dV[:, :, 0], do[:, :, 0], 1e-12, "causal row 0 -> dV[0]")
    _close(dV[:, :, 1:], np.zeros((1, 1, 3, 3)), 0.0, "causal row 0 touches no other key")


ALL_CHECKS = [check_finite_differences, check_torch_autograd, check_invariants, check_causal_unseen_keys]
