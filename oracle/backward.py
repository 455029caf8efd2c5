"""Float64 oracle of the attention backward pass: dQ, dK, dV.

Test infrastructure only (tests, the smoke check and the benchmark's
CPU-baseline leg); the product path never calls it.

"Building a FlashAttention-2 Forward Kernel in Pure NumPy" (Extending It)
names the backward pass as the step after the forward kernel: keep the
forward's softmax statistics and recompute the scores tile by tile while
streaming the gradients.  What that computes is the exact gradient of the
forward definition (the same function as ``oracle.attention``): for one
(batch, head), with S = scale * Q K^T (masked entries -inf), P = row
softmax of S, O = P V, and a given upstream gradient dO of O,

* dV = P^T dO
* dP = dO V^T
* dS = P * (dP - rowsum(P * dP))      (the softmax Jacobian applied row by row)
* dQ = scale * dS K,   dK = scale * dS^T Q

written out here from that definition with full rows (row chunks against all
keys, as the forward oracle does), not with the online recurrence and not
with the saved LSE.  Masked entries have P = 0, so they carry no gradient;
keys that no query sees get dK = dV = 0.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _as_f64, _check

__all__ = ["attention_backward", "attention_varlen_backward"]


def _block_grads(qi, kh, vh, doi, row_idx, causal, scale):
    """Gradients contributed by a block of query rows of one head.

    Returns dQ for the rows, and this block's parts of dK and dV.
    """
    s = (qi @ kh.T) * scale
    if causal:
        keys = np.arange(kh.shape[0])
        s = np.where(keys[None, :] <= row_idx[:, None], s, -np.inf)
    s = s - s.max(axis=1, keepdims=True)
    e = np.exp(s)
    p = e / e.sum(axis=1, keepdims=True)
    dv = p.T @ doi
    dp = doi @ vh.T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    dq = scale * (ds @ kh)
    dk = scale * (ds.T @ qi)
    return dq, dk, dv


def attention_backward(q, k, v, do, causal: bool, scale=None, row_chunk: int = 256):
    """Exact gradients of sum(dO * attention(q, k, v)) with respect to q, k, v.

    q, do: (B, H, Nq, D); k, v: (B, H, Nk, D); any real dtype (widened to
    float64).  scale defaults to 1/sqrt(D).  Returns float64 (dQ, dK, dV).
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H, Nq, Nk, D = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError(f"dO shape {do.shape} != q shape {q.shape}")
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    dQ = np.empty((B, H, Nq, D))
    dK = np.zeros((B, H, Nk, D))
    dV = np.zeros((B, H, Nk, D))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_chunk):
                r1 = min(r0 + row_chunk, Nq)
                dq, dk, dv = _block_grads(q[b, h, r0:r1], k[b, h], v[b, h], do[b, h, r0:r1],
                                          np.arange(r0, r1), causal, scale)
                dQ[b, h, r0:r1] = dq
                dK[b, h] += dk
                dV[b, h] += dv
    return dQ, dK, dV


def attention_varlen_backward(q, k, v, do, cu_q, cu_k, causal: bool, scale=None):
    """Exact gradients of sum(dO * attention_varlen(q, k, v, cu_q, cu_k)).

    Each packed sequence is an independent attention problem (its rows attend
    to its own keys only), so its gradients are ``attention_backward`` on its
    own rows; rows of sequences without keys get dQ = 0 (their O is the
    constant 0), keys of sequences without queries dK = dV = 0.  q, do:
    (H, total_q, D); k, v: (H, total_k, D); cu_q, cu_k: B + 1 offsets.
    Returns float64 (dQ, dK, dV) in those shapes.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    if do.shape != q.shape:
        raise ValueError(f"dO shape {do.shape} != q shape {q.shape}")
    dQ = np.zeros(q.shape)
    dK = np.zeros(k.shape)
    dV = np.zeros(v.shape)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        g = attention_backward(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], do[None, :, q0:q1], causal,
                               scale=scale)
        dQ[:, q0:q1] = g[0][0]
        dK[:, k0:k1] = g[1][0]
        dV[:, k0:k1] = g[2][0]
    return dQ, dK, dV
