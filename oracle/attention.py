"""Float64 oracle: exact softmax(Q K^T / sqrt(D)) V plus the row log-sum-exp.

Test infrastructure only (tests, the smoke check and the benchmark's
CPU-baseline leg); the product path never calls it.

What it computes, per batch b and head h, in float64 on the stored input
values:

* scale = 1 / sqrt(D)  (every page divides the scores by sqrt of the head
  dimension: "Build a FlashAttention Kernel from Scratch", Step 3;
  "Building a FlashAttention-2 Forward Kernel in Pure NumPy", Step 2;
  "Python Attention Mechanisms Explained", The Core Idea), unless an
  explicit ``scale`` is given (the softmax_scale argument of the library call
  on "Flash Attention vs Standard Attention", Implementation)
* the key set of query i is A_i = {j : 0 <= j < Nk, and j <= i if causal}.
  The causal mask keeps the diagonal (the first page's comment on its Step 3
  mask says lower triangle including the diagonal; the printed call drops
  it, which would leave row 0 empty).  For Nq != Nk the mask is aligned at
  the top-left (absolute indices), the plainest reading: the pages only show
  square causal examples.
* s_ij = scale * sum_d q[i,d] k[j,d]  for j in A_i
* m_i = max_j s_ij,  l_i = sum_j exp(s_ij - m_i)
* LSE_i = m_i + ln(l_i)  (natural log; the "log-sum-exp" the FlashAttention-2
  page names, i.e. scipy.special.logsumexp of the masked scaled scores)
* O_i = sum_j exp(s_ij - m_i) v[j,:] / l_i

The pages state that the tiled method reaches exactly this result, so the
oracle is the definition written out, not the online algorithm.  Rows are
processed in chunks against all keys at once, the row blocking of the first
page's Step 6 (with the mask in absolute indices); this is exact, not
online.  Masked entries become -inf before the max.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["attention_forward", "attention_rows", "scores_row", "attention_partial", "merge_partials",
           "attention_varlen"]


def _as_f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # a torch CPU tensor of any dtype
        x = x.detach().to("cpu").double().numpy()
    return np.asarray(x, dtype=np.float64)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be (B, H, N, D)")
    B, H, Nq, D = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != D or v.shape != k.shape:
        raise ValueError(f"shape mismatch: q{q.shape} k{k.shape} v{v.shape}")
    if Nq < 1 or k.shape[2] < 1 or D < 1:
        raise ValueError("empty attention is undefined (every row needs a key)")
    return B, H, Nq, k.shape[2], D


def _rows_block(qi, kh, vh, row_idx, causal, scale):
    """Exact attention for a block of query rows against all keys of one head.

    qi: (R, D) query rows, row_idx: (R,) their absolute indices.
    Returns O (R, D) and LSE (R,).
    """
    s = (qi @ kh.T) * scale  # (R, Nk)
    if causal:
        keys = np.arange(kh.shape[0])
        s = np.where(keys[None, :] <= row_idx[:, None], s, -np.inf)
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])  # exp(-inf) = 0 for masked keys
    l = e.sum(axis=1)
    o = (e @ vh) / l[:, None]
    lse = m + np.log(l)
    return o, lse


def _scale(D, scale):
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def attention_forward(q, k, v, causal: bool, row_chunk: int = 256, scale=None):
    """Exact attention over whole tensors.

    q: (B, H, Nq, D); k, v: (B, H, Nk, D); any real dtype (widened to float64).
    scale: the factor applied to q.k (default 1/sqrt(D)).
    Returns (O float64 (B, H, Nq, D), LSE float64 (B, H, Nq)).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, Nk, D = _check(q, k, v)
    scale = _scale(D, scale)
    O = np.empty((B, H, Nq, D))
    L = np.empty((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for r0 in range(0, Nq, row_chunk):
                r1 = min(r0 + row_chunk, Nq)
                o, lse = _rows_block(q[b, h, r0:r1], k[b, h], v[b, h],
                                     np.arange(r0, r1), causal, scale)
                O[b, h, r0:r1] = o
                L[b, h, r0:r1] = lse
    return O, L


def attention_rows(q, k, v, causal: bool, rows, scale=None):
    """Exact attention for selected query rows only.

    rows: iterable of (b, h, i).  Inputs may be torch tensors or arrays; only
    the needed head slices are widened.  Returns (O (R, D), LSE (R,)).
    """
    rows = [tuple(int(x) for x in r) for r in rows]
    D = q.shape[-1]
    scale = _scale(D, scale)
    O = np.empty((len(rows), D))
    L = np.empty(len(rows))
    by_head = {}
    for n, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((n, i))
    for (b, h), items in by_head.items():
        kh = _as_f64(k[b, h])
        vh = _as_f64(v[b, h])
        idx = np.array([i for _, i in items])
        if hasattr(q, "detach"):
            import torch

            qi = _as_f64(q[b, h][torch.as_tensor(idx)])
        else:
            qi = _as_f64(q[b, h])[idx]
        o, lse = _rows_block(qi, kh, vh, idx, causal, scale)
        for r, (n, _) in enumerate(items):
            O[n] = o[r]
            L[n] = lse[r]
    return O, L


def scores_row(q, k, b: int, h: int, i: int, causal: bool, scale=None):
    """Scaled, masked float64 scores of one query row (masked keys -> -inf)."""
    D = q.shape[-1]
    qi = _as_f64(q[b, h, i])
    kh = _as_f64(k[b, h])
    s = (kh @ qi) * _scale(D, scale)
    if causal:
        s = np.where(np.arange(kh.shape[0]) <= i, s, -np.inf)
    return s


def attention_partial(q, k, v, causal: bool, k0: int, k1: int, scale=None):
    """Exact attention of every query row against keys [k0, k1) only (the
    causal mask still compares absolute indices).  Rows that see no key of
    the range get O = 0 and LSE = -inf (the empty sum).  Returns float64
    (O (B, H, Nq, D), LSE (B, H, Nq))."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, Nq, Nk, D = _check(q, k, v)
    if not 0 <= k0 < k1 <= Nk:
        raise ValueError(f"key range [{k0}, {k1}) outside [0, {Nk})")
    scale = _scale(D, scale)
    O = np.zeros((B, H, Nq, D))
    L = np.full((B, H, Nq), -np.inf)
    keys = np.arange(k0, k1)
    for b in range(B):
        for h in range(H):
            s = (q[b, h] @ k[b, h, k0:k1].T) * scale
            if causal:
                s = np.where(keys[None, :] <= np.arange(Nq)[:, None], s, -np.inf)
            seen = np.isfinite(s).any(axis=1)
            if not seen.any():
                continue
            sr = s[seen]
            m = sr.max(axis=1)
            e = np.exp(sr - m[:, None])
            l = e.sum(axis=1)
            O[b, h, seen] = (e @ v[b, h, k0:k1]) / l[:, None]
            L[b, h, seen] = m + np.log(l)
    return O, L


def merge_partials(parts):
    """Combine exact partials (O_s, LSE_s) over disjoint key ranges into the
    result over their union, by the numerically stable associative update
    that folds partial results into one output row ("Building a
    FlashAttention-2 Forward Kernel in Pure NumPy", Architecture Overview):
    LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s (empty partials,
    LSE_s = -inf, weigh nothing)."""
    Ls = np.stack([np.asarray(L, dtype=np.float64) for _, L in parts])
    Os = np.stack([np.asarray(O, dtype=np.float64) for O, _ in parts])
    m = Ls.max(axis=0)
    w = np.exp(Ls - m[None])
    tot = w.sum(axis=0)
    O = (w[..., None] * Os).sum(axis=0) / tot[..., None]
    return O, m + np.log(tot)


def attention_varlen(q, k, v, cu_q, cu_k, causal: bool, scale=None):
    """Exact attention over packed variable-length sequences, un-padded
    ("Flash Attention vs Standard Attention", Frequently Asked Questions).

    q: (H, total_q, D), k, v: (H, total_k, D) (head-major packing); cu_q,
    cu_k: B + 1 offsets.  Sequence b's rows [cu_q[b], cu_q[b+1]) attend to
    its keys [cu_k[b], cu_k[b+1]) only, with the causal mask aligned at the
    sequence's first row and key.  A sequence with queries and no keys gets
    O = 0 and LSE = -inf.  Returns float64 (O (H, total_q, D), LSE (H, total_q)).
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    H, total_q, D = q.shape
    O = np.zeros((H, total_q, D))
    L = np.full((H, total_q), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b]), int(cu_k[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        o, lse = attention_forward(q[None, :, q0:q1], k[None, :, k0:k1], v[None, :, k0:k1], causal, scale=scale)
        O[:, q0:q1] = o[0]
        L[:, q0:q1] = lse[0]
    return O, L
