"""Independent float64 online-softmax tiled attention (test-only).

Written separately from the oracle to pin it: it follows the online update
of "Building a FlashAttention-2 Forward Kernel in Pure NumPy" (Step 3: new
running max, correction factor exp(m_old - m_new), new running sum; Step 4:
rescale the accumulator, add the tile's P V, divide by the running sum at
the end), but walks the loops the way the GPU kernel does: one Q tile at a
time (outer), streaming K/V tiles (inner).  Tile sizes are free; in exact
arithmetic the result does not depend on them.

The mask uses absolute indices (keep key j for query i when j <= i,
top-left aligned).  Rows whose keys in a tile are all masked keep their
state unchanged (the guard for exp(-inf - -inf)).
"""
from __future__ import annotations

import math

import numpy as np


def online_tiled_attention(q, k, v, causal, br, bc, skip_masked_tiles=True):
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    c = 1.0 / math.sqrt(D)
    O = np.zeros((B, H, Nq, D))
    LSE = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for i0 in range(0, Nq, br):
                i1 = min(i0 + br, Nq)
                qi = q[b, h, i0:i1]
                rows = np.arange(i0, i1)
                run_max = np.full(i1 - i0, -np.inf)
                run_sum = np.zeros(i1 - i0)
                acc = np.zeros((i1 - i0, D))
                # last key any row of this tile may see
                k_end = min(Nk, i1) if causal else Nk
                for j0 in range(0, Nk, bc):
                    if skip_masked_tiles and j0 >= k_end:
                        break
                    j1 = min(j0 + bc, Nk)
                    t = (qi @ k[b, h, j0:j1].T) * c
                    if causal:
                        cols = np.arange(j0, j1)
                        t = np.where(cols[None, :] <= rows[:, None], t, -np.inf)
                    tile_max = t.max(axis=1)
                    new_max = np.maximum(run_max, tile_max)
                    live = np.isfinite(new_max)
                    corr = np.where(live, np.exp(np.where(live, run_max - new_max, 0.0)), 1.0)
                    p = np.where(live[:, None], np.exp(t - np.where(live, new_max, 0.0)[:, None]), 0.0)
                    run_sum = corr * run_sum + p.sum(axis=1)
                    acc = corr[:, None] * acc + p @ v[b, h, j0:j1]
                    run_max = np.where(live, new_max, run_max)
                O[b, h, i0:i1] = acc / run_sum[:, None]
                LSE[b, h, i0:i1] = run_max + np.log(run_sum)
    return O, LSE
