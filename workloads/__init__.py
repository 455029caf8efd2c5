"""Seeded synthetic workloads for exact tiled attention.

This module holds no attention arithmetic.  It only knows the workload
shapes and how their inputs are drawn, so that the float64 oracle and the
HIP path can consume the very same input values.

Recipe (the pages fix only "Q, K, V drawn i.i.d. N(0,1) from a seed"):

* ``numpy.random.default_rng(seed)`` draws Q, then K, then V as float64
  ``standard_normal`` arrays of the full shape (the generator style of
  "Building a FlashAttention-2 Forward Kernel in Pure NumPy", Step 5).
* Q is multiplied by ``q_scale`` (4 for the peaky long-context workload;
  a power of two, so it commutes with rounding).
* The values are rounded to the storage dtype with round-to-nearest-even:
  float64 -> float32 for fp32; float64 -> float32 -> bfloat16 for bf16;
  float64 -> float16 for fp16.

Both sides receive the rounded values: the HIP path as device tensors of
the storage dtype, the oracle as the same values widened to float64.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Tuple

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "HEADLINE",
    "draw_float64",
    "round_to_dtype",
    "make_inputs",
    "make_p1_legacy_inputs",
    "make_dout",
    "conv_flops",
    "conv_flops_bwd",
    "algorithmic_bytes",
    "VarlenWorkload",
    "VARLEN_WORKLOADS",
    "make_varlen_inputs",
    "varlen_flops",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    D: int
    dtype: str  # "fp32" | "fp16" | "bf16"
    causal: bool
    seed: int
    q_scale: float = 1.0
    note: str = ""

    @property
    def q_shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.Nq, self.D)

    @property
    def kv_shape(self) -> Tuple[int, int, int, int]:
        return (self.B, self.H, self.Nk, self.D)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _w(*a, **kw) -> Workload:
    w = Workload(*a, **kw)
    return w


# The five measured workloads, then parity-only tail variants.
WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        _w("c1_fp32_causal_b2h4n128d64", 2, 4, 128, 128, 64, "fp32", True, 0,
           note="small causal case the oracle finishes in well under a second"),
        _w("c2_fp32_b1h8n1024d64", 1, 8, 1024, 1024, 64, "fp32", False, 1,
           note="non-causal; many K/V tiles exercise the online rescale"),
        _w("c3_bf16_causal_b4h16n4096d128", 4, 16, 4096, 4096, 128, "bf16", True, 2,
           note="headline: bf16 causal N=4096 D=128, fp32 accumulation"),
        _w("c4_bf16_causal_b1h32n16384d128_q4", 1, 32, 16384, 16384, 128, "bf16", True, 3,
           q_scale=4.0, note="long context; Q x4 gives peaky softmax rows"),
        _w("c5_fp16_cross_b8h32q512k8192d64", 8, 32, 512, 8192, 64, "fp16", False, 4,
           note="non-causal cross-attention, Nq != Nk"),
        # ragged tails (parity only)
        _w("c5t_fp16_cross_b8h32q511k8191d64", 8, 32, 511, 8191, 64, "fp16", False, 4,
           note="C5 with ragged Nq and Nk tails"),
        _w("c1t_fp32_causal_b1h2q77k131d64", 1, 2, 77, 131, 64, "fp32", True, 5,
           note="ragged, Nq != Nk, causal top-left"),
        _w("c1t_fp32_b1h2q77k131d64", 1, 2, 77, 131, 64, "fp32", False, 5,
           note="ragged, Nq != Nk, non-causal"),
        _w("c3t_bf16_causal_b1h3n1000d128", 1, 3, 1000, 1000, 128, "bf16", True, 6,
           note="bf16 D=128 causal with a ragged tail"),
        # head dimension 256 (the headline's FLOP count at twice the head size)
        _w("x1_bf16_causal_b4h8n4096d256", 4, 8, 4096, 4096, 256, "bf16", True, 10,
           note="head dimension 256, causal; 4 waves per workgroup, 32-key tiles in a 4-stage ring"),
        # decoding against a KV cache (split-KV path; HBM-bound)
        _w("d1_bf16_decode_b8h32q1k32768d128", 8, 32, 1, 32768, 128, "bf16", False, 7,
           note="one new query row per sequence against a 32K-key cache"),
        _w("d2_bf16_decode_b1h32q16k65536d128", 1, 32, 16, 65536, 128, "bf16", False, 8,
           note="16 query rows (a draft block) against a 64K-key cache, one sequence"),
    ]
}

HEADLINE = "c3_bf16_causal_b4h16n4096d128"


def draw_float64(w: Workload, seed: int | None = None):
    """Draw Q, K, V as float64 N(0,1) (Q times ``q_scale``), before rounding."""
    rng = np.random.default_rng(w.seed if seed is None else seed)
    q = rng.standard_normal(w.q_shape)
    k = rng.standard_normal(w.kv_shape)
    v = rng.standard_normal(w.kv_shape)
    if w.q_scale != 1.0:
        q *= w.q_scale
    return q, k, v


def round_to_dtype(x: np.ndarray, dtype: str):
    """Round a float64 array RNE to ``dtype``; returns a torch CPU tensor."""
    import torch

    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "fp16":
        return torch.from_numpy(np.ascontiguousarray(x.astype(np.float16)))
    if dtype == "bf16":
        # torch's float32 -> bfloat16 conversion rounds to nearest even.
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(w: Workload, seed: int | None = None):
    """Return (q, k, v) as contiguous torch CPU tensors of the storage dtype."""
    q, k, v = draw_float64(w, seed)
    return tuple(round_to_dtype(x, w.dtype) for x in (q, k, v))


def make_dout(w: Workload, seed: int | None = None):
    """The upstream gradient dO for a backward workload: float64 N(0,1) of
    Q's shape from its own generator (seed + 1000, drawn after nothing else),
    rounded to the storage dtype like Q, K, V."""
    rng = np.random.default_rng((w.seed if seed is None else seed) + 1000)
    return round_to_dtype(rng.standard_normal(w.q_shape), w.dtype)


def make_p1_legacy_inputs():
    """The worked example of "Build a FlashAttention Kernel from Scratch with
    Python and NumPy" (Step 2): legacy ``np.random.seed(0)`` and ``randn`` in
    Q, K, V order, shape (2, 4, 128, 64), float32."""
    import torch

    state = np.random.get_state()
    try:
        np.random.seed(0)
        arrs = [np.random.randn(2, 4, 128, 64).astype(np.float32) for _ in range(3)]
    finally:
        np.random.set_state(state)
    return tuple(torch.from_numpy(a) for a in arrs)


def conv_flops(B: int, H: int, Nq: int, Nk: int, D: int, causal: bool) -> float:
    """FLOP convention of the metric: 4*B*H*Nq*Nk*D, halved when causal."""
    f = 4.0 * B * H * Nq * Nk * D
    return f / 2.0 if causal else f


def conv_flops_bwd(B: int, H: int, Nq: int, Nk: int, D: int, causal: bool) -> float:
    """Backward FLOP convention: five products of the forward's size (S
    recomputed, dP = dO V^T, dV, dQ, dK), 10*B*H*Nq*Nk*D, halved when causal."""
    return 2.5 * conv_flops(B, H, Nq, Nk, D, causal)


def algorithmic_bytes(w: Workload) -> int:
    """Compulsory HBM bytes of one forward call: Q, K, V read once, O and
    LSE (fp32) written once."""
    esz = 4 if w.dtype == "fp32" else 2
    return (2 * w.B * w.H * w.Nq * w.D + 2 * w.B * w.H * w.Nk * w.D) * esz + 4 * w.B * w.H * w.Nq


@dataclasses.dataclass(frozen=True)
class VarlenWorkload:
    """Packed variable-length batch: sequence b has lens_q[b] query rows and
    lens_k[b] keys; q is [H, sum(lens_q), D], k and v [H, sum(lens_k), D]."""
    name: str
    H: int
    D: int
    dtype: str
    causal: bool
    seed: int
    lens_q: Tuple[int, ...]
    lens_k: Tuple[int, ...]

    @property
    def B(self) -> int:
        return len(self.lens_q)

    @property
    def cu_q(self):
        return np.concatenate([[0], np.cumsum(self.lens_q)]).astype(np.int32)

    @property
    def cu_k(self):
        return np.concatenate([[0], np.cumsum(self.lens_k)]).astype(np.int32)


def _mixed_lengths(seed: int, n: int, lo: int, hi: int):
    """n sequence lengths, log-uniform in [lo, hi] (a training batch packed
    without padding: many short sequences, a few long ones)."""
    r = np.random.default_rng(seed)
    return tuple(int(x) for x in np.exp(r.uniform(np.log(lo), np.log(hi), n)).round())


_V1 = _mixed_lengths(9, 16, 256, 8192)
VARLEN_WORKLOADS: Dict[str, VarlenWorkload] = {
    w.name: w
    for w in [
        VarlenWorkload("v1_bf16_causal_varlen_b16h16d128", 16, 128, "bf16", True, 9, _V1, _V1),
    ]
}


def make_varlen_inputs(w: VarlenWorkload, seed: int | None = None):
    """(q, k, v) as contiguous torch CPU tensors of the storage dtype, drawn
    like make_inputs (Q, then K, then V, float64 N(0,1), rounded), plus the
    int32 offset arrays (cu_q, cu_k)."""
    import torch

    rng = np.random.default_rng(w.seed if seed is None else seed)
    tq, tk = int(sum(w.lens_q)), int(sum(w.lens_k))
    q = rng.standard_normal((w.H, tq, w.D))
    k = rng.standard_normal((w.H, tk, w.D))
    v = rng.standard_normal((w.H, tk, w.D))
    ts = tuple(round_to_dtype(x, w.dtype) for x in (q, k, v))
    return ts + (torch.from_numpy(w.cu_q), torch.from_numpy(w.cu_k))


def varlen_flops(w: VarlenWorkload) -> float:
    """The FLOP convention per sequence (4*H*Nq*Nk*D, halved when causal), summed."""
    return float(sum(conv_flops(1, w.H, nq, nk, w.D, w.causal) for nq, nk in zip(w.lens_q, w.lens_k)))
