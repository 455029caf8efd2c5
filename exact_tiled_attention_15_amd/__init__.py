"""Exact tiled attention forward on AMD MI355X (gfx950): Python binding.

A thin ctypes layer over the C ABI in ``include/fa.h`` (``libfa.so``, built
in-tree by ``exact_tiled_attention_15_amd.build``).  It only marshals
arguments: every step of the attention runs in the HIP kernels.  PyTorch is
used for device memory and the current stream.

There is no fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["fa_fwd", "fa_fwd_scaled", "fa_fwd_varlen", "forward_varlen", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size", "forward_splitkv",
           "fa_fwd_splitkv_static", "FA_STATIC_SCRATCH_BYTES",
           "fa_bwd", "fa_bwd_workspace_size", "backward", "fa_bwd_varlen", "backward_varlen", "fa_status_str", "forward", "load_library", "LIB_PATH",
           "FA_DTYPE_FP32", "FA_DTYPE_FP16", "FA_DTYPE_BF16", "FA_OK", "FA_DEFAULT_SCALE", "FaError",
           "EXPORTED_SYMBOLS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_DTYPE_FP32, FA_DTYPE_FP16, FA_DTYPE_BF16 = 0, 1, 2
FA_OK = 0
# softmax_scale value that makes the C entry points use 1/sqrt(D)
FA_DEFAULT_SCALE = 0.0
# device scratch of fa_fwd_splitkv_static (bytes, per device)
FA_STATIC_SCRATCH_BYTES = 32 * 1024 * 1024
EXPORTED_SYMBOLS = ("fa_fwd", "fa_fwd_scaled", "fa_fwd_varlen", "fa_fwd_splitkv", "fa_fwd_splitkv_workspace_size",
                    "fa_fwd_splitkv_static", "fa_bwd", "fa_bwd_workspace_size", "fa_bwd_varlen", "fa_status_str")

_lib = None


class FaError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        super().__init__(fa_status_str(status))


def load_library(path: str | None = None) -> ctypes.CDLL:
    """Load libfa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(
            f"{p} is missing: build it with `python -m exact_tiled_attention_15_amd.build` "
            "(there is no CPU fallback)")
    lib = ctypes.CDLL(p)
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_void_p] + [ctypes.c_int64] * 5 + \
        [ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_scaled.restype = ctypes.c_int
    lib.fa_fwd_scaled.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_varlen.restype = ctypes.c_int
    lib.fa_fwd_varlen.argtypes = [ctypes.c_void_p] * 7 + [ctypes.c_int64] * 6 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_splitkv_workspace_size.restype = ctypes.c_int64
    lib.fa_fwd_splitkv_workspace_size.argtypes = [ctypes.c_int64] * 6
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int64] * 6 + \
        [ctypes.c_double, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_fwd_splitkv_static.restype = ctypes.c_int
    lib.fa_fwd_splitkv_static.argtypes = [ctypes.c_void_p] * 5 + [ctypes.c_int64] * 5 + \
        [ctypes.c_double, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_bwd_workspace_size.restype = ctypes.c_int64
    lib.fa_bwd_workspace_size.argtypes = [ctypes.c_int64] * 3
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd.argtypes = [ctypes.c_void_p] * 10 + [ctypes.c_int64] * 6 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_bwd_varlen.restype = ctypes.c_int
    lib.fa_bwd_varlen.argtypes = [ctypes.c_void_p] * 12 + [ctypes.c_int64] * 8 + \
        [ctypes.c_double, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.fa_status_str.restype = ctypes.c_char_p
    lib.fa_status_str.argtypes = [ctypes.c_int]
    if path is None:
        _lib = lib
    return lib


def fa_status_str(status: int) -> str:
    return load_library().fa_status_str(int(status)).decode()


def fa_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int, D: int,
           causal: int, dtype: int, stream: int | None) -> int:
    """Call the C ``fa_fwd`` with raw device addresses; returns the status code."""
    return load_library().fa_fwd(q, k, v, o, lse, B, H, Nq, Nk, D, int(causal), int(dtype), stream)


def fa_fwd_scaled(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int,
                  D: int, softmax_scale: float, causal: int, dtype: int, stream: int | None) -> int:
    """Call the C ``fa_fwd_scaled`` with raw device addresses; returns the status code."""
    return load_library().fa_fwd_scaled(q, k, v, o, lse, B, H, Nq, Nk, D, float(softmax_scale),
                                        int(causal), int(dtype), stream)


def fa_fwd_varlen(q: int, k: int, v: int, o: int, lse: int, cu_q: int, cu_k: int, B: int, H: int, total_q: int,
                  total_k: int, max_seqlen_q: int, D: int, softmax_scale: float, causal: int, dtype: int,
                  stream: int | None) -> int:
    """Call the C ``fa_fwd_varlen`` with raw device addresses; returns the status code."""
    return load_library().fa_fwd_varlen(q, k, v, o, lse, cu_q, cu_k, B, H, total_q, total_k, max_seqlen_q, D,
                                        float(softmax_scale), int(causal), int(dtype), stream)


def fa_fwd_splitkv_workspace_size(B: int, H: int, Nq: int, Nk: int, D: int, num_splits: int) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits))


def fa_fwd_splitkv(q: int, k: int, v: int, o: int, lse: int, workspace: int, workspace_bytes: int, B: int,
                   H: int, Nq: int, Nk: int, D: int, softmax_scale: float, num_splits: int, causal: int,
                   dtype: int, stream: int | None) -> int:
    """Call the C ``fa_fwd_splitkv`` with raw device addresses; returns the status code."""
    return load_library().fa_fwd_splitkv(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, D,
                                         float(softmax_scale), int(num_splits), int(causal), int(dtype), stream)


def fa_fwd_splitkv_static(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, Nq: int, Nk: int, D: int,
                          softmax_scale: float, num_splits: int, causal: int, dtype: int,
                          stream: int | None) -> int:
    """Call the C ``fa_fwd_splitkv_static`` (split-KV with the library's static
    device scratch, no allocation) with raw device addresses; returns the
    status code."""
    return load_library().fa_fwd_splitkv_static(q, k, v, o, lse, B, H, Nq, Nk, D, float(softmax_scale),
                                                int(num_splits), int(causal), int(dtype), stream)


def fa_bwd_workspace_size(B: int, H: int, Nq: int) -> int:
    return int(load_library().fa_bwd_workspace_size(B, H, Nq))


def fa_bwd_varlen(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int, cu_q: int,
                  cu_k: int, workspace: int, workspace_bytes: int, B: int, H: int, total_q: int, total_k: int,
                  max_seqlen_q: int, max_seqlen_k: int, D: int, softmax_scale: float, causal: int, dtype: int,
                  stream: int | None) -> int:
    """Call the C ``fa_bwd_varlen`` with raw device addresses; returns the status code."""
    return load_library().fa_bwd_varlen(q, k, v, o, lse, dout, dq, dk, dv, cu_q, cu_k, workspace, workspace_bytes,
                                        B, H, total_q, total_k, max_seqlen_q, max_seqlen_k, D,
                                        float(softmax_scale), int(causal), int(dtype), stream)


def fa_bwd(q: int, k: int, v: int, o: int, lse: int, dout: int, dq: int, dk: int, dv: int,
           workspace: int, workspace_bytes: int, B: int, H: int, Nq: int, Nk: int, D: int,
           softmax_scale: float, causal: int, dtype: int, stream: int | None) -> int:
    """Call the C ``fa_bwd`` with raw device addresses; returns the status code."""
    return load_library().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                                 B, H, Nq, Nk, D, float(softmax_scale), int(causal), int(dtype), stream)


def _dtype_code(t) -> int:
    import torch

    codes = {torch.float32: FA_DTYPE_FP32, torch.float16: FA_DTYPE_FP16,
             torch.bfloat16: FA_DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _require(name, t, device, dtype=None, shape=None, dim=None):
    """Raise unless `t` is a contiguous GPU tensor on `device` (and, when
    given, of `dtype`, exactly `shape`, or `dim` dimensions).  Every tensor
    reaches the kernels as a raw device address, so these checks run before
    any C call."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}; every tensor must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name} must have {dim} dimensions, got shape {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _scale_arg(softmax_scale) -> float:
    return FA_DEFAULT_SCALE if softmax_scale is None else float(softmax_scale)


def _stream(device, stream):
    import torch

    if stream is not None:
        return stream
    with torch.cuda.device(device):
        return torch.cuda.current_stream().cuda_stream


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def forward(q, k, v, causal: bool = False, out=None, lse=None, stream=None, softmax_scale=None):
    """Exact attention forward on the GPU.

    q: (B, H, Nq, D), k/v: (B, H, Nk, D), contiguous device tensors of one
    dtype (float32, float16 or bfloat16), D in {32, 64, 128, 256} (256: 16-bit
    dtypes only).  Returns
    (O (B, H, Nq, D) in the input dtype, LSE (B, H, Nq) float32).  ``out`` and
    ``lse`` may be given preallocated; ``stream`` defaults to torch's current
    stream; ``softmax_scale`` (default 1/sqrt(D), chosen by the C library)
    multiplies q.k.
    """
    import torch

    _require("q", q, q.device if isinstance(q, torch.Tensor) else None, dim=4)
    dev, dt = q.device, q.dtype
    B, H, Nq, D = q.shape
    _require("k", k, dev, dt, dim=4)
    Nk = k.shape[2]
    _require("k", k, dev, dt, (B, H, Nk, D))
    _require("v", v, dev, dt, (B, H, Nk, D))
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    _require("out", out, dev, dt, (B, H, Nq, D))
    _require("lse", lse, dev, torch.float32, (B, H, Nq))
    code = _dtype_code(q)
    stream = _stream(dev, stream)
    with torch.cuda.device(dev):
        if softmax_scale is None:
            rc = fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, Nq, Nk, D, bool(causal), code, stream)
        else:
            rc = fa_fwd_scaled(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, Nq, Nk, D, float(softmax_scale), bool(causal), code, stream)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = False, softmax_scale=None, dq=None, dk=None,
             dv=None, workspace=None, stream=None):
    """Exact attention backward on the GPU.

    q, k, v, causal and softmax_scale as given to ``forward``; o and lse as it
    returned them; dout: the gradient of o (like q).  float32 (D <= 128),
    float16 or bfloat16.
    Returns (dq, dk, dv) in the input dtype.  Output tensors and the
    workspace (a device tensor of at least ``fa_bwd_workspace_size`` bytes)
    may be given preallocated.
    """
    import torch

    _require("q", q, q.device if isinstance(q, torch.Tensor) else None, dim=4)
    dev, dt = q.device, q.dtype
    B, H, Nq, D = q.shape
    _require("k", k, dev, dt, dim=4)
    Nk = k.shape[2]
    _require("k", k, dev, dt, (B, H, Nk, D))
    _require("v", v, dev, dt, (B, H, Nk, D))
    _require("o", o, dev, dt, (B, H, Nq, D))
    _require("lse", lse, dev, torch.float32, (B, H, Nq))
    _require("dout", dout, dev, dt, (B, H, Nq, D))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require("dq", dq, dev, dt, (B, H, Nq, D))
    _require("dk", dk, dev, dt, (B, H, Nk, D))
    _require("dv", dv, dev, dt, (B, H, Nk, D))
    need = fa_bwd_workspace_size(B, H, Nq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _require("workspace", workspace, dev)
    code = _dtype_code(q)
    stream = _stream(dev, stream)
    with torch.cuda.device(dev):
        rc = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
                    _nbytes(workspace), B, H, Nq, Nk, D, _scale_arg(softmax_scale), bool(causal), code, stream)
    if rc != FA_OK:
        raise FaError(rc)
    return dq, dk, dv


def forward_splitkv(q, k, v, causal: bool = False, num_splits: int = 0, softmax_scale=None, out=None, lse=None,
                    workspace=None, stream=None):
    """``forward`` computed with the keys split into ranges (decoding shape:
    few query rows, many keys).  Dtypes and head dimensions as ``forward``.  ``num_splits`` 0 picks
    the count automatically; ``workspace`` (a device tensor of at least
    ``fa_fwd_splitkv_workspace_size`` bytes) may be given preallocated."""
    import torch

    _require("q", q, q.device if isinstance(q, torch.Tensor) else None, dim=4)
    dev, dt = q.device, q.dtype
    B, H, Nq, D = q.shape
    _require("k", k, dev, dt, dim=4)
    Nk = k.shape[2]
    _require("k", k, dev, dt, (B, H, Nk, D))
    _require("v", v, dev, dt, (B, H, Nk, D))
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev) if lse is None else lse
    _require("out", out, dev, dt, (B, H, Nq, D))
    _require("lse", lse, dev, torch.float32, (B, H, Nq))
    with torch.cuda.device(dev):
        need = fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits)
    if need < 0:
        raise ValueError("invalid sizes or num_splits")
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _require("workspace", workspace, dev)
    code = _dtype_code(q)
    stream = _stream(dev, stream)
    with torch.cuda.device(dev):
        rc = fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            workspace.data_ptr(), _nbytes(workspace), B, H, Nq, Nk, D, _scale_arg(softmax_scale),
                            num_splits, bool(causal), code, stream)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def _check_offsets(cu_seqlens_q, cu_seqlens_k, dev):
    import torch

    _require("cu_seqlens_q", cu_seqlens_q, dev, torch.int32, dim=1)
    _require("cu_seqlens_k", cu_seqlens_k, dev, torch.int32, tuple(cu_seqlens_q.shape))
    if cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must hold B + 1 offsets each")
    return cu_seqlens_q.numel() - 1


def forward_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, causal: bool = False,
                   softmax_scale=None, out=None, lse=None, stream=None):
    """Attention over packed variable-length sequences (dtypes and head
    dimensions as ``forward``).

    q: (H, total_q, D), k/v: (H, total_k, D) contiguous GPU tensors (head-major
    packing); cu_seqlens_q / cu_seqlens_k: int32 GPU tensors of B + 1
    offsets; max_seqlen_q: the longest sequence's query count.  Returns
    (O (H, total_q, D), LSE (H, total_q) float32).
    """
    import torch

    _require("q", q, q.device if isinstance(q, torch.Tensor) else None, dim=3)
    dev, dt = q.device, q.dtype
    H, total_q, D = q.shape
    _require("k", k, dev, dt, dim=3)
    total_k = k.shape[1]
    _require("k", k, dev, dt, (H, total_k, D))
    _require("v", v, dev, dt, (H, total_k, D))
    B = _check_offsets(cu_seqlens_q, cu_seqlens_k, dev)
    out = torch.empty_like(q) if out is None else out
    lse = torch.empty((H, total_q), dtype=torch.float32, device=dev) if lse is None else lse
    _require("out", out, dev, dt, (H, total_q, D))
    _require("lse", lse, dev, torch.float32, (H, total_q))
    code = _dtype_code(q)
    stream = _stream(dev, stream)
    with torch.cuda.device(dev):
        rc = fa_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                           cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), B, H, total_q, total_k,
                           int(max_seqlen_q), D, _scale_arg(softmax_scale), bool(causal), code, stream)
    if rc != FA_OK:
        raise FaError(rc)
    return out, lse


def backward_varlen(q, k, v, o, lse, dout, cu_seqlens_q, cu_seqlens_k, max_seqlen_q: int, max_seqlen_k: int,
                    causal: bool = False, softmax_scale=None, dq=None, dk=None, dv=None, workspace=None,
                    stream=None):
    """Exact attention backward over packed variable-length sequences.

    q, o, dout: (H, total_q, D); k, v: (H, total_k, D); lse: (H, total_q)
    float32 as ``forward_varlen`` returned it; cu_seqlens_q / cu_seqlens_k:
    int32 device tensors of B + 1 offsets.  Returns (dq, dk, dv).
    """
    import torch

    _require("q", q, q.device if isinstance(q, torch.Tensor) else None, dim=3)
    dev, dt = q.device, q.dtype
    H, total_q, D = q.shape
    _require("k", k, dev, dt, dim=3)
    total_k = k.shape[1]
    _require("k", k, dev, dt, (H, total_k, D))
    _require("v", v, dev, dt, (H, total_k, D))
    _require("o", o, dev, dt, (H, total_q, D))
    _require("lse", lse, dev, torch.float32, (H, total_q))
    _require("dout", dout, dev, dt, (H, total_q, D))
    B = _check_offsets(cu_seqlens_q, cu_seqlens_k, dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _require("dq", dq, dev, dt, (H, total_q, D))
    _require("dk", dk, dev, dt, (H, total_k, D))
    _require("dv", dv, dev, dt, (H, total_k, D))
    need = fa_bwd_workspace_size(1, H, total_q)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _require("workspace", workspace, dev)
    code = _dtype_code(q)
    stream = _stream(dev, stream)
    with torch.cuda.device(dev):
        rc = fa_bwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                           dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), cu_seqlens_q.data_ptr(),
                           cu_seqlens_k.data_ptr(), workspace.data_ptr(), _nbytes(workspace), B, H, total_q,
                           total_k, int(max_seqlen_q), int(max_seqlen_k), D, _scale_arg(softmax_scale),
                           bool(causal), code, stream)
    if rc != FA_OK:
        raise FaError(rc)
    return dq, dk, dv
