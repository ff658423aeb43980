"""Fused exact attention forward for MI355X (gfx950).

``forward(q, k, v, causal, scale)`` takes torch tensors of shape
[B, H, S, D] on the GPU (bf16 or float32, contiguous), allocates O and LSE with
torch, and calls the C ABI (``fa_fwd`` / ``fa_fwd_f32``) on torch's current
stream.  torch only provides device memory and the stream; the computation is
entirely in the library's HIP kernels.
"""

from __future__ import annotations

import math
from typing import Optional, Tuple

from ._lib import (  # noqa: F401
    ABI_VERSION,
    EXPORTS,
    FA_ERR_ALIAS,
    FA_ERR_ALIGN,
    FA_ERR_CAUSAL,
    FA_ERR_HEADDIM,
    FA_ERR_LAUNCH,
    FA_ERR_NULL,
    FA_ERR_SCALE,
    FA_ERR_SHAPE,
    FA_OK,
    LIB_PATH,
    FAError,
    fa_fwd,
    fa_fwd_f32,
    fa_fwd_plan,
    load,
    status_str,
)

__all__ = ["forward", "fa_fwd", "fa_fwd_f32", "fa_fwd_plan", "load", "status_str", "FAError"]


def forward(q, k, v, causal: bool = True, scale: Optional[float] = None,
            out=None, lse=None, stream=None) -> Tuple[object, object]:
    """Attention forward on torch tensors; returns (O, LSE).

    q, k, v: [B, H, S, D] contiguous CUDA/HIP tensors, all bf16 or all float32.
    scale defaults to 1/sqrt(D).  ``out``/``lse`` may be passed preallocated
    ([B,H,S,D] in the input dtype, [B,H,S] float32).  ``stream`` is a torch
    stream (default: the current stream).
    """
    import torch

    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise ValueError("q, k, v must share one dtype")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(f"unsupported dtype {q.dtype} (bf16 or float32)")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must all be [B, H, S, D] of one shape")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    B, H, S, D = (int(x) for x in q.shape)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    if out.dtype != q.dtype or tuple(out.shape) != (B, H, S, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,H,S,D] tensor of the input dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, S, D, int(bool(causal)), float(scale), s.cuda_stream)
    if st != FA_OK:
        raise FAError(st, fn.__name__)
    return out, lse
