"""Fused exact attention for MI355X (gfx950).

``forward(q, k, v, causal, scale)`` takes torch tensors of shape
[B, H, S, D] on the GPU (bf16 or float32, contiguous), allocates O and LSE with
torch, and calls the C ABI (``fa_fwd`` / ``fa_fwd_f32``) on torch's current
stream (or the stream passed).  ``forward_kv`` is the bf16 call with Sq queries
against Sk keys (``fa_fwd_kv``); ``merge`` combines results over disjoint key
sets (``fa_merge``); ``backward`` gives the gradients (``fa_bwd``).  torch only
provides device memory and the stream; the computation is entirely in the
library's HIP kernels.  Tensors allocated here are allocated on the stream the
kernels run on, so torch's caching allocator orders their reuse after them.
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
    FA_ERR_SCRATCH,
    FA_BWD_SCRATCH_ROWS,
    FA_ERR_SCALE,
    FA_ERR_SHAPE,
    FA_OK,
    LIB_PATH,
    FAError,
    fa_fwd,
    fa_bwd,
    fa_bwd_noalloc,
    fa_fwd_f32,
    fa_fwd_kv,
    fa_fwd_kv_plan,
    fa_fwd_plan,
    fa_merge,
    load,
    status_str,
)

__all__ = ["forward", "forward_kv", "merge", "backward", "fa_fwd", "fa_fwd_f32", "fa_fwd_kv",
           "fa_merge", "fa_bwd", "fa_bwd_noalloc", "fa_fwd_plan", "fa_fwd_kv_plan", "load", "status_str",
           "FAError"]


def _stream(stream, device):
    import torch
    return stream if stream is not None else torch.cuda.current_stream(device)


def _on_device(what: str, tensors, device) -> None:
    """Every tensor must live on `device` (a GPU): the kernels read and write
    them through plain device pointers."""
    for t in tensors:
        if not t.is_cuda or t.device != device:
            raise ValueError(f"{what} must be GPU tensors on {device} (got {t.device})")


def forward(q, k, v, causal: bool = True, scale: Optional[float] = None,
            out=None, lse=None, stream=None) -> Tuple[object, object]:
    """Attention forward on torch tensors; returns (O, LSE).

    q, k, v: [B, H, S, D] contiguous CUDA/HIP tensors, all bf16 or all float32.
    scale defaults to 1/sqrt(D).  ``out``/``lse`` may be passed preallocated
    ([B,H,S,D] in the input dtype, [B,H,S] float32).  ``stream`` is a torch
    stream (default: the current stream).
    """
    import torch

    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    _on_device("q, k, v", (k, v), q.device)
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
    s = _stream(stream, q.device)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    _on_device("out and lse", (out, lse), q.device)
    if out.dtype != q.dtype or tuple(out.shape) != (B, H, S, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B,H,S,D] tensor of the input dtype")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    fn = fa_fwd if q.dtype == torch.bfloat16 else fa_fwd_f32
    st = fn(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            B, H, S, D, int(bool(causal)), float(scale), s.cuda_stream)
    if st != FA_OK:
        raise FAError(st, fn.__name__)
    return out, lse


def forward_kv(q, k, v, causal: bool = True, scale: Optional[float] = None,
               out=None, lse=None, stream=None) -> Tuple[object, object]:
    """bf16 attention of q [B,H,Sq,D] against k, v [B,H,Sk,D] (causal mask
    aligned bottom-right: query i sees keys j <= i + Sk - Sq; rows with no
    visible key give O = 0, LSE = -inf).  Returns (O [B,H,Sq,D], LSE [B,H,Sq])."""
    import torch

    if not q.is_cuda:
        raise ValueError("q, k, v must be GPU tensors")
    _on_device("q, k, v", (k, v), q.device)
    if not (q.dtype == k.dtype == v.dtype == torch.bfloat16):
        raise ValueError("forward_kv takes bf16 q, k, v")
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B,H,Sq,D] and k, v one [B,H,Sk,D] shape")
    B, H, Sq, D = (int(x) for x in q.shape)
    if (int(k.shape[0]), int(k.shape[1]), int(k.shape[3])) != (B, H, D):
        raise ValueError("q and k, v must agree on B, H and D")
    Sk = int(k.shape[2])
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = _stream(stream, q.device)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    _on_device("out and lse", (out, lse), q.device)
    if out.dtype != q.dtype or tuple(out.shape) != (B, H, Sq, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [B,H,Sq,D] tensor")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,Sq] tensor")
    st = fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                   B, H, Sq, Sk, D, int(bool(causal)), float(scale), s.cuda_stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_kv")
    return out, lse


def merge(o_parts, lse_parts, out=None, lse=None, stream=None) -> Tuple[object, object]:
    """Merge G results over disjoint key sets: o_parts bf16 [G,B,H,S,D],
    lse_parts float32 [G,B,H,S] -> (O [B,H,S,D] bf16, LSE [B,H,S] float32)."""
    import torch

    if not o_parts.is_cuda:
        raise ValueError("o_parts and lse_parts must be GPU tensors")
    _on_device("o_parts and lse_parts", (lse_parts,), o_parts.device)
    if o_parts.dtype != torch.bfloat16 or lse_parts.dtype != torch.float32:
        raise ValueError("o_parts must be bf16 and lse_parts float32")
    if o_parts.dim() != 5 or tuple(lse_parts.shape) != tuple(o_parts.shape[:4]):
        raise ValueError("o_parts must be [G,B,H,S,D] and lse_parts [G,B,H,S]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    G, B, H, S, D = (int(x) for x in o_parts.shape)
    s = _stream(stream, o_parts.device)
    with torch.cuda.stream(s):
        if out is None:
            out = torch.empty((B, H, S, D), dtype=torch.bfloat16, device=o_parts.device)
        if lse is None:
            lse = torch.empty((B, H, S), dtype=torch.float32, device=o_parts.device)
    _on_device("out and lse", (out, lse), o_parts.device)
    if out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, S, D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bf16 [B,H,S,D] tensor")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, S) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 [B,H,S] tensor")
    st = fa_merge(o_parts.data_ptr(), lse_parts.data_ptr(), G, B, H, S, D, out.data_ptr(),
                  lse.data_ptr(), s.cuda_stream)
    if st != FA_OK:
        raise FAError(st, "fa_merge")
    return out, lse


def backward(q, k, v, o, lse, dout, causal: bool = True, scale: Optional[float] = None,
             stream=None) -> Tuple[object, object, object]:
    """Gradients (dq, dk, dv) of the bf16 forward for incoming gradient dout.

    q, k, v, o, dout: bf16 [B, H, S, D]; lse: float32 [B, H, S] (the forward's
    outputs o and lse, same causal and scale).  The Delta buffer the kernels
    need is allocated here with torch, on the stream the kernels run on, and
    released when the call returns (the allocator reuses it only after them)."""
    import torch

    ts = (q, k, v, o, dout)
    if not q.is_cuda:
        raise ValueError("inputs must be GPU tensors")
    _on_device("inputs", ts + (lse,), q.device)
    if not all(t.dtype == torch.bfloat16 for t in ts) or lse.dtype != torch.float32:
        raise ValueError("q, k, v, o, dout must be bf16 and lse float32")
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, o, dout must all be [B, H, S, D] of one shape")
    B, H, S, D = (int(x) for x in q.shape)
    if tuple(lse.shape) != (B, H, S):
        raise ValueError("lse must be [B, H, S]")
    if not all(t.is_contiguous() for t in ts + (lse,)):
        raise ValueError("inputs must be contiguous")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    s = _stream(stream, q.device)
    with torch.cuda.stream(s):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty((B, H, S), dtype=torch.float32, device=q.device)
    st = fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                B, H, S, D, int(bool(causal)), float(scale), s.cuda_stream)
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv
