"""Oracle for attention of Sq queries against Sk keys, and for merging
attention computed over disjoint key sets.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
module; only the tests and the benchmark's CPU-baseline leg use it. It shares
no code with the HIP path.

Queries against a key prefix (chunked prefill, decode).  The query block is
the last Sq positions of a sequence of Sk positions: query i sits at absolute
position i + (Sk - Sq).  With the causal mask, key j is visible to query i iff
j <= i + (Sk - Sq) ("bottom-right" alignment).  The keep-matrix is the same
ones-then-tril construction as in the "Math backend" section of "Profiling in
PyTorch (Part 3): Attention is all you profile", with the diagonal moved by
Sk - Sq; for Sq = Sk it is the plain lower triangle.  The pages do not treat
Sq != Sk: this alignment is the reading taken (it is the one under which a
block of queries appended to a cached prefix sees exactly what it would see
in the full sequence).

Fully masked rows.  With Sq > Sk (or a key set that lies entirely in a row's
future) a row can have no visible key.  The same "Math backend" section
describes the math path's safe softmax, which gives such rows zero weights
instead of NaN: the row of O is 0, and its LSE is log(0) = -inf.

Merging (split over keys).  Softmax over a union of disjoint key sets can be
assembled from the per-set results: with LSE_g and O_g computed over key set
g, LSE = log sum_g exp(LSE_g) and O = sum_g exp(LSE_g - LSE) O_g.  This is
what the per-row LSE output is for (not on the pages; it follows from the
definition of softmax).  Sets with LSE_g = -inf contribute nothing; if every
set is empty for a row, O = 0 and LSE = -inf.

Everything is float64 on the CPU from the exact input values.  Pins:
tests/test_oracle_prefix.py.
"""

from __future__ import annotations

from typing import Optional, Sequence, Tuple

import torch

from .attention import causal_keep_mask, default_scale

__all__ = ["prefix_keep_mask", "attention_prefix", "merge_reference"]


def _as_f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _keep(n_rows: int, s_q_total: int, s_k: int, row0: int) -> torch.Tensor:
    # Rows row0 .. row0+n_rows-1 of the [s_q_total, s_k] bottom-right keep
    # matrix: key j visible to query i iff j <= i + (s_k - s_q_total).
    return causal_keep_mask(n_rows, s_k, q_offset=(s_k - s_q_total) + row0)


def prefix_keep_mask(s_q: int, s_k: int, row0: int = 0) -> torch.Tensor:
    """Boolean [s_q - row0, s_k] rows ``row0..s_q-1`` of the bottom-right keep
    matrix of ``s_q`` queries against ``s_k`` keys: key j is visible to query
    i iff j <= i + (s_k - s_q)."""
    return _keep(s_q - row0, s_q, s_k, row0)


def _block(q64, k64, v64, causal, scale, s_q_total, row0):
    scores = torch.matmul(q64, k64.transpose(-2, -1)) * float(scale)
    if causal:
        keep = _keep(q64.shape[-2], s_q_total, k64.shape[-2], row0)
        scores = scores.masked_fill(~keep, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)                 # -inf on empty rows
    attn = torch.softmax(scores, dim=-1)                  # NaN on empty rows
    attn = torch.where(torch.isneginf(lse).unsqueeze(-1), torch.zeros_like(attn), attn)
    return torch.matmul(attn, v64), lse


def attention_prefix(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool,
                     scale: Optional[float] = None, row_block: Optional[int] = None
                     ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention of q [B,H,Sq,D] against k, v [B,H,Sk,D], causal mask aligned
    bottom-right, safe softmax on rows with no visible key.

    Returns (O [B,H,Sq,D], LSE [B,H,Sq]) in float64.  For Sq = Sk this is the
    same quantity as ``attention_reference``."""
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q64.shape[-1])
    s_q = q64.shape[-2]
    if row_block is None or row_block >= s_q:
        return _block(q64, k64, v64, causal, scale, s_q, 0)
    outs, lses = [], []
    for r0 in range(0, s_q, row_block):
        r1 = min(s_q, r0 + row_block)
        o, l = _block(q64[..., r0:r1, :], k64, v64, causal, scale, s_q, r0)
        outs.append(o)
        lses.append(l)
    return torch.cat(outs, dim=-2), torch.cat(lses, dim=-1)


def merge_reference(o_parts: Sequence[torch.Tensor] | torch.Tensor,
                    lse_parts: Sequence[torch.Tensor] | torch.Tensor
                    ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge G partial results computed over disjoint key sets.

    o_parts: G tensors [..., S, D] (or one [G, ..., S, D] tensor); lse_parts:
    G tensors [..., S] (natural-log LSE, -inf for rows that saw no key).
    Returns (O [..., S, D], LSE [..., S]) in float64:
    LSE = log sum_g exp(LSE_g), O = sum_g exp(LSE_g - LSE) O_g (0 where LSE = -inf).
    """
    o = torch.stack([_as_f64(t) for t in o_parts]) if not torch.is_tensor(o_parts) \
        else _as_f64(o_parts)
    l = torch.stack([_as_f64(t) for t in lse_parts]) if not torch.is_tensor(lse_parts) \
        else _as_f64(lse_parts)
    lse = torch.logsumexp(l, dim=0)
    w = torch.exp(l - lse.unsqueeze(0))                   # NaN where lse = -inf
    w = torch.where(torch.isneginf(lse).unsqueeze(0), torch.zeros_like(w), w)
    out = (w.unsqueeze(-1) * o).sum(dim=0)
    return out, lse
