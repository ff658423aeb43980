"""Oracle for the exact scaled-dot-product attention forward.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg
use it. It shares no code with the HIP path.

What it computes (all in float64 on the CPU, from the exact input values):

The definition is the five-step naive attention of "Profiling in PyTorch
(Part 3): Attention is all you profile", section "Naive attention" (the step
list and the ``NaiveCausalAttention`` module there):

  1. scores = q @ k^T                       (one matmul per (batch, head))
  2. scores = scores * scale                (scale = 1/sqrt(head_dim) by default)
  3. causal: scores[i, j] = -inf for j > i  (masked_fill with a boolean mask)
  4. attn = softmax(scores, dim=-1)         (the library softmax, max-subtracted)
  5. out = attn @ v

The mask direction follows the same page's "Math backend" section, where the
causal mask is built as a lower-triangular keep-matrix (ones, then tril): key j
is kept for query i iff j <= i.  (The "FlashAttention-2" blog's "Causal
Masking" paragraph states the condition with the comparison the other way
round; the tril construction is taken as authoritative.)

The per-row log-sum-exp is not on the pages; it is the natural-log
``LSE_i = log sum_j exp(scores_ij)`` over the unmasked keys of row i, with the
scale already applied, i.e. ``torch.logsumexp`` of the masked scores.

Layout: q, k, v are [batch, heads, seq, head_dim] (the layout comment in the
"Naive attention with in-place causal masking" listing of the same page);
O is [B, H, S, D] and LSE is [B, H, S].

Rows are independent, so evaluating the definition on a subset of query rows
(``rows=``) or in blocks of rows (``row_block=``) is still the definition, not
a reformulation: each row sees the same full set of keys.

Parity pins: every function here is pinned by tests/test_oracle.py against
closed forms, invariants, an independent pure-Python triple loop and the
library routine the pages call the reference implementation.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import torch

__all__ = [
    "default_scale",
    "causal_keep_mask",
    "attention_weights",
    "attention_reference",
    "attention_rows",
]


def default_scale(head_dim: int) -> float:
    """1/sqrt(head_dim), the scale of the ``NaiveCausalAttention`` module
    ("Profiling in PyTorch (Part 3)", section "Naive attention")."""
    return 1.0 / math.sqrt(head_dim)


def causal_keep_mask(s_q: int, s_k: int, q_offset: int = 0) -> torch.Tensor:
    """Boolean [s_q, s_k] matrix, True where key j is visible to query i.

    Built the way the "Math backend" section of "Profiling in PyTorch
    (Part 3)" describes SDPA building it: a ones matrix made lower triangular
    (tril).  ``q_offset`` shifts the query positions, so that a block of rows
    starting at absolute row ``q_offset`` sees keys j <= q_offset + i.
    """
    ones = torch.ones(s_q, s_k, dtype=torch.bool)
    return torch.tril(ones, diagonal=q_offset)


def _as_f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _scores(q: torch.Tensor, k: torch.Tensor, scale: float) -> torch.Tensor:
    # Steps 1 and 2 of the naive attention: matmul, then multiply by scale.
    scores = torch.matmul(q, k.transpose(-2, -1))
    return scores * float(scale)


def attention_weights(q: torch.Tensor, k: torch.Tensor, causal: bool,
                      scale: float) -> torch.Tensor:
    """Steps 1-4: the [B, H, S, S] softmax weights in float64.

    Only for small shapes (it materialises the full score matrix, which is
    exactly what the fused method avoids)."""
    q64, k64 = _as_f64(q), _as_f64(k)
    scores = _scores(q64, k64, scale)
    if causal:
        keep = causal_keep_mask(q64.shape[-2], k64.shape[-2])
        scores = scores.masked_fill(~keep, float("-inf"))
    return torch.softmax(scores, dim=-1)


def _rows_block(q64: torch.Tensor, k64: torch.Tensor, v64: torch.Tensor,
                causal: bool, scale: float, r0: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """The definition applied to query rows r0 .. r0+q64.shape[-2]-1."""
    scores = _scores(q64, k64, scale)                     # [..., rb, S]
    if causal:
        keep = causal_keep_mask(q64.shape[-2], k64.shape[-2], q_offset=r0)
        scores = scores.masked_fill(~keep, float("-inf"))  # step 3
    lse = torch.logsumexp(scores, dim=-1)                 # natural-log LSE
    attn = torch.softmax(scores, dim=-1)                  # step 4
    out = torch.matmul(attn, v64)                         # step 5
    return out, lse


def attention_reference(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                        causal: bool, scale: Optional[float] = None,
                        row_block: Optional[int] = None
                        ) -> Tuple[torch.Tensor, torch.Tensor]:
    """Full attention forward: returns (O [B,H,S,D], LSE [B,H,S]) in float64.

    q, k, v: [B, H, S, D] tensors of any floating dtype; they are widened to
    float64 exactly.  ``scale`` defaults to 1/sqrt(D); pass the float32 value
    a kernel receives to compare against that kernel.  ``row_block`` bounds
    the score matrix held at once to row_block x S per head.
    """
    q64, k64, v64 = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q64.shape[-1])
    S = q64.shape[-2]
    if row_block is None or row_block >= S:
        return _rows_block(q64, k64, v64, causal, scale, 0)
    outs, lses = [], []
    for r0 in range(0, S, row_block):
        r1 = min(S, r0 + row_block)
        o, l = _rows_block(q64[..., r0:r1, :], k64, v64, causal, scale, r0)
        outs.append(o)
        lses.append(l)
    return torch.cat(outs, dim=-2), torch.cat(lses, dim=-1)


def attention_rows(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                   causal: bool, scale: float, b: int, h: int,
                   rows: Sequence[int] | Iterable[int]
                   ) -> Tuple[torch.Tensor, torch.Tensor]:
    """The definition evaluated for selected query rows of one (b, h).

    Returns (O_rows [n, D], LSE_rows [n]) in float64, in the order of
    ``rows``.  Each row is the same computation as in ``attention_reference``
    (all keys of that head, masked to j <= i when causal); used to check
    full-size outputs one row at a time.
    """
    rows = [int(r) for r in rows]
    k64 = _as_f64(k[b, h])
    v64 = _as_f64(v[b, h])
    q64 = _as_f64(q[b, h, rows])                          # [n, D]
    scores = _scores(q64, k64, scale)                     # [n, S]
    if causal:
        j = torch.arange(k64.shape[0]).unsqueeze(0)
        i = torch.tensor(rows).unsqueeze(1)
        scores = scores.masked_fill(j > i, float("-inf"))
    lse = torch.logsumexp(scores, dim=-1)
    attn = torch.softmax(scores, dim=-1)
    return torch.matmul(attn, v64), lse
