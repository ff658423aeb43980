"""Oracle for the attention backward pass (gradients of O with respect to q,
k and v).

TEST INFRASTRUCTURE ONLY. Nothing in the library imports, links or calls this
module; only the tests use it. It shares no code with the HIP path.

The pages do not describe the backward pass ("Profiling in PyTorch (Part 3):
Attention is all you profile" and the "FlashAttention-2" blog only say the
fused kernels serve training as well); this is the gradient of the forward
definition (matmul, scale, causal masked_fill, softmax, matmul; see
oracle/attention.py), written out with the chain rule, in float64 on the CPU
from the exact input values.

With S = scale * q k^T (masked entries -inf), P = softmax_rows(S), O = P v and
an incoming gradient dO of O:

    dv    = P^T dO                          (O = P v)
    dP    = dO v^T
    Delta = rowsum(dO * O)  (= rowsum(P * dP), since O = P v)
    dS    = P * (dP - Delta)                (softmax Jacobian, row by row)
    dq    = scale * dS k
    dk    = scale * dS^T q

Masked entries have P = 0, hence dS = 0: they contribute nothing.  P is
recomputed from the scores and the per-row LSE, P = exp(S - LSE), which is
the softmax of the row.  Pins: tests/test_oracle_backward.py.
"""

from __future__ import annotations

from typing import Optional, Tuple

import torch

from .attention import causal_keep_mask, default_scale

__all__ = ["attention_backward", "attention_delta"]


def _as_f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def attention_delta(o: torch.Tensor, do: torch.Tensor) -> torch.Tensor:
    """Delta_i = sum_d dO[i, d] * O[i, d]  ([B, H, S] float64)."""
    return (_as_f64(do) * _as_f64(o)).sum(dim=-1)


def attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, do: torch.Tensor,
                       causal: bool, scale: Optional[float] = None
                       ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """(dq, dk, dv) in float64 for q, k, v [B, H, S, D] and dO [B, H, S, D].

    Recomputes the forward (scores, P, O) from q, k, v in float64, then
    applies the formulas in the module docstring."""
    q64, k64, v64, do64 = (_as_f64(t) for t in (q, k, v, do))
    if scale is None:
        scale = default_scale(q64.shape[-1])
    s = torch.matmul(q64, k64.transpose(-2, -1)) * float(scale)
    if causal:
        keep = causal_keep_mask(q64.shape[-2], k64.shape[-2])
        s = s.masked_fill(~keep, float("-inf"))
    lse = torch.logsumexp(s, dim=-1, keepdim=True)
    p = torch.exp(s - lse)                                   # softmax rows
    o = torch.matmul(p, v64)
    dv = torch.matmul(p.transpose(-2, -1), do64)
    dp = torch.matmul(do64, v64.transpose(-2, -1))
    delta = (do64 * o).sum(dim=-1, keepdim=True)
    ds = p * (dp - delta)
    dq = torch.matmul(ds, k64) * float(scale)
    dk = torch.matmul(ds.transpose(-2, -1), q64) * float(scale)
    return dq, dk, dv
