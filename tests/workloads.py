"""Seeded synthetic workloads for the attention forward.

Shared by the tests, the smoke check and the benchmark. It holds no attention
arithmetic: it only draws inputs. Neither the oracle nor the HIP path is
imported here.

Recipe (the pages name no dataset; the five shapes below are the workloads):
  * ``torch.Generator('cpu').manual_seed(seed)``; draw q, k, v in that order
    as float32 N(0, 1) tensors of shape [B, H, S, D];
  * "stress" workloads then scale 1% of sequence positions of q, and then of
    k, by 8, per (b, h) independently: ceil(0.01*S) positions chosen by a
    seeded ``randperm`` (q's draw first, then k's, looping b outer, h inner);
    the multiplication by 8 is exact, so it commutes with the later cast;
  * cast to the workload dtype (bf16: round-to-nearest-even) and return CPU
    tensors; the caller moves them to the device.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Tuple

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    H: int
    S: int
    D: int
    causal: Tuple[bool, ...]
    seed: int
    stress_rows: bool = False
    note: str = field(default="", compare=False)

    @property
    def scale(self) -> float:
        """float32(1/sqrt(D)), the value handed to the kernel."""
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    def flops(self, causal: bool) -> float:
        """Nominal attention flops 4*S^2*D*B*H, halved when causal."""
        f = 4.0 * self.S * self.S * self.D * self.B * self.H
        return f / 2 if causal else f


WORKLOADS: Dict[str, Workload] = {
    "c1_f32_causal_1x2x128x64": Workload(
        "c1_f32_causal_1x2x128x64", torch.float32, 1, 2, 128, 64, (True,), 1,
        note="fp32 parity case"),
    "c2_bf16_causal_4x16x1024x64": Workload(
        "c2_bf16_causal_4x16x1024x64", torch.bfloat16, 4, 16, 1024, 64, (True,), 2),
    "c3_bf16_2x16x4096x128": Workload(
        "c3_bf16_2x16x4096x128", torch.bfloat16, 2, 16, 4096, 128, (True, False), 3,
        note="run causal and non-causal on the same tensors"),
    "c4_bf16_causal_1x32x16384x128": Workload(
        "c4_bf16_causal_1x32x16384x128", torch.bfloat16, 1, 32, 16384, 128, (True,), 4,
        note="long sequence: many query tiles, causal tile skipping"),
    "c5_bf16_causal_2x8x8192x256_stress": Workload(
        "c5_bf16_causal_2x8x8192x256_stress", torch.bfloat16, 2, 8, 8192, 256, (True,), 5,
        stress_rows=True, note="1% of q and k rows scaled x8 (softmax rescale stress)"),
}

ORDER = list(WORKLOADS)


def stress_count(S: int) -> int:
    return int(math.ceil(0.01 * S))


def make_inputs(w: Workload, device: str = "cpu"
                ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Deterministic q, k, v for workload ``w`` (see the module docstring)."""
    return make_qkv(w.B, w.H, w.S, w.D, w.dtype, w.seed,
                    stress_rows=w.stress_rows, device=device)


def make_qkv(B: int, H: int, S: int, D: int, dtype: torch.dtype, seed: int,
             stress_rows: bool = False, device: str = "cpu"
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    g = torch.Generator("cpu").manual_seed(seed)
    shape = (B, H, S, D)
    q = torch.randn(shape, generator=g, dtype=torch.float32)
    k = torch.randn(shape, generator=g, dtype=torch.float32)
    v = torch.randn(shape, generator=g, dtype=torch.float32)
    if stress_rows and S > 0:
        n = stress_count(S)
        for t in (q, k):
            for b in range(B):
                for h in range(H):
                    idx = torch.randperm(S, generator=g)[:n]
                    t[b, h, idx] *= 8.0
    q, k, v = (t.to(dtype) for t in (q, k, v))
    if device != "cpu":
        q, k, v = (t.to(device) for t in (q, k, v))
    return q, k, v


# ---------------------------------------------------------------------------
# Queries against a key prefix and merges over key sets (measurement shapes)
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class PrefixWorkload:
    """Sq bf16 queries against Sk keys per (batch, head); the queries are the
    last Sq positions of the Sk-position sequence (chunked prefill, decode)."""
    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed: int

    @property
    def scale(self) -> float:
        return float(torch.tensor(1.0 / math.sqrt(self.D), dtype=torch.float32))

    def visible_pairs(self) -> int:
        """(query, key) pairs the mask keeps, per (batch, head)."""
        if not self.causal:
            return self.Sq * self.Sk
        shift = self.Sk - self.Sq
        return sum(max(0, min(self.Sk, i + shift + 1)) for i in range(self.Sq))

    def flops(self) -> float:
        """Nominal flops: 4*D per visible (query, key) pair."""
        return 4.0 * self.D * self.visible_pairs() * self.B * self.H

    def kv_bytes(self) -> int:
        return 2 * self.B * self.H * self.Sk * self.D * 2


PREFIX_WORKLOADS: Dict[str, PrefixWorkload] = {
    "prefill_bf16_causal_1x32_q2048_k16384_d128": PrefixWorkload(
        "prefill_bf16_causal_1x32_q2048_k16384_d128", 1, 32, 2048, 16384, 128, True, 11),
    "decode_bf16_causal_16x32_q1_k8192_d128": PrefixWorkload(
        "decode_bf16_causal_16x32_q1_k8192_d128", 16, 32, 1, 8192, 128, True, 12),
    # few heads, long prefix: the same K/V bytes on 128 heads
    "decode_bf16_causal_4x32_q1_k32768_d128": PrefixWorkload(
        "decode_bf16_causal_4x32_q1_k32768_d128", 4, 32, 1, 32768, 128, True, 13),
}


def make_prefix_inputs(w: PrefixWorkload, device: str = "cpu"):
    """q [B,H,Sq,D] from seed w.seed; k, v [B,H,Sk,D] from seed w.seed + 1000."""
    q = make_qkv(w.B, w.H, w.Sq, w.D, torch.bfloat16, w.seed, device=device)[0]
    _, k, v = make_qkv(w.B, w.H, w.Sk, w.D, torch.bfloat16, w.seed + 1000, device=device)
    return q, k, v


@dataclass(frozen=True)
class MergeWorkload:
    """G partial results (bf16 O, float32 LSE) of [B,H,S,D] to merge."""
    name: str
    G: int
    B: int
    H: int
    S: int
    D: int
    seed: int

    def bytes_moved(self) -> int:
        rows = self.B * self.H * self.S
        return self.G * rows * (self.D * 2 + 4) + rows * (self.D * 2 + 4)


MERGE_WORKLOADS: Dict[str, MergeWorkload] = {
    "merge_g4_1x32x16384x128": MergeWorkload("merge_g4_1x32x16384x128", 4, 1, 32, 16384, 128, 13),
}


def make_merge_inputs(w: MergeWorkload, device: str = "cpu"):
    """o_parts bf16 N(0,1) [G,B,H,S,D]; lse_parts float32 N(0,1)*4 [G,B,H,S]."""
    g = torch.Generator("cpu").manual_seed(w.seed)
    o = torch.randn((w.G, w.B, w.H, w.S, w.D), generator=g, dtype=torch.float32)
    l = torch.randn((w.G, w.B, w.H, w.S), generator=g, dtype=torch.float32) * 4.0
    return o.to(torch.bfloat16).to(device), l.to(device)
