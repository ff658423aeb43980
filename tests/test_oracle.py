"""Pins for the oracle (CPU only).

The oracle is the plain float64 definition of attention. These tests tie it to
things other than itself: a hand-worked example, closed forms, invariants, an
independent pure-Python triple loop, and the library routine the "Math
backend" section of "Profiling in PyTorch (Part 3)" calls the reference
implementation (PyTorch's scaled_dot_product_attention).

``PINS`` are written against an arbitrary attention callable so that
``test_pins_catch_planted_mistakes`` can run them on deliberately broken copies
of the oracle and show that each plausible mistake fails at least one pin.
"""

import json
import math
import os
import random

import pytest
import torch
import torch.nn.functional as F

from oracle import attention as orc
from tests import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, dtype=torch.float64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).to(dtype)


# ----------------------------------------------------------------------------
# Independent pure-Python implementation (loops, math.fsum, math.exp)
# ----------------------------------------------------------------------------

def brute_attention(q, k, v, causal, scale):
    """Triple loop over rows, keys and features with exact-ish sums."""
    B, H, S, D = q.shape
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    O = [[[[0.0] * D for _ in range(S)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * S for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(S):
                keys = [j for j in range(S) if (not causal or j <= i)]
                sc = [scale * math.fsum(ql[b][h][i][d] * kl[b][h][j][d] for d in range(D))
                      for j in keys]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                den = math.fsum(w)
                L[b][h][i] = mx + math.log(den)
                for d in range(D):
                    O[b][h][i][d] = math.fsum(w[t] * vl[b][h][j][d]
                                              for t, j in enumerate(keys)) / den
    return torch.tensor(O, dtype=torch.float64), torch.tensor(L, dtype=torch.float64)


# ----------------------------------------------------------------------------
# Pins, written against an attention callable  att(q, k, v, causal, scale)
# ----------------------------------------------------------------------------

def pin_hand_worked(att):
    with open(os.path.join(GOLDEN, "hand_worked_d1.json")) as f:
        g = json.load(f)
    q = torch.tensor(g["q"], dtype=torch.float64)
    k = torch.tensor(g["k"], dtype=torch.float64)
    v = torch.tensor(g["v"], dtype=torch.float64)
    ev = {"ln": math.log}
    for key, causal in (("non_causal", False), ("causal", True)):
        o, l = att(q, k, v, causal, g["scale"])
        want_o = [eval(e, ev) for e in g[key]["O"]]
        want_l = [eval(e, ev) for e in g[key]["LSE"]]
        assert torch.allclose(o[0, 0, :, 0], torch.tensor(want_o, dtype=torch.float64),
                              atol=1e-14, rtol=0), key
        assert torch.allclose(l[0, 0], torch.tensor(want_l, dtype=torch.float64),
                              atol=1e-14, rtol=0), key


def pin_brute_force(att):
    for seed, (B, H, S, D) in enumerate([(1, 1, 1, 1), (1, 2, 5, 3), (2, 1, 8, 4), (2, 2, 7, 2)]):
        q, k, v = (_rand((B, H, S, D), 100 + 3 * seed + t) for t in range(3))
        scale = 0.37 + 0.1 * seed
        for causal in (False, True):
            o, l = att(q, k, v, causal, scale)
            ob, lb = brute_attention(q, k, v, causal, scale)
            assert torch.allclose(o, ob, atol=1e-12, rtol=0), (B, H, S, D, causal)
            assert torch.allclose(l, lb, atol=1e-12, rtol=0), (B, H, S, D, causal)


def pin_library_sdpa(att):
    # PyTorch's SDPA math path on the CPU in float64: the "reference
    # implementation" role the Math-backend section gives it.
    q, k, v = (_rand((2, 3, 33, 16), 7 + t) for t in range(3))
    for causal in (False, True):
        for scale in (0.25, 1.0 / math.sqrt(16)):
            o, _ = att(q, k, v, causal, scale)
            ref = F.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale)
            assert torch.allclose(o, ref, atol=1e-12, rtol=0), (causal, scale)


def pin_constant_v(att):
    q, k = _rand((1, 2, 19, 8), 11), _rand((1, 2, 19, 8), 12)
    c = torch.linspace(-3, 5, 8, dtype=torch.float64)
    v = c.expand(1, 2, 19, 8).clone()
    for causal in (False, True):
        o, _ = att(q, k, v, causal, 0.5)
        assert torch.allclose(o, v, atol=1e-12, rtol=0)


def pin_causal_row0(att):
    q, k, v = (_rand((2, 2, 9, 5), 21 + t) for t in range(3))
    scale = 0.3
    o, l = att(q, k, v, True, scale)
    for b in range(2):
        for h in range(2):
            assert torch.allclose(o[b, h, 0], v[b, h, 0], atol=1e-14, rtol=0)
            s00 = scale * math.fsum(x * y for x, y in zip(q[b, h, 0].tolist(), k[b, h, 0].tolist()))
            assert abs(l[b, h, 0].item() - s00) < 1e-13


def pin_uniform_scores(att):
    S, D = 13, 6
    q, v = _rand((1, 1, S, D), 31), _rand((1, 1, S, D), 32)
    k = torch.zeros(1, 1, S, D, dtype=torch.float64)
    o, l = att(q, k, v, False, 0.7)
    mean = v[0, 0].sum(0) / S
    assert torch.allclose(o[0, 0], mean.expand(S, D), atol=1e-13, rtol=0)
    assert torch.allclose(l[0, 0], torch.full((S,), math.log(S), dtype=torch.float64), atol=1e-13)
    o, l = att(q, k, v, True, 0.7)
    for i in range(S):
        assert torch.allclose(o[0, 0, i], v[0, 0, : i + 1].sum(0) / (i + 1), atol=1e-13, rtol=0)
        assert abs(l[0, 0, i].item() - math.log(i + 1)) < 1e-13


def pin_one_hot(att):
    # Orthogonal keys (S <= D) and q_i = t * k_i: row i is dominated by key i.
    S, D, t, scale = 6, 8, 40.0, 0.5
    k = torch.zeros(1, 1, S, D, dtype=torch.float64)
    for i in range(S):
        k[0, 0, i, i] = 1.0 + 0.1 * i
    q = t * k
    v = _rand((1, 1, S, D), 41)
    o, l = att(q, k, v, False, scale)
    for i in range(S):
        s_ii = t * scale * (1.0 + 0.1 * i) ** 2
        # all other scores are exactly 0; LSE = log(e^{s_ii} + (S-1))
        assert abs(l[0, 0, i].item() - (s_ii + math.log1p((S - 1) * math.exp(-s_ii)))) < 1e-12
        assert torch.allclose(o[0, 0, i], v[0, 0, i], atol=1e-6, rtol=0)


def pin_causal_is_prefix(att):
    q, k, v = (_rand((1, 2, 11, 4), 51 + t) for t in range(3))
    oc, lc = att(q, k, v, True, 0.8)
    for i in range(11):
        on, ln = att(q[:, :, i:i + 1], k[:, :, : i + 1], v[:, :, : i + 1], False, 0.8)
        assert torch.allclose(oc[:, :, i], on[:, :, 0], atol=1e-13, rtol=0)
        assert torch.allclose(lc[:, :, i], ln[:, :, 0], atol=1e-13, rtol=0)


def pin_permutation(att):
    q, k, v = (_rand((1, 1, 10, 3), 61 + t) for t in range(3))
    perm = torch.randperm(10, generator=torch.Generator().manual_seed(5))
    o1, l1 = att(q, k, v, False, 1.1)
    o2, l2 = att(q, k[:, :, perm], v[:, :, perm], False, 1.1)
    assert torch.allclose(o1, o2, atol=1e-13, rtol=0)
    assert torch.allclose(l1, l2, atol=1e-13, rtol=0)


PINS = [pin_hand_worked, pin_brute_force, pin_library_sdpa, pin_constant_v,
        pin_causal_row0, pin_uniform_scores, pin_one_hot, pin_causal_is_prefix,
        pin_permutation]


def _oracle(q, k, v, causal, scale):
    return orc.attention_reference(q, k, v, causal, scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(_oracle)


# ----------------------------------------------------------------------------
# Planted mistakes: each broken copy of the oracle must fail at least one pin.
# ----------------------------------------------------------------------------

def _mut_mask_flipped(q, k, v, causal, scale):
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    if causal:
        keep = torch.triu(torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool))
        s = s.masked_fill(~keep, float("-inf"))
    return torch.softmax(s, -1) @ v, torch.logsumexp(s, -1)


def _mut_no_scale(q, k, v, causal, scale):
    return orc.attention_reference(q, k, v, causal, 1.0)


def _mut_mask_off_by_one(q, k, v, causal, scale):
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    if causal:
        keep = torch.tril(torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool), diagonal=-1)
        keep[..., 0, 0] = True
        s = s.masked_fill(~keep, float("-inf"))
    return torch.softmax(s, -1) @ v, torch.logsumexp(s, -1)


def _mut_softmax_wrong_dim(q, k, v, causal, scale):
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    if causal:
        keep = torch.tril(torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool))
        s = s.masked_fill(~keep, float("-inf"))
    return torch.nan_to_num(torch.softmax(s, -2)) @ v, torch.logsumexp(s, -1)


def _mut_lse_log2(q, k, v, causal, scale):
    o, l = orc.attention_reference(q, k, v, causal, scale)
    return o, l / math.log(2.0)


def _mut_v_transposed_keys(q, k, v, causal, scale):
    # uses v with its key order reversed (a wrong index into v)
    return orc.attention_reference(q, k, v.flip(-2), causal, scale)


def _mut_dropped_max_shift_lse(q, k, v, causal, scale):
    q64, k64, v64 = (t.to(torch.float64) for t in (q, k, v))
    s = (q64 @ k64.transpose(-2, -1)) * scale
    if causal:
        keep = torch.tril(torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool))
        s = s.masked_fill(~keep, float("-inf"))
    m = s.max(-1).values
    return torch.softmax(s, -1) @ v64, torch.log(torch.exp(s - m[..., None]).sum(-1))


MUTANTS = [_mut_mask_flipped, _mut_no_scale, _mut_mask_off_by_one, _mut_softmax_wrong_dim,
           _mut_lse_log2, _mut_v_transposed_keys, _mut_dropped_max_shift_lse]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda m: m.__name__)
def test_pins_catch_planted_mistakes(mutant):
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutant.__name__}"


# ----------------------------------------------------------------------------
# Consistency of the oracle's own entry points
# ----------------------------------------------------------------------------

def test_weights_rows_sum_to_one_and_masked_zero():
    q, k = _rand((2, 2, 17, 8), 71), _rand((2, 2, 17, 8), 72)
    for causal in (False, True):
        p = orc.attention_weights(q, k, causal, 0.35)
        assert torch.allclose(p.sum(-1), torch.ones(2, 2, 17, dtype=torch.float64), atol=1e-12)
        if causal:
            upper = torch.triu(torch.ones(17, 17, dtype=torch.bool), diagonal=1)
            assert (p[..., upper] == 0).all()
        assert (p >= 0).all()


def test_row_block_and_rows_match_full():
    q, k, v = (_rand((1, 2, 50, 8), 81 + t) for t in range(3))
    for causal in (False, True):
        o, l = orc.attention_reference(q, k, v, causal, 0.4)
        ob, lb = orc.attention_reference(q, k, v, causal, 0.4, row_block=7)
        assert torch.allclose(o, ob, atol=1e-13, rtol=0)
        assert torch.allclose(l, lb, atol=1e-13, rtol=0)
        rows = [0, 1, 6, 7, 31, 49]
        orow, lrow = orc.attention_rows(q, k, v, causal, 0.4, 0, 1, rows)
        assert torch.allclose(orow, o[0, 1, rows], atol=1e-13, rtol=0)
        assert torch.allclose(lrow, l[0, 1, rows], atol=1e-13, rtol=0)


def test_low_precision_inputs_are_widened_exactly():
    q, k, v = (_rand((1, 1, 9, 8), 91 + t).to(torch.bfloat16) for t in range(3))
    o1, l1 = orc.attention_reference(q, k, v, True, 0.125)
    o2, l2 = orc.attention_reference(q.double(), k.double(), v.double(), True, 0.125)
    assert o1.dtype == torch.float64
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_page_arithmetic_scores_per_head():
    with open(os.path.join(GOLDEN, "page_arithmetic.json")) as f:
        item = json.load(f)["items"][0]
    n = item["seq"] ** 2
    assert n == 16_777_216
    assert abs(n - item["scores_per_head_approx"]) / n < item["relative_tolerance"]


# ----------------------------------------------------------------------------
# The input generator (no attention arithmetic; checked for its recipe)
# ----------------------------------------------------------------------------

def test_generator_deterministic_and_dtypes():
    w = wl.WORKLOADS["c2_bf16_causal_4x16x1024x64"]
    small = wl.make_qkv(2, 2, 64, 64, torch.bfloat16, w.seed)
    again = wl.make_qkv(2, 2, 64, 64, torch.bfloat16, w.seed)
    for a, b in zip(small, again):
        assert a.dtype == torch.bfloat16 and torch.equal(a, b)


def test_generator_stress_rows():
    B, H, S, D = 2, 3, 500, 16
    plain = wl.make_qkv(B, H, S, D, torch.float32, 5, stress_rows=False)
    stress = wl.make_qkv(B, H, S, D, torch.float32, 5, stress_rows=True)
    n = wl.stress_count(S)
    assert n == 5
    for t_plain, t_stress in zip(plain[:2], stress[:2]):
        ratio = (t_stress / t_plain)
        for b in range(B):
            for h in range(H):
                rows8 = (ratio[b, h] == 8).all(-1)
                rows1 = (ratio[b, h] == 1).all(-1)
                assert int(rows8.sum()) == n and int(rows1.sum()) == S - n
    assert torch.equal(plain[2], stress[2])  # v untouched


def test_generator_statistics_sane():
    # q,k ~ N(0,1), scale 1/sqrt(D): scores ~ N(0,1), so LSE_i ~ ln(n_i) + 1/2.
    q, k, v = wl.make_qkv(1, 2, 512, 64, torch.float32, 3)
    _, l = orc.attention_reference(q, k, v, False, 1 / 8)
    assert abs(l.mean().item() - (math.log(512) + 0.5)) < 0.1


def test_default_scale_closed_forms():
    # 1/sqrt(head_dim) is a power of two at D = 64 and D = 256, and at D = 128
    # its square times D is 1; a call without a scale uses it
    assert orc.default_scale(64) == 0.125
    assert orc.default_scale(256) == 0.0625
    assert abs(orc.default_scale(128) ** 2 * 128 - 1.0) < 1e-15
    g = torch.Generator().manual_seed(3)
    q, k, v = (torch.randn((1, 2, 9, 64), generator=g, dtype=torch.float64) for _ in range(3))
    o_default, l_default = orc.attention_reference(q, k, v, True)
    o_eighth, l_eighth = orc.attention_reference(q, k, v, True, 0.125)
    assert torch.equal(o_default, o_eighth) and torch.equal(l_default, l_eighth)


def test_zero_scale_closed_form():
    # scale = 0: every score is 0, so each row's softmax is uniform over its
    # visible keys: O = mean of those v rows, LSE = log(count).
    g = torch.Generator().manual_seed(91)
    B, H, S, D = 1, 2, 9, 8
    q, k, v = (torch.randn(B, H, S, D, generator=g, dtype=torch.float64) for _ in range(3))
    for causal in (False, True):
        o, lse = orc.attention_reference(q, k, v, causal, 0.0)
        for i in range(S):
            n = i + 1 if causal else S
            assert torch.allclose(o[..., i, :], v[..., :n, :].mean(dim=-2), rtol=0, atol=1e-14)
            assert torch.allclose(lse[..., i], torch.full((B, H), math.log(n), dtype=torch.float64),
                                  rtol=0, atol=1e-14)


def test_negative_scale_is_the_positive_one_on_negated_queries():
    # scale * q.k = (-scale) * (-q).k: the oracle must use the scale's sign
    # (a dropped sign, |scale|, fails this for a non-symmetric input).
    g = torch.Generator().manual_seed(92)
    q, k, v = (torch.randn(1, 2, 17, 16, generator=g, dtype=torch.float64) for _ in range(3))
    for causal in (False, True):
        o1, l1 = orc.attention_reference(q, k, v, causal, -0.3)
        o2, l2 = orc.attention_reference(-q, k, v, causal, 0.3)
        o3, _ = orc.attention_reference(q, k, v, causal, 0.3)
        assert torch.allclose(o1, o2, rtol=0, atol=1e-13) and torch.allclose(l1, l2, rtol=0, atol=1e-13)
        assert (o1 - o3).abs().max().item() > 1e-3
