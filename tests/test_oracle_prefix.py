"""Pins for the Sq != Sk oracle and the split-over-keys merge (CPU only).

``attention_prefix`` (queries that are the last Sq positions of an Sk-long
sequence; causal mask aligned bottom-right; safe softmax on rows with no
visible key) and ``merge_reference`` (LSE-weighted merge of results over
disjoint key sets) are tied to things other than themselves:

- the already-pinned square oracle, through facts that must hold whatever
  the implementation: a block of queries appended to a prefix sees exactly
  what the same rows see in the full sequence; a single query sees every key;
  with more queries than keys the first Sq - Sk rows see nothing;
- an independent pure-Python loop implementing the stated rule;
- the merge identity: attention over a key set assembled from attention over
  its parts, for non-causal partitions and for the split a chunked prefill
  makes (cached prefix, then the chunk itself).

Pins are written against callables, and broken copies of both functions must
each fail at least one of them.
"""

import math

import pytest
import torch

from oracle import attention as orc
from oracle import prefix as pre


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def _close(a, b, tol=1e-12):
    assert a.shape == b.shape, (a.shape, b.shape)
    fin = torch.isfinite(b)
    assert torch.equal(torch.isfinite(a), fin) and torch.equal(a[~fin], b[~fin]), "non-finite mismatch"
    err = (a[fin] - b[fin]).abs().max().item() if fin.any() else 0.0
    assert err <= tol, err


# ----------------------------------------------------------------------------
# Independent pure-Python implementation of the stated rule
# ----------------------------------------------------------------------------

def brute_prefix(q, k, v, causal, scale):
    B, H, Sq, D = q.shape
    Sk = k.shape[-2]
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    O = [[[[0.0] * D for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                pos = i + (Sk - Sq)               # absolute position of query i
                keys = [j for j in range(Sk) if (not causal or j <= pos)]
                if not keys:
                    L[b][h][i] = -math.inf        # O row stays 0
                    continue
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
# Pins of the attention function  att(q, k, v, causal, scale)
# ----------------------------------------------------------------------------

def pin_square_is_reference(att):
    for causal in (False, True):
        q, k, v = (_rand((2, 2, 9, 4), s) for s in (1, 2, 3))
        o, l = att(q, k, v, causal, 0.4)
        o_r, l_r = orc.attention_reference(q, k, v, causal, 0.4)
        _close(o, o_r)
        _close(l, l_r)


def pin_chunk_rows_are_tail_of_full_sequence(att):
    S = 23
    q, k, v = (_rand((1, 2, S, 5), s) for s in (4, 5, 6))
    o_full, l_full = orc.attention_reference(q, k, v, True, 0.3)
    for sq in (1, 2, 7, 16, 22):
        o, l = att(q[..., S - sq:, :], k, v, True, 0.3)
        _close(o, o_full[..., S - sq:, :])
        _close(l, l_full[..., S - sq:])


def pin_single_query_sees_every_key(att):
    q = _rand((2, 1, 1, 6), 7)
    k, v = _rand((2, 1, 19, 6), 8), _rand((2, 1, 19, 6), 9)
    o_c, l_c = att(q, k, v, True, 0.5)
    o_n, l_n = att(q, k, v, False, 0.5)
    _close(o_c, o_n)
    _close(l_c, l_n)
    s = (q @ k.transpose(-2, -1)).squeeze(-2) * 0.5          # [2, 1, 19]
    _close(l_n[..., 0], torch.logsumexp(s, -1), 1e-12)


def pin_more_queries_than_keys(att):
    Sq, Sk = 20, 7
    q = _rand((1, 2, Sq, 4), 10)
    k, v = _rand((1, 2, Sk, 4), 11), _rand((1, 2, Sk, 4), 12)
    o, l = att(q, k, v, True, 0.6)
    empty = Sq - Sk
    assert torch.all(o[..., :empty, :] == 0.0)
    assert torch.all(torch.isneginf(l[..., :empty]))
    o_r, l_r = orc.attention_reference(q[..., empty:, :], k, v, True, 0.6)
    _close(o[..., empty:, :], o_r)
    _close(l[..., empty:], l_r)
    # without the mask every row sees all keys
    o_n, _ = att(q, k, v, False, 0.6)
    assert torch.isfinite(o_n).all() and (o_n[..., :empty, :] != 0).any()


def pin_brute_force(att):
    for sq, sk in ((1, 5), (3, 5), (5, 3), (4, 4), (6, 2), (2, 7)):
        q = _rand((1, 2, sq, 3), 20 + sq)
        k, v = _rand((1, 2, sk, 3), 30 + sk), _rand((1, 2, sk, 3), 40 + sk)
        for causal in (False, True):
            o, l = att(q, k, v, causal, 0.7)
            o_b, l_b = brute_prefix(q, k, v, causal, 0.7)
            _close(o, o_b, 1e-12)
            _close(l, l_b, 1e-12)


PINS = [pin_square_is_reference, pin_chunk_rows_are_tail_of_full_sequence,
        pin_single_query_sees_every_key, pin_more_queries_than_keys, pin_brute_force]


def _att(q, k, v, causal, scale):
    return pre.attention_prefix(q, k, v, causal, scale)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_prefix_oracle_pin(pin):
    pin(_att)


def test_row_blocks_match_whole():
    q = _rand((1, 2, 37, 4), 50)
    k, v = _rand((1, 2, 50, 4), 51), _rand((1, 2, 50, 4), 52)
    for causal in (False, True):
        o, l = pre.attention_prefix(q, k, v, causal, 0.5)
        o_b, l_b = pre.attention_prefix(q, k, v, causal, 0.5, row_block=8)
        _close(o_b, o)
        _close(l_b, l)
    q2 = _rand((1, 1, 30, 4), 53)                 # more queries than keys, blocked
    o, l = pre.attention_prefix(q2, k[:, :1, :12], v[:, :1, :12], True, 0.5)
    o_b, l_b = pre.attention_prefix(q2, k[:, :1, :12], v[:, :1, :12], True, 0.5, row_block=7)
    _close(o_b, o)
    _close(l_b, l)


# ----------------------------------------------------------------------------
# Pins of the merge  merge(o_parts, lse_parts)
# ----------------------------------------------------------------------------

def pin_merge_key_partition(merge):
    q = _rand((2, 2, 11, 5), 60)
    k, v = _rand((2, 2, 29, 5), 61), _rand((2, 2, 29, 5), 62)
    o_full, l_full = pre.attention_prefix(q, k, v, False, 0.45)
    for cuts in ((0, 29), (0, 10, 29), (0, 1, 13, 14, 29), (0, 5, 9, 20, 27, 29)):
        parts = [pre.attention_prefix(q, k[..., a:b, :], v[..., a:b, :], False, 0.45)
                 for a, b in zip(cuts[:-1], cuts[1:])]
        o, l = merge([p[0] for p in parts], [p[1] for p in parts])
        _close(o, o_full, 1e-12)
        _close(l, l_full, 1e-12)


def pin_merge_chunked_prefill_split(merge):
    # A chunk of Sq queries appended to a cached prefix of P keys: the prefix
    # is visible to every query of the chunk, the chunk itself causally.
    P, Sq = 17, 9
    q = _rand((1, 3, Sq, 4), 70)
    k, v = _rand((1, 3, P + Sq, 4), 71), _rand((1, 3, P + Sq, 4), 72)
    o_full, l_full = pre.attention_prefix(q, k, v, True, 0.55)
    o1, l1 = pre.attention_prefix(q, k[..., :P, :], v[..., :P, :], False, 0.55)
    o2, l2 = pre.attention_prefix(q, k[..., P:, :], v[..., P:, :], True, 0.55)
    o, l = merge([o1, o2], [l1, l2])
    _close(o, o_full, 1e-12)
    _close(l, l_full, 1e-12)


def pin_merge_empty_parts(merge):
    o1, l1 = _rand((2, 3, 4), 80), _rand((2, 3), 81)
    junk = _rand((2, 3, 4), 82)
    empty = torch.full((2, 3), -math.inf, dtype=torch.float64)
    o, l = merge([o1, junk], [l1, empty])          # an empty part changes nothing
    _close(o, o1, 1e-14)
    _close(l, l1, 1e-14)
    o, l = merge([o1], [l1])                       # one part: identity
    _close(o, o1, 1e-14)
    o, l = merge([junk, junk], [empty, empty])     # nothing visible: 0 and -inf
    assert torch.all(o == 0) and torch.all(torch.isneginf(l))


def pin_merge_weights_closed_form(merge):
    # two parts with LSE a and b: weights e^a/(e^a+e^b), e^b/(e^a+e^b)
    a, b = 0.3, -1.7
    o1 = torch.full((1, 1, 2), 2.0, dtype=torch.float64)
    o2 = torch.full((1, 1, 2), -1.0, dtype=torch.float64)
    la = torch.full((1, 1), a, dtype=torch.float64)
    lb = torch.full((1, 1), b, dtype=torch.float64)
    o, l = merge([o1, o2], [la, lb])
    wa = math.exp(a) / (math.exp(a) + math.exp(b))
    _close(o, torch.full((1, 1, 2), 2.0 * wa - (1 - wa), dtype=torch.float64), 1e-14)
    _close(l, torch.full((1, 1), math.log(math.exp(a) + math.exp(b)), dtype=torch.float64), 1e-14)


MERGE_PINS = [pin_merge_key_partition, pin_merge_chunked_prefill_split, pin_merge_empty_parts,
              pin_merge_weights_closed_form]


@pytest.mark.parametrize("pin", MERGE_PINS, ids=lambda p: p.__name__)
def test_merge_oracle_pin(pin):
    pin(pre.merge_reference)


def test_merge_accepts_stacked_parts():
    o = _rand((3, 2, 5, 4), 90)
    l = _rand((3, 2, 5), 91)
    a = pre.merge_reference(o, l)
    b = pre.merge_reference(list(o), list(l))
    _close(a[0], b[0], 0.0)
    _close(a[1], b[1], 0.0)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _mut_top_left(q, k, v, causal, scale):
    # causal mask aligned top-left (key j visible iff j <= i)
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    if causal:
        s = s.masked_fill(~torch.tril(torch.ones(s.shape[-2], s.shape[-1], dtype=torch.bool)),
                          float("-inf"))
    l = torch.logsumexp(s, -1)
    w = torch.nan_to_num(torch.softmax(s, -1))
    return w @ v, l


def _mut_diagonal_off_by_one(q, k, v, causal, scale):
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    sq, sk = s.shape[-2], s.shape[-1]
    if causal:
        keep = torch.tril(torch.ones(sq, sk, dtype=torch.bool), diagonal=sk - sq - 1)
        s = s.masked_fill(~keep, float("-inf"))
    l = torch.logsumexp(s, -1)
    w = torch.nan_to_num(torch.softmax(s, -1))
    return w @ v, l


def _mut_unsafe_softmax(q, k, v, causal, scale):
    # no special case for rows without a visible key (NaN rows)
    q, k, v = (t.to(torch.float64) for t in (q, k, v))
    s = (q @ k.transpose(-2, -1)) * scale
    sq, sk = s.shape[-2], s.shape[-1]
    if causal:
        keep = torch.tril(torch.ones(sq, sk, dtype=torch.bool), diagonal=sk - sq)
        s = s.masked_fill(~keep, float("-inf"))
    return torch.softmax(s, -1) @ v, torch.logsumexp(s, -1)


def _mut_empty_rows_uniform(q, k, v, causal, scale):
    # rows without a visible key averaged over all keys instead of 0
    o, l = pre.attention_prefix(q, k, v, causal, scale)
    empty = torch.isneginf(l)
    if empty.any():
        mean_v = v.to(torch.float64).mean(-2, keepdim=True).expand_as(o)
        o = torch.where(empty.unsqueeze(-1), mean_v, o)
    return o, l


def _mut_merge_unnormalised(o_parts, lse_parts):
    o = torch.stack([t.to(torch.float64) for t in o_parts])
    l = torch.stack([t.to(torch.float64) for t in lse_parts])
    w = torch.nan_to_num(torch.exp(l), nan=0.0)
    return (w.unsqueeze(-1) * o).sum(0), torch.logsumexp(l, 0)


def _mut_merge_max_instead_of_logsumexp(o_parts, lse_parts):
    o = torch.stack([t.to(torch.float64) for t in o_parts])
    l = torch.stack([t.to(torch.float64) for t in lse_parts])
    lse = l.max(0).values
    w = torch.nan_to_num(torch.exp(l - lse), nan=0.0)
    w = w / w.sum(0).clamp_min(1e-300)
    return (w.unsqueeze(-1) * o).sum(0), lse


def _mut_merge_plain_mean(o_parts, lse_parts):
    o = torch.stack([t.to(torch.float64) for t in o_parts])
    l = torch.stack([t.to(torch.float64) for t in lse_parts])
    return o.mean(0), torch.logsumexp(l, 0)


@pytest.mark.parametrize("mutant", [_mut_top_left, _mut_diagonal_off_by_one, _mut_unsafe_softmax,
                                    _mut_empty_rows_uniform], ids=lambda m: m.__name__)
def test_prefix_pins_catch_planted_mistakes(mutant):
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutant.__name__}"


@pytest.mark.parametrize("mutant", [_mut_merge_unnormalised, _mut_merge_max_instead_of_logsumexp,
                                    _mut_merge_plain_mean], ids=lambda m: m.__name__)
def test_merge_pins_catch_planted_mistakes(mutant):
    failed = []
    for pin in MERGE_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutant.__name__}"


def test_workload_visible_pairs_match_the_mask():
    from tests import workloads as wl
    for sq, sk in ((1, 9), (5, 9), (9, 9), (12, 5), (7, 1)):
        for causal in (False, True):
            w = wl.PrefixWorkload("t", 1, 1, sq, sk, 64, causal, 0)
            keep = pre.prefix_keep_mask(sq, sk) if causal else torch.ones(sq, sk, dtype=torch.bool)
            assert w.visible_pairs() == int(keep.sum())
