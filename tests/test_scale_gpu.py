"""GPU parity for negative and zero scales, through the C ABI.

The boundary accepts any finite scale.  A negative scale is computed as
|scale| on negated queries (forward, dQ) or keys (dK/dV): a sign-bit flip of a
register fragment, which is exact, so the results must equal those of the
positive scale on -q bit for bit (the gradient with respect to q changes sign;
dK, summed over the negated q, agrees to one bf16 ulp).  A zero scale gives every visible key weight 1: O is
the mean of the visible v rows and LSE the log of their count; dq = dk = 0.

Each case is also checked against the float64 oracle (oracle/attention.py,
oracle/prefix.py, oracle/backward.py) to the tolerances of the positive-scale
tests."""

import math
import sys

import pytest
import torch

import exact_attention_67_amd as fa
from oracle import attention as orc
from oracle import backward as bwd
from oracle import prefix as pre
from tests import workloads as wl
from tests.test_backward_gpu import check_grads
from tests.test_parity_gpu import check
from tests.test_prefix_gpu import check as check_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _f32(x):
    return float(torch.tensor(x, dtype=torch.float32))


SCALES = [("neg", lambda D: _f32(-1 / math.sqrt(D))), ("neg_large", lambda D: -0.5),
          ("zero", lambda D: 0.0), ("negzero", lambda D: -0.0)]


@pytest.mark.parametrize("tag,mk", SCALES, ids=[t for t, _ in SCALES])
@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [True, False])
def test_forward_bf16_matches_oracle(tag, mk, D, causal):
    scale = mk(D)
    q, k, v = wl.make_qkv(1, 3, 333, D, torch.bfloat16, seed=8100 + D)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
    check(o.cpu(), lse.cpu(), o_ref, l_ref, torch.bfloat16,
          f"bf16 scale={scale} D={D} causal={causal}")


@pytest.mark.parametrize("tag,mk", SCALES[:3], ids=[t for t, _ in SCALES[:3]])
@pytest.mark.parametrize("D", [64, 128])
def test_forward_f32_matches_oracle(tag, mk, D):
    scale = mk(D)
    q, k, v = wl.make_qkv(1, 2, 200, D, torch.float32, seed=8200 + D)
    o, lse = fa.forward(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = orc.attention_reference(q, k, v, True, scale)
    check(o.cpu(), lse.cpu(), o_ref, l_ref, torch.float32, f"f32 scale={scale} D={D}")


# B, H, S, D, causal: 128-row and 256-row workgroups, the D = 256 wave-pair kernel
FLIP_SHAPES = [(1, 3, 333, 128, True), (2, 32, 1000, 128, True), (1, 32, 2048, 128, False),
               (2, 2, 777, 64, True), (1, 4, 600, 256, True)]


@pytest.mark.parametrize("B,H,S,D,causal", FLIP_SHAPES,
                         ids=[f"B{B}-H{H}-S{S}-D{D}-{'c' if c else 'n'}"
                              for B, H, S, D, c in FLIP_SHAPES])
def test_forward_negative_scale_is_positive_on_negated_q(B, H, S, D, causal):
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=8300 + S))
    s = _f32(1 / math.sqrt(D))
    o1, l1 = fa.forward(q, k, v, causal=causal, scale=-s)
    o2, l2 = fa.forward(-q, k, v, causal=causal, scale=s)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("tag,mk", SCALES[:3], ids=[t for t, _ in SCALES[:3]])
@pytest.mark.parametrize("Sq,Sk", [(40, 300), (300, 120)])
def test_forward_kv_matches_oracle(tag, mk, Sq, Sk):
    D = 128
    scale = mk(D)
    q = wl.make_qkv(1, 2, Sq, D, torch.bfloat16, seed=8400)[0]
    _, k, v = wl.make_qkv(1, 2, Sk, D, torch.bfloat16, seed=8401)
    o, lse = fa.forward_kv(q.cuda(), k.cuda(), v.cuda(), causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref, l_ref = pre.attention_prefix(q, k, v, True, scale)
    check_kv(o, lse, o_ref, l_ref, f"kv scale={scale} Sq={Sq} Sk={Sk}")


def _dout(B, H, S, D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, H, S, D), generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("tag,mk", SCALES[:3], ids=[t for t, _ in SCALES[:3]])
@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_matches_oracle(tag, mk, D):
    scale = mk(D)
    B, H, S = 1, 2, 200
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=8500 + D)
    do = _dout(B, H, S, D, 8600 + D)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=True, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=True, scale=scale)
    torch.cuda.synchronize()
    ref = bwd.attention_backward(q, k, v, do, True, scale)
    if scale == 0.0:  # the gradients through the scores vanish exactly
        assert torch.count_nonzero(dq) == 0 and torch.count_nonzero(dk) == 0
    check_grads((dq.cpu(), dk.cpu(), dv.cpu()), ref, f"bwd scale={scale} D={D}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_negative_scale_is_positive_on_negated_q(D):
    B, H, S = 2, 8, 700
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=8700 + D))
    do = _dout(B, H, S, D, 8800 + D).cuda()
    s = _f32(1 / math.sqrt(D))
    o1, l1 = fa.forward(q, k, v, causal=True, scale=-s)
    g1 = fa.backward(q, k, v, o1, l1, do, causal=True, scale=-s)
    o2, l2 = fa.forward(-q, k, v, causal=True, scale=s)
    g2 = fa.backward(-q, k, v, o2, l2, do, causal=True, scale=s)
    torch.cuda.synchronize()
    assert torch.equal(g1[0], -g2[0])   # d/dq of f(q) = g(-q) is -g'(-q)
    assert torch.equal(g1[2], g2[2])
    # dK accumulates dS^T q in one case and dS^T (-q) in the other: the matrix
    # cores' float32 sums of negated products are not bit-symmetric in every
    # case (measured: 3-11 elements per million differ, by about one bf16 ulp),
    # so dK is compared to one ulp of the element (or, where the sum cancels
    # to near zero, 2^-12 of the tensor's largest element), on at most 1e-4 of
    # its elements.
    a, b = g1[1].float(), g2[1].float()
    d = (a - b).abs()
    assert torch.all(d <= torch.maximum(a.abs(), b.abs()) * 2.0 ** -7 + a.abs().max() * 2.0 ** -12)
    assert torch.count_nonzero(d).item() <= 1e-4 * d.numel()
