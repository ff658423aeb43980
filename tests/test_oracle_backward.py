"""Pins for the backward-pass oracle (CPU only).

``attention_backward`` writes the gradient of the forward definition out with
the chain rule.  It is tied to things other than itself:

- automatic differentiation (torch.autograd) of the float64 forward oracle, a
  different way of differentiating the same definition;
- central finite differences of  L = sum(O * dO)  on tiny inputs;
- closed forms: with k = 0 every row attends uniformly (dq = 0 and dv is a
  prefix mean of dO); with the causal mask, row 0's output is v_0 whatever
  q_0 is, so dq_0 = 0;
- invariances: adding one vector to every key shifts each row's scores by a
  constant, which changes nothing (so no gradient changes); gradients are
  linear in dO.

Broken copies of the oracle must each fail at least one pin.
"""

import pytest
import torch

from oracle import attention as orc
from oracle import backward as bwd


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64)


def _close(a, b, tol):
    assert a.shape == b.shape, (a.shape, b.shape)
    err = (a - b).abs().max().item()
    assert err <= tol, err


def _inputs(B, H, S, D, seed):
    return tuple(_rand((B, H, S, D), seed + i) for i in range(4))   # q, k, v, dO


# ----------------------------------------------------------------------------
# Pins of a backward callable  grad(q, k, v, do, causal, scale) -> (dq, dk, dv)
# ----------------------------------------------------------------------------

def pin_autograd(grad):
    for causal in (False, True):
        q, k, v, do = _inputs(2, 2, 13, 6, 10 + causal)
        qa, ka, va = (t.clone().requires_grad_(True) for t in (q, k, v))
        # the forward oracle detaches its inputs; differentiate the same
        # definition written with the same torch operations
        s = torch.matmul(qa, ka.transpose(-2, -1)) * 0.45
        if causal:
            s = s.masked_fill(~orc.causal_keep_mask(13, 13), float("-inf"))
        o = torch.matmul(torch.softmax(s, dim=-1), va)
        o_ref, _ = orc.attention_reference(q, k, v, causal, 0.45)
        _close(o.detach(), o_ref, 1e-13)                     # same forward
        (o * do).sum().backward()
        dq, dk, dv = grad(q, k, v, do, causal, 0.45)
        _close(dq, qa.grad, 1e-12)
        _close(dk, ka.grad, 1e-12)
        _close(dv, va.grad, 1e-12)


def pin_finite_differences(grad):
    h = 1e-6
    for causal in (False, True):
        q, k, v, do = _inputs(1, 1, 5, 3, 20 + causal)
        dq, dk, dv = grad(q, k, v, do, causal, 0.8)

        def loss(qq, kk, vv):
            o, _ = orc.attention_reference(qq, kk, vv, causal, 0.8)
            return float((o * do).sum())

        for t, g, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
            for idx in range(t.numel()):
                tp, tm = t.clone(), t.clone()
                tp.view(-1)[idx] += h
                tm.view(-1)[idx] -= h
                args_p = [q, k, v]
                args_m = [q, k, v]
                args_p[which], args_m[which] = tp, tm
                fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
                assert abs(fd - g.view(-1)[idx].item()) <= 1e-7, (which, idx, fd)


def pin_zero_keys(grad):
    # k = 0: every visible key scores 0, rows attend uniformly
    B, H, S, D = 1, 2, 9, 4
    q, _, v, do = _inputs(B, H, S, D, 30)
    k = torch.zeros_like(q)
    for causal in (False, True):
        dq, dk, dv = grad(q, k, v, do, causal, 0.5)
        assert torch.all(dq.abs() <= 1e-15)
        ref = torch.zeros_like(v)
        for j in range(S):
            rows = range(j, S) if causal else range(S)
            for i in rows:
                n = (i + 1) if causal else S
                ref[..., j, :] += do[..., i, :] / n
        _close(dv, ref, 1e-13)


def pin_causal_row0_has_no_query_gradient(grad):
    q, k, v, do = _inputs(2, 1, 7, 5, 40)
    dq, _, _ = grad(q, k, v, do, True, 0.7)
    # zero up to rounding: Delta_0 and dP_00 are the same dot product summed
    # in different orders
    assert dq[..., 0, :].abs().max().item() <= 1e-13
    assert dq[..., 1:, :].abs().max().item() > 1e-3


def pin_key_shift_invariance(grad):
    q, k, v, do = _inputs(1, 2, 11, 4, 50)
    shift = _rand((1, 2, 1, 4), 55) * 3.0
    for causal in (False, True):
        a = grad(q, k, v, do, causal, 0.6)
        b = grad(q, k + shift, v, do, causal, 0.6)
        for x, y in zip(a, b):
            _close(x, y, 1e-10)


def pin_linear_in_dout(grad):
    q, k, v, do = _inputs(1, 1, 8, 3, 60)
    do2 = _rand(do.shape, 66)
    a = grad(q, k, v, do, True, 0.9)
    b = grad(q, k, v, do2, True, 0.9)
    c = grad(q, k, v, 2.0 * do - do2, True, 0.9)
    for x, y, z in zip(a, b, c):
        _close(z, 2.0 * x - y, 1e-12)


PINS = [pin_autograd, pin_finite_differences, pin_zero_keys, pin_causal_row0_has_no_query_gradient,
        pin_key_shift_invariance, pin_linear_in_dout]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(bwd.attention_backward)


def test_delta_is_rowsum_of_p_times_dp():
    q, k, v, do = _inputs(1, 2, 10, 4, 70)
    o, _ = orc.attention_reference(q, k, v, True, 0.5)
    p = orc.attention_weights(q, k, True, 0.5)
    dp = do @ v.transpose(-2, -1)
    _close(bwd.attention_delta(o, do), (p * dp).sum(-1), 1e-13)


# ----------------------------------------------------------------------------
# Planted mistakes
# ----------------------------------------------------------------------------

def _parts(q, k, v, do, causal, scale):
    s = (q @ k.transpose(-2, -1)) * scale
    if causal:
        s = s.masked_fill(~orc.causal_keep_mask(s.shape[-2], s.shape[-1]), float("-inf"))
    p = torch.softmax(s, -1)
    o = p @ v
    dp = do @ v.transpose(-2, -1)
    return s, p, o, dp


def _mut_no_delta(q, k, v, do, causal, scale):
    s, p, o, dp = _parts(q, k, v, do, causal, scale)
    ds = p * dp
    return ds @ k * scale, ds.transpose(-2, -1) @ q * scale, p.transpose(-2, -1) @ do


def _mut_delta_sign(q, k, v, do, causal, scale):
    s, p, o, dp = _parts(q, k, v, do, causal, scale)
    ds = p * (dp + (do * o).sum(-1, keepdim=True))
    return ds @ k * scale, ds.transpose(-2, -1) @ q * scale, p.transpose(-2, -1) @ do


def _mut_dk_not_transposed(q, k, v, do, causal, scale):
    dq, dk, dv = bwd.attention_backward(q, k, v, do, causal, scale)
    s, p, o, dp = _parts(q, k, v, do, causal, scale)
    ds = p * (dp - (do * o).sum(-1, keepdim=True))
    return dq, ds @ q * scale, dv


def _mut_dq_unscaled(q, k, v, do, causal, scale):
    dq, dk, dv = bwd.attention_backward(q, k, v, do, causal, scale)
    return dq / scale, dk, dv


def _mut_mask_dropped(q, k, v, do, causal, scale):
    return bwd.attention_backward(q, k, v, do, False, scale)


def _mut_dv_not_transposed(q, k, v, do, causal, scale):
    dq, dk, dv = bwd.attention_backward(q, k, v, do, causal, scale)
    s, p, o, dp = _parts(q, k, v, do, causal, scale)
    return dq, dk, p @ do


@pytest.mark.parametrize("mutant", [_mut_no_delta, _mut_delta_sign, _mut_dk_not_transposed,
                                    _mut_dq_unscaled, _mut_mask_dropped, _mut_dv_not_transposed],
                         ids=lambda m: m.__name__)
def test_backward_pins_catch_planted_mistakes(mutant):
    failed = []
    for pin in PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin caught {mutant.__name__}"
