"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
float64 backward oracle (oracle/backward.py).

Flow: the HIP forward computes O and LSE from bf16 q, k, v; the HIP backward
takes them with a seeded bf16 dO.  The oracle computes exact float64
gradients of the same bf16 inputs.  Tolerance per gradient tensor and head:
relative RMS error ||g - g_ref|| / ||g_ref|| <= 1e-2, and max |g - g_ref| <=
2e-2 * max |g_ref|.  (bf16 rounding of P and dS before the products they feed,
of O inside Delta, and of the results bounds the error at a few times 2^-9
relative.)
"""

import math
import sys

import pytest
import torch

import exact_attention_67_amd as fa
from oracle import backward as bwd
from tests import workloads as wl

pytestmark = pytest.mark.gpu

REL_RMS = 1e-2
MAX_REL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _dout(B, H, S, D, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((B, H, S, D), generator=g).to(torch.bfloat16)


def run_backward(q, k, v, do, causal, scale):
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qd, kd, vd, o, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse, dq.cpu(), dk.cpu(), dv.cpu()


def check_grads(got, ref, label):
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        g64 = g.double()
        assert torch.isfinite(g64).all(), (label, name)
        err = g64 - r
        num = err.pow(2).sum(dim=(-2, -1)).sqrt()
        den = r.pow(2).sum(dim=(-2, -1)).sqrt()
        live = den > 1e-6
        rel = (num[live] / den[live]).max().item() if live.any() else num.max().item()
        mx = err.abs().max().item() / max(r.abs().max().item(), 1e-6)
        say(f"{label} {name}: rel_rms={rel:.3e} max_rel={mx:.3e}")
        assert rel <= REL_RMS, (label, name, rel)
        assert mx <= MAX_REL, (label, name, mx)


# S = 777: several 256-query dq blocks with a ragged tail, an odd number of
# 128-key dk/dv blocks
SHAPES = [(1, 2, 17), (2, 2, 64), (1, 3, 65), (1, 2, 127), (2, 1, 128), (1, 2, 129), (2, 2, 200),
          (1, 2, 300), (1, 1, 511), (1, 2, 777)]
CASES = [(B, H, S, D, c) for (B, H, S) in SHAPES for D in (64, 128, 256) for c in (False, True)]


@pytest.mark.parametrize("B,H,S,D,causal", CASES,
                         ids=[f"B{B}H{H}S{S}-D{D}-{'c' if c else 'n'}" for B, H, S, D, c in CASES])
def test_backward_parity(B, H, S, D, causal):
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=11000 + S + D)
    do = _dout(B, H, S, D, 12000 + S + D)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    _, _, dq, dk, dv = run_backward(q, k, v, do, causal, scale)
    ref = bwd.attention_backward(q, k, v, do, causal, scale)
    check_grads((dq, dk, dv), ref, f"bwd B={B} H={H} S={S} D={D} causal={causal}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_larger(D):
    B, H, S = 2, 4, 1024
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=13000 + D)
    do = _dout(B, H, S, D, 14000 + D)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    for causal in (False, True):
        _, _, dq, dk, dv = run_backward(q, k, v, do, causal, scale)
        ref = bwd.attention_backward(q, k, v, do, causal, scale)
        check_grads((dq, dk, dv), ref, f"bwd 2x4x1024 D={D} causal={causal}")


def test_backward_tensors_beyond_4gib():
    # Every tensor larger than 4 GiB (heads at the end lie more than 2^32
    # bytes past the base); gradients of the first head and of the last one
    # against the oracle on those heads (inputs drawn on the GPU from a seeded
    # generator, the two heads copied back).
    S, D, causal = 1000, 128, True
    heads = (1 << 32) // (S * D * 2) + 3
    B, H = 2, (heads + 1) // 2
    assert B * H * S * D * 2 > (1 << 32)
    g = torch.Generator(device="cuda").manual_seed(19500)
    q, k, v, do = (torch.randn((B, H, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
                   for _ in range(4))
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
    torch.cuda.synchronize()
    for b, h in [(0, 0), (B - 1, H - 1)]:
        sl = lambda t: t[b:b + 1, h:h + 1].cpu()
        ref = bwd.attention_backward(sl(q), sl(k), sl(v), sl(do), causal, scale)
        check_grads((sl(dq), sl(dk), sl(dv)), ref, f"bwd >4GiB b={b} h={h}")
    del q, k, v, do, o, lse, dq, dk, dv
    torch.cuda.empty_cache()


FULL = [("c3_bf16_2x16x4096x128", False, [(0, 0), (1, 15)]),
        ("c3_bf16_2x16x4096x128", True, [(0, 0), (1, 15)]),
        ("c4_bf16_causal_1x32x16384x128", True, [(0, 31)]),
        ("c5_bf16_causal_2x8x8192x256_stress", True, [(1, 7)])]


@pytest.mark.parametrize("name,causal,heads", FULL,
                         ids=[f"{n}-{'c' if c else 'n'}" for n, c, _ in FULL])
def test_backward_full_size_sampled_heads(name, causal, heads):
    # the backward the benchmark times, at full size and in its launch
    # configuration (dO drawn as the benchmark draws it); whole gradients of
    # sampled heads against the oracle on those heads
    w = wl.WORKLOADS[name]
    q, k, v = wl.make_inputs(w)
    g = torch.Generator("cpu").manual_seed(w.seed + 100)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    _, _, dq, dk, dv = run_backward(q, k, v, do, causal, w.scale)
    torch.cuda.empty_cache()
    for b, h in heads:
        sl = lambda t: t[b:b + 1, h:h + 1]
        ref = bwd.attention_backward(sl(q), sl(k), sl(v), sl(do), causal, w.scale)
        check_grads((sl(dq), sl(dk), sl(dv)), ref, f"bwd {name} causal={causal} b={b} h={h}")
        del ref


def test_delta_buffer_is_rowsum():
    B, H, S, D = 1, 2, 200, 128
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=15000))
    do = _dout(B, H, S, D, 15001).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    delta = torch.empty((B, H, S), dtype=torch.float32, device="cuda")
    st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                   B, H, S, D, 1, 1 / math.sqrt(D), torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    torch.cuda.synchronize()
    ref = bwd.attention_delta(o.cpu(), do.cpu())
    assert (delta.cpu().double() - ref).abs().max().item() <= 1e-4 * max(1.0, ref.abs().max().item())


def test_single_key_closed_form():
    # S = 1: P = 1, O = v, so dv = dO and dS = dO.v - dO.O = 0 (dq = dk = 0
    # up to the rounding of two equal dot products)
    B, H, S, D = 2, 3, 1, 128
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=16000)
    do = _dout(B, H, S, D, 16001)
    for causal in (False, True):
        _, _, dq, dk, dv = run_backward(q, k, v, do, causal, 1 / math.sqrt(D))
        assert torch.equal(dv, do)
        assert dq.abs().max().item() <= 1e-3 and dk.abs().max().item() <= 1e-3


def test_backward_on_a_side_stream_matches_current_stream():
    # The Delta buffer is released when backward() returns; it must be
    # allocated on the stream the kernels run on, so that allocations made
    # meanwhile on the current stream cannot take its memory.
    B, H, S, D = 1, 8, 2048, 128
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=19000))
    do = _dout(B, H, S, D, 19001).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    got = fa.backward(q, k, v, o, lse, do, causal=True, stream=side)
    churn = [torch.full((B, H, S), float("nan"), dtype=torch.float32, device="cuda")
             for _ in range(16)]
    torch.cuda.synchronize()
    del churn
    for name, a, b in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(a, b), name
