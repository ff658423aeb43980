"""Launches of the library captured in a HIP graph (torch.cuda.CUDAGraph).

Every entry point enqueues kernel launches on the caller's stream and nothing
else (no memset, no allocation, no host synchronisation), so a captured call
must replay to the same bits as the eager call on the same inputs.  Each graph
is replayed several times; between replays the program does eager work of its
own (the outputs are overwritten with NaN and the inputs are read by an eager
reduction), and every replay is checked against the eager result.
"""

import math

import pytest
import torch

import exact_attention_67_amd as fa
from tests import workloads as wl

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def _capture_and_replay(launch, outs, inputs, expect):
    """Capture `launch` (which writes `outs`), replay it REPLAYS times with
    eager work between the replays, compare every replay with `expect`."""
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        launch()
    for r in range(REPLAYS):
        for t in outs:
            t.fill_(float("nan"))
        checksum = sum(float(x.float().sum()) for x in inputs)   # eager reads, synchronising
        assert math.isfinite(checksum)
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, expect):
            assert torch.equal(t, e), f"replay {r}: output differs from the eager call"
    del g


@pytest.mark.parametrize("D,causal", [(64, True), (128, True), (128, False), (256, True)])
def test_forward_in_graph(D, causal):
    q, k, v = (t.cuda() for t in wl.make_qkv(2, 3, 333, D, torch.bfloat16, seed=60 + D))
    o_ref, l_ref = fa.forward(q, k, v, causal=causal)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    _capture_and_replay(lambda: fa.forward(q, k, v, causal=causal, out=o, lse=lse),
                        (o, lse), (q, k, v), (o_ref, l_ref))


def test_forward_f32_in_graph():
    q, k, v = (t.cuda() for t in wl.make_qkv(1, 2, 128, 64, torch.float32, seed=65))
    o_ref, l_ref = fa.forward(q, k, v, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    _capture_and_replay(lambda: fa.forward(q, k, v, causal=True, out=o, lse=lse),
                        (o, lse), (q, k, v), (o_ref, l_ref))


@pytest.mark.parametrize("B,H,Sq,Sk,D", [(2, 3, 1, 3000, 128),    # decode kernel
                                         (2, 3, 1, 3000, 256),    # one query row, tiled
                                         (1, 4, 200, 1000, 128)])  # chunk against a prefix
def test_forward_kv_in_graph(B, H, Sq, Sk, D):
    q = wl.make_qkv(B, H, Sq, D, torch.bfloat16, seed=70)[0].cuda()
    _, k, v = (t.cuda() for t in wl.make_qkv(B, H, Sk, D, torch.bfloat16, seed=71))
    o_ref, l_ref = fa.forward_kv(q, k, v, causal=True)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    _capture_and_replay(lambda: fa.forward_kv(q, k, v, causal=True, out=o, lse=lse),
                        (o, lse), (q, k, v), (o_ref, l_ref))


def test_merge_in_graph():
    G, B, H, S, D = 5, 1, 4, 300, 128
    gen = torch.Generator().manual_seed(80)
    op = torch.randn((G, B, H, S, D), generator=gen).to(torch.bfloat16).cuda()
    lp = (torch.randn((G, B, H, S), generator=gen) * 3).cuda()
    o_ref, l_ref = fa.merge(op, lp)
    o, lse = torch.empty_like(o_ref), torch.empty_like(l_ref)
    _capture_and_replay(lambda: fa.merge(op, lp, out=o, lse=lse), (o, lse), (op, lp),
                        (o_ref, l_ref))


@pytest.mark.parametrize("D", [64, 128, 256])
def test_backward_in_graph(D):
    B, H, S = 1, 3, 300
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=90 + D))
    gen = torch.Generator().manual_seed(91)
    do = torch.randn((B, H, S, D), generator=gen).to(torch.bfloat16).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, causal=True)
    dq, dk, dv = (torch.empty_like(t) for t in ref)
    delta = torch.empty_like(lse)
    stream = [None]
    scale = 1.0 / math.sqrt(D)

    def launch():
        s = torch.cuda.current_stream().cuda_stream
        st = fa.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                       lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                       delta.data_ptr(), B, H, S, D, 1, scale, s)
        stream[0] = st

    _capture_and_replay(launch, (dq, dk, dv), (q, k, v, do), ref)
    assert stream[0] == fa.FA_OK


def test_backward_noalloc_in_graph():
    # the entry point for callers that cannot allocate: its scratch array is
    # set up by an eager call, then the captured call reuses it
    B, H, S, D = 1, 2, 257, 128
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=95))
    gen = torch.Generator().manual_seed(96)
    do = torch.randn((B, H, S, D), generator=gen).to(torch.bfloat16).cuda()
    o, lse = fa.forward(q, k, v, causal=True)
    ref = fa.backward(q, k, v, o, lse, do, causal=True)
    dq, dk, dv = (torch.empty_like(t) for t in ref)
    scale = 1.0 / math.sqrt(D)
    status = []

    def launch():
        s = torch.cuda.current_stream().cuda_stream
        status.append(fa.fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        do.data_ptr(), lse.data_ptr(), dq.data_ptr(),
                                        dk.data_ptr(), dv.data_ptr(), B, H, S, D, 1, scale, s))

    launch()                      # eager: sets up the scratch array on this device
    torch.cuda.synchronize()
    for t, e in zip((dq, dk, dv), ref):
        assert torch.equal(t, e)
    _capture_and_replay(launch, (dq, dk, dv), (q, k, v, do), ref)
    assert all(s == fa.FA_OK for s in status)
