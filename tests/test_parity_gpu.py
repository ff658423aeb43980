"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (stated for this operation): O max-abs error <= 2e-2; O relative
RMS error <= 1e-2 for bf16 inputs and <= 1e-4 for float32 inputs, where the
relative RMS error is max over (b, h) of ||O - O_ref||_2 / ||O_ref||_2; LSE
max-abs error <= 1e-3 (natural-log units).
"""

import math
import sys

import pytest
import torch

import exact_attention_67_amd as fa
from oracle import attention as orc
from tests import workloads as wl

pytestmark = pytest.mark.gpu

TOL = {
    torch.bfloat16: dict(max_abs=2e-2, rel_rms=1e-2, lse=1e-3),
    torch.float32: dict(max_abs=2e-2, rel_rms=1e-4, lse=1e-3),
}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    fa.load()


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def run(q, k, v, causal, scale=None):
    """Inputs on the CPU -> (O, LSE) on the CPU, computed by the HIP kernels."""
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    o, lse = fa.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o.cpu(), lse.cpu()


def metrics(o, lse, o_ref, lse_ref):
    err = o.to(torch.float64) - o_ref
    max_abs = err.abs().max().item()
    num = err.pow(2).sum(dim=(-2, -1)).sqrt()
    den = o_ref.pow(2).sum(dim=(-2, -1)).sqrt().clamp_min(1e-300)
    rel = (num / den).max().item()
    lse_err = (lse.to(torch.float64) - lse_ref).abs().max().item()
    return max_abs, rel, lse_err


def check(o, lse, o_ref, lse_ref, dtype, label):
    assert torch.isfinite(o).all() and torch.isfinite(lse).all(), label
    max_abs, rel, lse_err = metrics(o, lse, o_ref, lse_ref)
    t = TOL[dtype]
    say(f"{label}: max_abs={max_abs:.3e} rel_rms={rel:.3e} lse={lse_err:.3e}")
    assert max_abs <= t["max_abs"], (label, max_abs)
    assert rel <= t["rel_rms"], (label, rel)
    assert lse_err <= t["lse"], (label, lse_err)


# ---------------------------------------------------------------------------
# The five workloads at full size
# ---------------------------------------------------------------------------

def _heads_to_check(w):
    if w.B * w.H * w.S <= 2 * 16 * 4096:
        return [(b, h) for b in range(w.B) for h in range(w.H)]
    if w.B == 1:
        return [(0, 0), (0, w.H // 3), (0, 2 * w.H // 3), (0, w.H - 1)]
    return [(0, 0), (0, w.H - 1), (w.B - 1, 0), (w.B - 1, w.H - 1)]


WL_CASES = [(name, c) for name in wl.ORDER for c in wl.WORKLOADS[name].causal]


@pytest.mark.parametrize("name,causal", WL_CASES,
                         ids=[f"{n}-{'causal' if c else 'full'}" for n, c in WL_CASES])
def test_workload_parity(name, causal):
    w = wl.WORKLOADS[name]
    say(f"[parity] {name} causal={causal} B={w.B} H={w.H} S={w.S} D={w.D} {w.dtype}")
    q, k, v = wl.make_inputs(w)
    o, lse = run(q, k, v, causal, w.scale)
    heads = _heads_to_check(w)
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = orc.attention_reference(q[sl], k[sl], v[sl], causal, w.scale,
                                               row_block=4096)
        check(o[sl], lse[sl], o_ref, l_ref, w.dtype, f"{name} causal={causal} b={b} h={h}")


# ---------------------------------------------------------------------------
# Small and ragged shapes, every head dimension, both masks, both dtypes
# ---------------------------------------------------------------------------

SMALL_S = [1, 2, 3, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 257, 300]
SMALL = [(S, D, c, dt) for dt in ("bf16", "f32") for D in (64, 128, 256)
         for c in (False, True) for S in SMALL_S]


@pytest.mark.parametrize("S,D,causal,dt", SMALL,
                         ids=[f"{dt}-D{D}-S{S}-{'c' if c else 'n'}" for S, D, c, dt in SMALL])
def test_small_shapes(S, D, causal, dt):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H = (2, 3) if S < 100 else (1, 2)
    q, k, v = wl.make_qkv(B, H, S, D, dtype, seed=1000 + S + D + int(causal))
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o, lse = run(q, k, v, causal, scale)
    o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
    check(o, lse, o_ref, l_ref, dtype, f"small {dt} B={B} H={H} S={S} D={D} causal={causal}")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("scale", [0.01, 0.3, 1.0, 3.0])
def test_other_scales(scale, D):
    # large scales spread the scores far apart: the reference max of a row is
    # raised on many tiles (at D = 256 the weights' wave raises it and the
    # P*V wave rescales O from the reference that comes with the weights)
    q, k, v = wl.make_qkv(1, 2, 333, D, torch.bfloat16, seed=77)
    for causal in (False, True):
        o, lse = run(q, k, v, causal, scale)
        o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
        check(o, lse, o_ref, l_ref, torch.bfloat16, f"scale={scale} D={D} causal={causal}")


# ---------------------------------------------------------------------------
# Both bf16 workgroup shapes at D = 128 (4 waves = 128 query rows, 8 waves =
# 256 rows; the library picks by grid size), with ragged last query tiles in
# which some waves hold no rows at all
# ---------------------------------------------------------------------------

WG_CASES = [  # B, H, S, causal, rows per workgroup the library must pick
    (32, 16, 300, True, 256),
    (32, 16, 257, True, 256),
    (16, 16, 300, False, 256),
    (16, 16, 511, False, 256),
    (1, 4, 300, True, 128),
    (1, 4, 300, False, 128),
]


@pytest.mark.parametrize("B,H,S,causal,rows", WG_CASES,
                         ids=[f"B{B}-H{H}-S{S}-{'c' if c else 'n'}-r{r}"
                              for B, H, S, c, r in WG_CASES])
def test_workgroup_shapes(B, H, S, causal, rows):
    plan = fa.fa_fwd_plan(B, H, S, 128, int(causal), 2)
    assert plan["rows_per_group"] == rows, plan
    q, k, v = wl.make_qkv(B, H, S, 128, torch.bfloat16, seed=4000 + S + B)
    scale = float(torch.tensor(1 / math.sqrt(128), dtype=torch.float32))
    o, lse = run(q, k, v, causal, scale)
    o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
    check(o, lse, o_ref, l_ref, torch.bfloat16,
          f"workgroup rows={rows} B={B} H={H} S={S} causal={causal}")


# ---------------------------------------------------------------------------
# Closed forms on the GPU path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("D", [64, 128, 256])
@pytest.mark.parametrize("causal", [False, True])
def test_long_sequence_sampled_rows(D, causal):
    # 131072 keys: 64-bit row offsets, and the running softmax carried over
    # more than 2000 key tiles; rows checked one by one against the oracle
    B, H, S = 1, 2, 131072
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=17000 + D + causal)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o, lse = run(q, k, v, causal, scale)
    g = torch.Generator().manual_seed(18000 + D)
    rows = sorted(set([0, 1, 63, 64, 255, 256, S // 2, S - 257, S - 2, S - 1] +
                      torch.randint(0, S, (14,), generator=g).tolist()))
    for h in range(H):
        o_ref, l_ref = orc.attention_rows(q, k, v, causal, scale, 0, h, rows)
        check(o[0, h, rows].unsqueeze(0), lse[0, h, rows].unsqueeze(0), o_ref.unsqueeze(0),
              l_ref.unsqueeze(0), torch.bfloat16, f"long S={S} D={D} causal={causal} h={h}")


@pytest.mark.parametrize("D,causal", [(64, False), (128, True), (256, True)])
def test_tensors_beyond_4gib(D, causal):
    # Every tensor is larger than 4 GiB, so the heads at its end lie more than
    # 2^32 bytes past its base: the per-head and per-tile base addresses of
    # the K/V copies, the Q loads and the O/LSE stores are 64-bit while the
    # per-lane offsets are 32-bit.  Ragged S; sampled rows of the first head
    # and of the last two, against the oracle (inputs drawn on the GPU from a
    # seeded generator, the sampled heads copied back for the oracle).
    S = 1000
    heads = (1 << 32) // (S * D * 2) + 3
    B, H = 2, (heads + 1) // 2
    assert B * H * S * D * 2 > (1 << 32)
    g = torch.Generator(device="cuda").manual_seed(19000 + D)
    q, k, v = (torch.randn((B, H, S, D), generator=g, device="cuda", dtype=torch.bfloat16)
               for _ in range(3))
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    say(f"tensors beyond 4 GiB: B={B} H={H} S={S} D={D} causal={causal}")
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    rows = [0, 1, 127, 128, 255, 256, 511, 777, 998, 999]
    for b, h in [(0, 0), (B - 1, H - 2), (B - 1, H - 1)]:
        qh, kh, vh = (t[b:b + 1, h:h + 1].cpu() for t in (q, k, v))
        o_ref, l_ref = orc.attention_rows(qh, kh, vh, causal, scale, 0, 0, rows)
        check(o[b, h, rows].cpu().unsqueeze(0), lse[b, h, rows].cpu().unsqueeze(0),
              o_ref.unsqueeze(0), l_ref.unsqueeze(0), torch.bfloat16,
              f">4GiB D={D} causal={causal} b={b} h={h}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("D", [64, 128, 256])
def test_zero_keys_give_prefix_means(D):
    S = 200
    q, _, v = wl.make_qkv(1, 1, S, D, torch.bfloat16, seed=5)
    k = torch.zeros_like(q)
    o, lse = run(q, k, v, True, 0.125)
    vv = v[0, 0].double()
    pref = vv.cumsum(0) / torch.arange(1, S + 1, dtype=torch.float64).unsqueeze(1)
    assert (o[0, 0].double() - pref).abs().max().item() < 1e-2
    want = torch.log(torch.arange(1, S + 1, dtype=torch.float64))
    assert (lse[0, 0].double() - want).abs().max().item() < 1e-4
    o, lse = run(q, k, v, False, 0.125)
    assert (o[0, 0].double() - vv.mean(0)).abs().max().item() < 1e-2
    assert (lse[0, 0].double() - math.log(S)).abs().max().item() < 1e-4


@pytest.mark.parametrize("D", [64, 128, 256])
def test_causal_row0_is_v0_and_constant_v(D):
    q, k, v = wl.make_qkv(2, 2, 150, D, torch.bfloat16, seed=9)
    o, lse = run(q, k, v, True, 1 / math.sqrt(D))
    assert torch.equal(o[:, :, 0], v[:, :, 0])
    s00 = (q[:, :, 0].double() * k[:, :, 0].double()).sum(-1) * float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    assert (lse[:, :, 0].double() - s00).abs().max().item() < 1e-4
    c = torch.linspace(-2, 3, D).to(torch.bfloat16)
    vc = c.expand_as(v).contiguous()
    for causal in (False, True):
        o, _ = run(q, k, vc, causal)
        err = (o.double() - c.double()).abs()
        assert (err <= c.double().abs() * 2 ** -7 + 1e-6).all()


def test_stress_rows_large_scores():
    # scores of several hundred: the reference max moves by large jumps
    q, k, v = wl.make_qkv(1, 2, 1000, 256, torch.bfloat16, seed=11, stress_rows=True)
    q = (q.float() * 4).to(torch.bfloat16)
    for causal in (False, True):
        o, lse = run(q, k, v, causal)
        o_ref, l_ref = orc.attention_reference(q, k, v, causal, 1 / 16)
        check(o, lse, o_ref, l_ref, torch.bfloat16, f"stress x32 causal={causal}")


@pytest.mark.parametrize("D", [64, 128, 256])
def test_reference_max_raised_many_times(D):
    # keys scaled up along the sequence (x1 to x31): each row's largest score
    # keeps growing from tile to tile, far past any threshold for moving the
    # row's reference max, so the rescale runs several times per row
    B, H, S = 1, 2, 600
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=12)
    ramp = (1.0 + torch.arange(S, dtype=torch.float32) / 20.0).view(1, 1, S, 1)
    k = (k.float() * ramp).to(torch.bfloat16)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    for causal in (False, True):
        o, lse = run(q, k, v, causal, scale)
        o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
        check(o, lse, o_ref, l_ref, torch.bfloat16, f"ramp D={D} causal={causal}")


# ---------------------------------------------------------------------------
# Hygiene: every output written, nothing outside written, deterministic,
# concurrent streams, host-side rejection of bad pointers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_poisoned_outputs_and_guard_bands(dt):
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    B, H, S, D = 2, 3, 129, 128
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, dtype, seed=21))
    n, nl, pad = B * H * S * D, B * H * S, 4096
    obuf = torch.full((n + 2 * pad,), float("nan"), dtype=dtype, device="cuda")
    lbuf = torch.full((nl + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    obuf[:pad] = 7.0
    obuf[-pad:] = 7.0
    lbuf[:pad] = 7.0
    lbuf[-pad:] = 7.0
    o = obuf[pad:pad + n].view(B, H, S, D)
    lse = lbuf[pad:pad + nl].view(B, H, S)
    for causal in (False, True):
        fa.forward(q, k, v, causal=causal, out=o, lse=lse)
        torch.cuda.synchronize()
        assert torch.isfinite(o).all() and torch.isfinite(lse).all()
        assert (obuf[:pad] == 7).all() and (obuf[-pad:] == 7).all()
        assert (lbuf[:pad] == 7).all() and (lbuf[-pad:] == 7).all()


@pytest.mark.parametrize("name", ["c4_bf16_causal_1x32x16384x128",
                                  "c5_bf16_causal_2x8x8192x256_stress"])
def test_full_size_outputs_all_written(name):
    # the launch shapes bench.py times, on outputs poisoned with NaN and
    # guarded by sentinel bands: every O and LSE element is written (finite),
    # nothing beyond them is
    w = wl.WORKLOADS[name]
    q, k, v = (t.cuda() for t in wl.make_inputs(w))
    n, nl, pad = w.B * w.H * w.S * w.D, w.B * w.H * w.S, 1 << 16
    obuf = torch.full((n + 2 * pad,), float("nan"), dtype=torch.bfloat16, device="cuda")
    lbuf = torch.full((nl + 2 * pad,), float("nan"), dtype=torch.float32, device="cuda")
    for buf in (obuf, lbuf):
        buf[:pad] = 7.0
        buf[-pad:] = 7.0
    o = obuf[pad:pad + n].view(w.B, w.H, w.S, w.D)
    lse = lbuf[pad:pad + nl].view(w.B, w.H, w.S)
    fa.forward(q, k, v, causal=True, scale=w.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    assert bool((obuf[:pad] == 7).all()) and bool((obuf[-pad:] == 7).all())
    assert bool((lbuf[:pad] == 7).all()) and bool((lbuf[-pad:] == 7).all())


def test_deterministic():
    q, k, v = (t.cuda() for t in wl.make_qkv(2, 4, 777, 128, torch.bfloat16, seed=31))
    for causal in (False, True):
        o1, l1 = fa.forward(q, k, v, causal=causal)
        o2, l2 = fa.forward(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_two_streams():
    a = [t.cuda() for t in wl.make_qkv(2, 8, 1024, 128, torch.bfloat16, seed=41)]
    b = [t.cuda() for t in wl.make_qkv(2, 8, 1024, 64, torch.bfloat16, seed=42)]
    ra = fa.forward(*a, causal=True)
    rb = fa.forward(*b, causal=False)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s1):
        xa = fa.forward(*a, causal=True, stream=s1)
    with torch.cuda.stream(s2):
        xb = fa.forward(*b, causal=False, stream=s2)
    torch.cuda.synchronize()
    assert torch.equal(ra[0], xa[0]) and torch.equal(ra[1], xa[1])
    assert torch.equal(rb[0], xb[0]) and torch.equal(rb[1], xb[1])


def test_bad_pointers_rejected_outputs_untouched():
    B, H, S, D = 1, 2, 64, 64
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=51))
    o = torch.full((B, H, S, D), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, S), 3.0, dtype=torch.float32, device="cuda")
    flat = torch.empty(B * H * S * D + 8, dtype=torch.bfloat16, device="cuda")
    mis = flat[1:1 + B * H * S * D]
    st = fa.fa_fwd(mis.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                   B, H, S, D, 1, 0.125, None)
    assert st == fa.FA_ERR_ALIGN
    st = fa.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), q.data_ptr(), lse.data_ptr(),
                   B, H, S, D, 1, 0.125, None)
    assert st == fa.FA_ERR_ALIAS
    torch.cuda.synchronize()
    assert (o == 3).all() and (lse == 3).all()
