"""The tile-pipeline study builds (libfa_mi355x_pipe_<name>.so: the bf16
forward with K/V tiles copied without prefetch, without prefetch and K in two
head-dim halves (the products over the first half start once it has landed),
or two or three steps ahead into three or four buffers each; and the D = 256
forward on the one-wave ring kernel in place of the wave-pair kernel) compute
the same attention as the library.

Each is checked against the float64 oracle, to the tolerances of
test_parity_gpu.py, on ragged shapes that run the 128-row and the 256-row
workgroups and enough key tiles to pass through every unrolled step group,
and bit for bit against the library on a longer causal problem (the three
builds run the same arithmetic in the same order; only the copies and waits
differ; the head-dim split sums the same products in the same order).  The
two D = 256 kernels form the same products, weights and sums in the same
order; they differ only in when a row's reference max is raised (the ring
kernel on a tile max more than 2^24 above it, the pair kernel on a lane's
weight sum above 2^24), so they agree bit for bit on inputs where it never
moves after the first tile, and to the oracle's tolerances on the stress rows
where it does.  The products-only probe (mfma_only) is a timing probe whose
results are void: it is only checked to run."""

import math

import pytest
import torch

import exact_attention_67_amd as fa
from exact_attention_67_amd import _lib
from oracle import attention as orc
from tests import workloads as wl
from tests.test_parity_gpu import check

pytestmark = pytest.mark.gpu

CORRECT = ("noprefetch", "ksplit", "ring3", "ring4", "ring256")

# B, H, S, D, causal (rows per workgroup follow from the library's plan)
SHAPES = [
    (1, 3, 333, 128, True),     # 128-row workgroups, ragged last tiles
    (1, 3, 1000, 128, False),   # 16 key tiles: full unrolled groups and a remainder
    (1, 2, 1000, 128, True),
    (32, 16, 300, 128, True),   # 256-row workgroups (eight waves)
    (16, 16, 511, 128, False),
    (2, 2, 777, 64, True),      # D = 64
    (1, 1, 1, 128, True),       # one query, one key
]


def _call(lib, q, k, v, causal, scale):
    o = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    B, H, S, D = q.shape
    st = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                    B, H, S, D, int(causal), scale, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK, fa.status_str(st)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("name", CORRECT)
@pytest.mark.parametrize("B,H,S,D,causal", SHAPES,
                         ids=[f"B{B}-H{H}-S{S}-D{D}-{'c' if c else 'n'}"
                              for B, H, S, D, c in SHAPES])
def test_variant_matches_oracle(name, B, H, S, D, causal):
    lib = _lib.load_variant(name)
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=7100 + S + D)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o, lse = _call(lib, q.cuda(), k.cuda(), v.cuda(), causal, scale)
    o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
    check(o.cpu(), lse.cpu(), o_ref, l_ref, torch.bfloat16,
          f"pipeline {name} B={B} H={H} S={S} D={D} causal={causal}")


@pytest.mark.parametrize("name", CORRECT)
@pytest.mark.parametrize("causal", [True, False])
def test_variant_bitwise_equal_to_library(name, causal):
    B, H, S, D = 2, 32, 3000, 128   # 256-row workgroups, 47 key tiles
    assert fa.fa_fwd_plan(B, H, S, D, int(causal), 2)["rows_per_group"] == 256
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=7300))
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o_lib, l_lib = _call(fa.load(), q, k, v, causal, scale)
    o_var, l_var = _call(_lib.load_variant(name), q, k, v, causal, scale)
    assert torch.equal(o_var, o_lib)
    assert torch.equal(l_var, l_lib)


def test_mfma_only_probe_runs():
    lib = _lib.load_variant("mfma_only")
    q, k, v = (t.cuda() for t in wl.make_qkv(2, 16, 1024, 128, torch.bfloat16, seed=7400))
    _call(lib, q, k, v, True, 1 / math.sqrt(128))


# B, H, S, causal, stress rows (D = 256)
SHAPES_256 = [
    (1, 3, 333, True, False),
    (1, 2, 700, False, False),
    (2, 2, 65, True, False),
    (1, 1, 1, True, False),
    (1, 2, 900, True, True),     # 1% of q and k rows x8: the reference max moves
]


@pytest.mark.parametrize("B,H,S,causal,stress", SHAPES_256,
                         ids=[f"B{B}-H{H}-S{S}-{'c' if c else 'n'}{'-stress' if st else ''}"
                              for B, H, S, c, st in SHAPES_256])
def test_ring256_matches_oracle(B, H, S, causal, stress):
    D = 256
    lib = _lib.load_variant("ring256")
    q, k, v = wl.make_qkv(B, H, S, D, torch.bfloat16, seed=7500 + S, stress_rows=stress)
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o, lse = _call(lib, q.cuda(), k.cuda(), v.cuda(), causal, scale)
    o_ref, l_ref = orc.attention_reference(q, k, v, causal, scale)
    check(o.cpu(), lse.cpu(), o_ref, l_ref, torch.bfloat16,
          f"ring256 B={B} H={H} S={S} causal={causal} stress={stress}")


@pytest.mark.parametrize("causal", [True, False])
def test_ring256_bitwise_equal_to_library(causal):
    B, H, S, D = 2, 8, 1500, 256   # 47 key tiles: every unrolled step position
    q, k, v = (t.cuda() for t in wl.make_qkv(B, H, S, D, torch.bfloat16, seed=7600))
    scale = float(torch.tensor(1 / math.sqrt(D), dtype=torch.float32))
    o_lib, l_lib = _call(fa.load(), q, k, v, causal, scale)
    o_var, l_var = _call(_lib.load_variant("ring256"), q, k, v, causal, scale)
    assert torch.equal(o_var, o_lib)
    assert torch.equal(l_var, l_lib)
