#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step = one call of fa_fwd over the whole workload (inputs resident in HBM
before timing starts).  Default workload: causal bf16 attention, B=1 H=32
S=16384 D=128 (the long-sequence causal shape with S >= 4096 and D = 128).
Prints ONE JSON line on stdout; a per-workload table goes to stderr with
--all.  The line's "secondary" object adds, outside `value`, the forward on
the other workloads (S = 4096 D = 128 causal and unmasked, S = 8192 D = 256,
S = 1024 D = 64), the queries-against-a-prefix path (prefill, decode), the
merge and the backward pass.  The secondary work runs first, so the headline
launches start on a GPU whose shader clock has settled under load (the
timed region is still exactly --steps launches after --warmup untimed ones).

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                  [--all] [--no-cpu-baseline] [--copy-calibration]
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOPS (bf16, causal) and % of MI355X bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 matrix peak
PEAK_F32_TFLOPS = 157.3     # MI355X published fp32 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X published HBM3E bandwidth
DEFAULT_WORKLOAD = "c4_bf16_causal_1x32x16384x128"
# sources of the forward kernels (the profile summaries are keyed to them)
SRCS = [os.path.join(ROOT, "exact_attention_67_amd", "csrc", n) for n in ("fa_fwd.hip", "fa_device.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_bf16_c4_hbm_traffic.txt")
NOMINAL_SCLK_MHZ = 2400.0   # clock of the published peak
COLD_EVICT_BYTES = 512 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_digest() -> str:
    h = hashlib.sha256()
    for p in SRCS:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_profile_value(workload: str, key: str):
    """A figure from the committed rocprofv3 summary (HBM bytes per launch,
    sustained shader clock), if it was taken on the current kernel source for
    this workload; else None."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        m = re.match(r"^\s*([a-z0-9_]+)\s*:\s*(\S+)", line)
        if m:
            kv[m.group(1)] = m.group(2)
    if kv.get("source_sha256") != source_digest() or kv.get("workload") != workload:
        return None
    try:
        return float(kv[key])
    except (KeyError, ValueError):
        return None


def recorded_traffic(workload: str):
    return recorded_profile_value(workload, "traffic_bytes_per_launch")


def time_workload(w, causal, steps, warmup, cold_launches=0, inputs=None):
    """Time `steps` back-to-back launches after `warmup` untimed ones; inputs
    (q, k, v on the GPU) are made here unless given."""
    import torch
    import exact_attention_67_amd as fa
    from tests import workloads as wl

    q, k, v = wl.make_inputs(w, device="cuda") if inputs is None else inputs
    out = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    fn = fa.fa_fwd if w.dtype == torch.bfloat16 else fa.fa_fwd_f32
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.S, w.D, int(causal), w.scale, stream.cuda_stream)

    def step():
        st = fn(*args)
        if st != fa.FA_OK:
            raise fa.FAError(st, fn.__name__)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # Whole timed region: exactly `steps` back-to-back launches.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t0.elapsed_time(t1)

    # Per-launch durations: an event pair around each launch on the same
    # stream (separate pass, so the pairs do not perturb the timed region).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    res = dict(total_ms=total_ms, wall_s=wall, ms_per_step=total_ms / steps,
               launch_ms_avg=sum(per) / len(per), launch_ms_min=per[0],
               launch_ms_med=per[len(per) // 2])

    # Cold: before each timed launch (outside its event pair) write a 512 MiB
    # buffer on the same stream, evicting L2 and the last-level cache.
    if cold_launches > 0:
        scratch = torch.empty(COLD_EVICT_BYTES, dtype=torch.uint8, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(cold_launches)]
        for i, (a, b) in enumerate(evs):
            scratch.fill_(i & 0xFF)
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        cold = sorted(a.elapsed_time(b) for a, b in evs)
        res.update(cold_ms_med=cold[len(cold) // 2], cold_ms_min=cold[0])
        del scratch
    return res


def _time_launches(fn, steps, warmup):
    """Mean, median and min of per-launch HIP event pairs on the current stream."""
    import torch
    stream = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    return sum(per) / len(per), per[len(per) // 2], per[0]


def kernel_name(w, causal) -> str:
    """Name of the forward kernel fa_fwd launches for workload w (from the
    host-side launch plan)."""
    import torch
    import exact_attention_67_amd as fa
    c = "true" if causal else "false"
    if w.dtype != torch.bfloat16:
        return f"fa_fwd_f32_kernel<{w.D},{c}>"
    plan = fa.fa_fwd_plan(w.B, w.H, w.S, w.D, int(causal), 2)
    waves, bc = plan["threads"] // 64, plan["keys_per_tile"]
    if w.D == 256:
        return f"fa_fwd_bf16_pair_kernel<{c}>"
    return f"fa_fwd_bf16_kernel<{w.D},{bc},{waves},{c},true>"


# forward figures beside the headline: (workload, causal)
SECONDARY_FWD = (("c3_bf16_2x16x4096x128", True), ("c3_bf16_2x16x4096x128", False),
                 ("c5_bf16_causal_2x8x8192x256_stress", True),
                 ("c2_bf16_causal_4x16x1024x64", True))


def time_secondary_forward():
    """The forward on the other workloads: warm-up launches worth about 200 ms
    of GPU time, then back-to-back launches worth about 50 ms, timed as the
    headline (TFLOP/s over the whole timed region)."""
    import torch
    from tests import workloads as wl
    out = {}
    for name, causal in SECONDARY_FWD:
        w = wl.WORKLOADS[name]
        probe = time_workload(w, causal, 3, 1)
        warm = max(3, min(2000, int(200.0 / max(probe["ms_per_step"], 1e-3))))
        steps = max(10, min(500, int(50.0 / max(probe["ms_per_step"], 1e-3))))
        r = time_workload(w, causal, steps, warm)
        tf = w.flops(causal) / (r["ms_per_step"] * 1e-3) / 1e12
        key = f"forward_{name}_{'causal' if causal else 'full'}"
        out[key] = {"tflops": round(tf, 2), "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
                    "ms_per_step": round(r["ms_per_step"], 5), "steps": steps, "warmup": warm,
                    "launch_ms_avg": round(r["launch_ms_avg"], 5),
                    "launch_ms_median": round(r["launch_ms_med"], 5),
                    "causal": causal, "flops_per_launch": w.flops(causal),
                    "kernel": kernel_name(w, causal)}
        log(f"[bench] {key}: {r['ms_per_step']:.4f} ms/step, {tf:.1f} TFLOP/s "
            f"({100 * tf / PEAK_BF16_TFLOPS:.1f}% of peak)")
        torch.cuda.empty_cache()
    return out


def time_secondary(steps):
    """The other forward workloads, the Sq != Sk path (chunked prefill,
    decode), the merge over key sets and the backward pass, each on its own
    synthetic workload; reported beside the headline figure."""
    import torch
    import exact_attention_67_amd as fa
    from tests import workloads as wl

    out = time_secondary_forward()
    for name, w in wl.PREFIX_WORKLOADS.items():
        q, k, v = (t.cuda() for t in wl.make_prefix_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.Sq), dtype=torch.float32, device="cuda")

        def call():
            fa.forward_kv(q, k, v, causal=w.causal, scale=w.scale, out=o, lse=lse)

        avg, med, mn = _time_launches(call, steps, 3)
        out[name] = {"launch_ms_avg": round(avg, 5), "launch_ms_median": round(med, 5),
                     "tflops": round(w.flops() / (avg * 1e-3) / 1e12, 2),
                     "kv_read_gbs": round(w.kv_bytes() / (avg * 1e-3) / 1e9, 1)}
        log(f"[bench] {name}: {avg:.4f} ms, {out[name]['tflops']} TFLOP/s, "
            f"K/V read {out[name]['kv_read_gbs']} GB/s")
        del q, k, v, o, lse
    for name in ("c3_bf16_2x16x4096x128", "c4_bf16_causal_1x32x16384x128",
                 "c5_bf16_causal_2x8x8192x256_stress"):
        w = wl.WORKLOADS[name]
        q, k, v = (t.cuda() for t in wl.make_inputs(w))
        g = torch.Generator("cpu").manual_seed(w.seed + 100)
        do = torch.randn(q.shape, generator=g).to(torch.bfloat16).cuda()
        o, lse = fa.forward(q, k, v, causal=True, scale=w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
        stream = torch.cuda.current_stream().cuda_stream
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                w.B, w.H, w.S, w.D, 1, w.scale, stream)

        def call():
            st = fa.fa_bwd(*args)
            if st != fa.FA_OK:
                raise fa.FAError(st, "fa_bwd")

        avg, med, mn = _time_launches(call, max(3, steps // 2), 2)
        flops = 2.5 * w.flops(True)   # five products: S, dP, dV, dK, dQ (nominal)
        key = "backward_" + name
        out[key] = {"launch_ms_avg": round(avg, 5), "launch_ms_median": round(med, 5),
                    "tflops": round(flops / (avg * 1e-3) / 1e12, 2), "causal": True,
                    "flops_per_launch": flops}
        log(f"[bench] {key}: {avg:.4f} ms, {out[key]['tflops']} TFLOP/s (2.5x forward flops)")
        del q, k, v, do, o, lse, dq, dk, dv, delta
    for name, w in wl.MERGE_WORKLOADS.items():
        op, lp = (t.cuda() for t in wl.make_merge_inputs(w))
        o = torch.empty(op.shape[1:], dtype=torch.bfloat16, device="cuda")
        lse = torch.empty(lp.shape[1:], dtype=torch.float32, device="cuda")

        def call():
            fa.merge(op, lp, out=o, lse=lse)

        avg, med, mn = _time_launches(call, steps, 3)
        gbs = w.bytes_moved() / (avg * 1e-3) / 1e9
        out[name] = {"launch_ms_avg": round(avg, 5), "launch_ms_median": round(med, 5),
                     "bound": "hbm", "achieved_gbs": round(gbs, 1), "peak_gbs": PEAK_HBM_GBS,
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "bytes_per_launch": w.bytes_moved()}
        log(f"[bench] {name}: {avg:.4f} ms, {gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM)")
        del op, lp, o, lse
    return out


# The tile-pipeline study (the "Pipelining GmemCopy on kHeadDim" issue's
# questions): the bf16 forward with its K/V tiles copied one step ahead (the
# library), copied and waited for in the step that reads them, or copied two
# or three steps ahead into three or four buffers each, and the products with
# their operand reads alone (no copies, no exponentials); at D = 256 the
# library's wave-pair kernel against the one-wave ring kernel (ring256).
STUDY_WORKLOADS = (("c4_bf16_causal_1x32x16384x128", True), ("c3_bf16_2x16x4096x128", True),
                   ("c3_bf16_2x16x4096x128", False), ("c5_bf16_causal_2x8x8192x256_stress", True))


def pipeline_study(rounds=3):
    """TFLOP/s of each pipeline-study build against the library on the same
    inputs, alternating builds within each round (median over rounds)."""
    import ctypes
    import torch
    import exact_attention_67_amd as fa
    from exact_attention_67_amd import _lib
    from tests import workloads as wl

    libs = {"overlap (library)": fa.load()}
    for name in _lib.PIPE_VARIANTS:
        libs[name] = _lib.load_variant(name)
    stream = torch.cuda.current_stream()
    out = {}
    for name, causal in STUDY_WORKLOADS:
        w = wl.WORKLOADS[name]
        q, k, v = wl.make_inputs(w, device="cuda")
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.H, w.S), dtype=torch.float32, device="cuda")
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                w.B, w.H, w.S, w.D, int(causal), ctypes.c_float(w.scale), stream.cuda_stream)
        flops = w.flops(causal)
        times = {n: [] for n in libs}
        for r in range(rounds):
            for n, lib in libs.items():
                def launch():
                    st = lib.fa_fwd(*args)
                    if st != fa.FA_OK:
                        raise fa.FAError(st, f"fa_fwd ({n})")
                launch()
                torch.cuda.synchronize()
                t0 = time.perf_counter()
                launch()
                torch.cuda.synchronize()
                one = max(time.perf_counter() - t0, 1e-5)
                for _ in range(max(2, int(0.1 / one))):   # ~100 ms of warm-up
                    launch()
                n_t = max(5, int(0.05 / one))             # ~50 ms timed
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(n_t):
                    launch()
                e1.record(stream)
                torch.cuda.synchronize()
                times[n].append(e0.elapsed_time(e1) / n_t)
        key = f"{name}_{'causal' if causal else 'full'}"
        out[key] = {}
        for n in libs:
            ms = sorted(times[n])[len(times[n]) // 2]
            out[key][n] = {"ms": round(ms, 5), "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        log(f"[study] {key}: " + "  ".join(f"{n} {out[key][n]['tflops']}" for n in libs))
        del q, k, v, o, lse
        torch.cuda.empty_cache()
    return out


def cpu_baseline(w, causal, budget_s=20.0):
    """The oracle, as it stands, on the host cores over a bounded sample of the
    same workload: whole heads (row-blocked), one after another until the time
    budget is spent (or every head is done).  Torch runs one thread per host
    CPU this process may run on (all of them unless the process is pinned)."""
    import torch
    from oracle import attention as orc
    from tests import workloads as wl

    cores = os.cpu_count() or 1
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else cores
    torch.set_num_threads(max(1, usable))
    q, k, v = wl.make_inputs(w)
    flops_head = 4.0 * w.S * w.S * w.D * (0.5 if causal else 1.0)
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done, t_total = 0, 0.0
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        t = time.perf_counter()
        orc.attention_reference(q[sl], k[sl], v[sl], causal, w.scale, row_block=2048)
        t_total += time.perf_counter() - t
        done += 1
        if t_total >= budget_s:
            break
    return {
        "value": flops_head * done / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "cores_usable": usable,
        "threads": torch.get_num_threads(),
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} heads of {w.name} "
                  f"({'causal' if causal else 'non-causal'}), float64 torch CPU, "
                  f"row blocks of 2048, {t_total:.1f} s",
        "seconds_per_head": t_total / done,
    }


def copy_calibration():
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE /
    WRITE_SIZE readings (run under the same --pmc command as the bench)."""
    import torch
    n = 256 << 20  # bytes
    a = torch.empty(n // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[copy-calibration] copied {n} bytes x3 (read {n}, write {n} per copy)")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--noncausal", action="store_true", help="time the non-causal mask")
    ap.add_argument("--all", action="store_true", help="also time every workload (stderr)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the secondary figures (Sq != Sk, merge, backward)")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the cold-cache launches (profiling runs count warm launches only)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--pipeline-study", action="store_true",
                    help="also time the tile-pipeline study builds against the library "
                         "(TFLOP/s table on stderr, 'pipeline_study' in the JSON line)")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    a = ap.parse_args()

    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {a.gpus}); "
              "the forward is independent per (batch, head) and shards by head without "
              "collectives, but no multi-GPU path is built.", file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    from tests import workloads as wl
    if not torch.cuda.is_available():
        log("bench.py: no GPU visible")
        sys.exit(1)
    import exact_attention_67_amd as fa
    fa.load()

    if a.copy_calibration:
        copy_calibration()

    w = wl.WORKLOADS[a.workload]
    causal = (not a.noncausal) and (True in w.causal)
    # The headline inputs are made (on the host, then copied) before the
    # secondary figures, so that the headline launches follow those without
    # an idle gap (see the module docstring).
    inputs = wl.make_inputs(w, device="cuda")
    secondary = None if a.no_secondary else time_secondary(max(5, a.steps // 5))
    study = pipeline_study() if a.pipeline_study else None

    log(f"[bench] {w.name} causal={causal} steps={a.steps} warmup={a.warmup}")
    r = time_workload(w, causal, a.steps, a.warmup,
                      cold_launches=0 if a.no_cold else min(20, a.steps), inputs=inputs)
    flops = w.flops(causal)
    value = flops / (r["ms_per_step"] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
    achieved = flops / (r["launch_ms_avg"] * 1e-3) / 1e12
    log(f"[bench] ms/step={r['ms_per_step']:.4f} launch avg={r['launch_ms_avg']:.4f} "
        f"min={r['launch_ms_min']:.4f} med={r['launch_ms_med']:.4f} -> {value:.1f} TFLOP/s "
        f"({100 * value / peak:.1f}% of peak)")
    cold = None
    if "cold_ms_med" in r:
        cold_diff = 100.0 * (r["cold_ms_med"] - r["launch_ms_med"]) / r["launch_ms_med"]
        log(f"[bench] cold launch median {r['cold_ms_med']:.4f} ms ({cold_diff:+.1f}% vs warm)")
        if abs(cold_diff) > 5.0:
            log(f"[bench] warm and cold launches differ by {cold_diff:.1f}%")
        cold = {"evict_bytes": COLD_EVICT_BYTES,
                "launch_ms_median": round(r["cold_ms_med"], 5),
                "launch_ms_min": round(r["cold_ms_min"], 5),
                "cold_vs_warm_pct": round(cold_diff, 2)}
    sclk = recorded_profile_value(w.name, "sclk_mhz_under_load")

    if a.all:
        # Each workload: warm-up launches worth about 200 ms of GPU time (the
        # shader clock settles under load), then back-to-back launches as in
        # the headline line; the isolated per-launch average is shown beside.
        log(f"{'workload':40s} {'mask':7s} {'ms':>9s} {'TFLOP/s':>9s} {'%peak':>6s}"
            f" {'ms/launch pair':>15s}")
        for name in wl.ORDER:
            ww = wl.WORKLOADS[name]
            for c in ww.causal:
                probe = time_workload(ww, c, 3, 1)
                warm = max(3, min(2000, int(200.0 / max(probe["ms_per_step"], 1e-3))))
                steps = max(10, min(500, int(50.0 / max(probe["ms_per_step"], 1e-3))))
                rr = time_workload(ww, c, steps, warm)
                pk = PEAK_BF16_TFLOPS if ww.dtype == torch.bfloat16 else PEAK_F32_TFLOPS
                tf = ww.flops(c) / (rr["ms_per_step"] * 1e-3) / 1e12
                log(f"{name:40s} {'causal' if c else 'full':7s} {rr['ms_per_step']:9.4f} "
                    f"{tf:9.1f} {100 * tf / pk:6.1f} {rr['launch_ms_avg']:15.4f}")

    cpu = None
    if rank == 0 and not a.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample ...")
        cpu = cpu_baseline(w, causal, a.cpu_budget)
        log(f"[bench] cpu oracle: {cpu['value'] * 1e3:.1f} GFLOP/s on {cpu['threads']} threads "
            f"({cpu['cores']} host CPUs)")

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "S": w.S, "D": w.D,
                   "causal": causal, "scale": w.scale, "parallelism": "single-gpu"},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": recorded_traffic(w.name),
            "kernel": kernel_name(w, causal),
            "launch_ms_avg": round(r["launch_ms_avg"], 5),
            "launch_ms_median": round(r["launch_ms_med"], 5),
            "launch_ms_min": round(r["launch_ms_min"], 5),
            "flops_per_launch": flops,
            # peak scaled to the shader clock this kernel sustained (rocprofv3
            # counters over kernel time, committed summary), when available
            "sclk_mhz_under_load": sclk,
            "peak_at_sclk": round(peak * sclk / NOMINAL_SCLK_MHZ, 1) if sclk else None,
            "frac_at_sclk": round(achieved / (peak * sclk / NOMINAL_SCLK_MHZ), 4) if sclk else None,
        },
        "cold": cold,
        "cpu_baseline": cpu,
        # not part of `value`: the forward on the other workloads, the Sq != Sk
        # path, the merge and the backward pass, each on its own workloads
        "secondary": secondary,
    }
    if study is not None:
        # not part of `value`: the tile-pipeline study builds, same inputs
        line["pipeline_study"] = study
    if rank == 0:
        print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
