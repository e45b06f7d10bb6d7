#!/usr/bin/env python3
"""Benchmark of the exact attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--mode bf16]

A step is one pass of the whole path over one batch of resident inputs: one
fab_backward call with O and LSE left to the library (the op's own semantics:
mask block map, bf16 copies of K and V, forward with row LSE, D = rowsum(dO o
O), the key-block-outer dK/dV kernel, the query-block-outer dQ kernel, the
grouped-query reduction and the blob packing).  `value` counts the work that
pass must do: forward 2*N*M*(DK+DV)*H*B plus the backward 10*N*M*(DK+DV)/2*H*B,
each halved under a causal mask, over K steps timed with two HIP events on the
launch stream and nothing else in between (after at least W warm-up steps and
1 s of warm-up; the median of three such runs, the fastest run beside it).  The same K steps are then run
again with every kernel bracketed by HIP events (which adds gaps between the
kernels: `ms_per_step_with_kernel_events`) for every kernel's time per step
and its algorithmic rate (TFLOP/s for the matrix-core kernels, GB/s for the
memory-bound ones) and the `roofline` object of the dominant kernel.  The line
also reports the backward alone (O and LSE supplied by a prior forward, the
usual training convention; with its own per-kernel breakdown, whose "pack" is
the one launch that packs Q, K, V and preps d, O and the LSE) and the forward
alone, and (`other_workloads`,
--also) the whole step and the backward alone of further workloads, by
default the long-context one.  Causal workloads are also timed with the causal
rule passed as a flag instead of the mask tensor (`causal_flag_instead_of_mask`:
same result, no block map or mask reads), bf16 mode with q, k, v, d stored
as bf16 (`bf16_inputs`: the values the matrix cores read), and the other
arithmetic mode on the same workload (`other_mode`: f32 operands on the f32
matrix cores, priced against the f32 peak).  `cpu_baseline` times the
f64 CPU oracle on a bounded sample of the same workload on this host's cores.

Prints exactly one JSON line.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import fab_inputs as fi  # noqa: E402

# HBM bytes of the dominant kernel measured by rocprofv3 counters (FETCH_SIZE and
# WRITE_SIZE, scaled by the same counters on a copy kernel of known size), with a
# hash of the sources they were taken on; reported only while the sources match.
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_backward_causal_gqa_B1_H32x8_N2048_D128_bf16.json")
KERNEL_SOURCES = ("fab_bwd.hip", "fab_tiles.h", "fab_common.h")


def source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "exact_attention_backward_fab_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel or t.get("workload") != workload or t.get("source_hash") != source_hash():
        return None
    return t.get("bytes_per_launch")

METRIC = "attention-backward TFLOP/s and % of MFMA peak (bf16 and fp32 modes), 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # MI355X dense matrix peaks (published)
HBM_GBS = 8000.0


def fwd_flops(s, causal):
    f = 2.0 * s.N * s.M * (s.DK + s.DV) * s.H * s.B
    return f / 2 if causal else f


def bwd_flops(s, causal):
    f = 10.0 * s.N * s.M * (s.DK + s.DV) / 2.0 * s.H * s.B
    return f / 2 if causal else f


def kernel_work(s, causal, mode, has_mask):
    """Algorithmic work of one launch-set of each kernel in a step: (amount,
    unit), flops for the matrix-core kernels and bytes for the memory-bound
    ones.  A causal mask halves the (query, key) pairs the contractions visit."""
    half = 0.5 if causal else 1.0
    pairs = float(s.N) * s.M * s.H * s.B * half
    bf16 = mode == "bf16"
    rows = float(s.N) * s.H * s.B
    # padded head dims of the bf16 copies: the first instantiated pair covering (DK, DV)
    dkp, dvp = next((a, b) for a, b in ((32, 32), (64, 64), (128, 128), (192, 128), (192, 192))
                    if s.DK <= a and s.DV <= b)
    mp = (s.M + 63) // 64 * 64
    np_ = (s.N + 63) // 64 * 64
    dq_from_ds = bf16 and dkp + dvp <= 256 and s.B * s.H * (np_ // 64) * math.ceil(s.M / 128) * 16384 <= 4 << 30
    w = {
        # S = Q K^T and O = P V
        "forward": (2.0 * pairs * (s.DK + s.DV), "flop"),
        # bf16: S, dP, dV, dK; f32: also dQ (atomics)
        "backward": (2.0 * pairs * ((2 * s.DK + 2 * s.DV) if bf16 else (3 * s.DK + 2 * s.DV)), "flop"),
        # dQ: from the dS^T tiles the dK/dV kernel stores (head-dim pairs up to
        # 128/128 and tiles within 4 GiB, as the library decides) a memory-bound
        # product that reads 2 bytes of dS per visited pair and writes dQ, with the
        # grouped-query reduction of dK and dV in the same launch; otherwise S, dP
        # and dQ by the recompute kernel
        "dq": ((2.0 * pairs + 4.0 * rows * s.DK
                + (4.0 * s.M * (s.DK + s.DV) * s.B * (s.H + s.Hkv) if s.H > s.Hkv else 0.0), "byte")
               if dq_from_ds else (2.0 * pairs * (2 * s.DK + s.DV), "flop")),
        "block_map": (2.0 * s.M * s.N + math.ceil(s.N / 32) * math.ceil(s.M / 32), "byte"),
        # bf16: read d, O and the LSE, write the bf16 dO tiles and the LSE/D blocks;
        # f32: read d and O, write D and zero the dQ slice
        "prep": ((rows * (8.0 * s.DV + 4.0) + s.H * s.B * (np_ * dvp * 2.0 + np_ / 64 * 512.0)) if bf16
                 else rows * (8.0 * s.DV + 4.0) + rows * s.DK * 4.0, "byte"),
        # (the whole step, bf16) read K, V in f32, write the bf16 tiles, and, with a
        # mask, read it and write its block map in the same launch
        "pack": (s.Hkv * s.B * (4.0 * s.M * (s.DK + s.DV) + 2.0 * mp * (dkp + dvp))
                 + ((2.0 * s.M * s.N + math.ceil(s.N / 32) * math.ceil(s.M / 32)) if has_mask else 0.0), "byte"),
        # read per-query-head partials, write per-group sums
        "gqa_reduce": (4.0 * s.M * (s.DK + s.DV) * s.B * (s.H + s.Hkv), "byte"),
        # (the backward alone, bf16) the pack of Q, K, V (f32 read, bf16 tiles
        # written) with the block map, and the prep of d, O and the LSE (dO tiles
        # and LSE/D blocks written), one launch
        "pack_prep": (s.B * (s.H * 4.0 * s.N * s.DK + s.Hkv * 4.0 * s.M * (s.DK + s.DV))
                      + s.B * (s.H * 2.0 * np_ * dkp + s.Hkv * 2.0 * mp * (dkp + dvp))
                      + ((2.0 * s.M * s.N + math.ceil(s.N / 32) * math.ceil(s.M / 32)) if has_mask else 0.0)
                      + rows * (8.0 * s.DV + 4.0) + s.H * s.B * (np_ * dvp * 2.0 + np_ / 64 * 512.0), "byte"),
    }
    return w


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=3, choices=sorted(fi.WORKLOADS))
    ap.add_argument("--mode", default=None, choices=["f32", "bf16"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--also", default="4",
                    help="comma-separated workloads also timed (whole step and backward alone), '' for none")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--min-warm-s", type=float, default=1.0,
                    help="warm-up of every timed loop lasts at least this long (seconds of GPU work)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="run one 256 MiB device-to-device copy before the timed region (the known-size "
                         "reference of the HBM byte counters)")
    return ap.parse_args()


def time_loop(torch, fn, steps, warmup, stream, min_warm_s=1.0, repeats=3, stats=None):
    # warm-up: at least `warmup` steps and at least min_warm_s of GPU work (the
    # chip's clocks settle over the first tens of milliseconds of load)
    t0 = time.perf_counter()
    i = 0
    while i < warmup or time.perf_counter() - t0 < min_warm_s:
        fn()
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # three back-to-back timed runs of `steps` steps each; the median run counts
    runs = []
    for _ in range(repeats):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(steps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / steps)
    if stats is not None:
        stats["min"] = min(runs)
    return sorted(runs)[len(runs) // 2]


def cpu_baseline(s, q, k, v, d, mask, scale, causal, budget_s):
    """The oracle, as it stands, on a bounded sample of the workload: whole
    key/value groups (b, g) with all their H/Hkv query heads, as many as fit the
    time budget (all of them when they do), else the first queries of group 0.
    Counted like `value`: forward plus backward flops of the (query, key) pairs
    attended."""
    from oracle import oracle as orc
    rk2 = s.H // s.Hkv
    cores = orc.default_threads()

    def group(b, g, n_keep):
        sub = fi.Shape(1, rk2, 1, n_keep, s.M, s.DK, s.DV)
        args = (np.ascontiguousarray(q[b:b + 1, g * rk2:(g + 1) * rk2, :n_keep]),
                np.ascontiguousarray(k[b:b + 1, g:g + 1]), np.ascontiguousarray(v[b:b + 1, g:g + 1]),
                None if mask is None else np.ascontiguousarray(mask[:n_keep]),
                np.ascontiguousarray(d[b:b + 1, :n_keep, g * rk2:(g + 1) * rk2]))
        return sub, args

    # calibration on the first 64 queries of group 0
    n_cal = min(s.N, 64)
    sub, a = group(0, 0, n_cal)
    t0 = time.perf_counter()
    orc.backward(sub, a[0], a[1], a[2], a[3], a[4], scale)
    per_row = (time.perf_counter() - t0) / n_cal
    units = [(b, g) for b in range(s.B) for g in range(s.Hkv)]
    per_group = per_row * s.N
    if per_group <= budget_s:
        units = units[:max(1, min(len(units), int(budget_s / per_group)))]
        n_keep = s.N
    else:
        units = units[:1]
        n_keep = max(64, min(s.N, int(budget_s / per_row)))
    t0 = time.perf_counter()
    for b, g in units:
        sub, a = group(b, g, n_keep)
        orc.backward(sub, a[0], a[1], a[2], a[3], a[4], scale)
    dt = time.perf_counter() - t0
    if causal:
        pairs = sum(min(n + 1, s.M) for n in range(n_keep))
    else:
        pairs = n_keep * s.M
    pairs *= rk2 * len(units)
    flops = pairs * (2.0 * (s.DK + s.DV) + 5.0 * (s.DK + s.DV))
    what = (f"{len(units)} of {len(units) if n_keep < s.N else s.B * s.Hkv} key/value groups" if n_keep == s.N
            else f"key/value group 0, queries 0..{n_keep - 1} of {s.N}")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{what} ({rk2} query heads each, all {s.M} keys); f64 forward + backward, "
                      f"counted as the forward plus the backward flops of the attended pairs"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the split of this path "
              f"over several GPUs (by key/value head group) is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_attention_backward_fab_amd as fab

    w = fi.WORKLOADS[args.workload]
    mode = args.mode or ("bf16" if "bf16" in w.modes else w.modes[0])
    causal = w.mask == "causal"
    s, q, k, v, d, mask, scale = fi.workload_inputs(args.workload)
    dev = torch.device("cuda:0")
    tq, tk, tv, td = (torch.from_numpy(x).to(dev) for x in (q, k, v, d))
    tm = None if mask is None else torch.from_numpy(mask.view(np.int16)).to(dev)
    fs = fab.Shape(*s.astuple())
    total = fab.blob_layout(fs)[3]
    blob = torch.empty(total, dtype=torch.float32, device=dev)
    O = torch.empty((s.B, s.N, s.H, s.DV), dtype=torch.float32, device=dev)
    lse = torch.empty((s.B, s.H, s.N), dtype=torch.float32, device=dev)
    ws_full, _ = fab.alloc_workspace(fs, mode, tm is not None, False, dev)
    ws_bwd, _ = fab.alloc_workspace(fs, mode, tm is not None, True, dev)
    stream = torch.cuda.current_stream()

    def step_full():
        fab.backward(tq, tk, tv, td, scale, mask=tm, mode=mode, blob=blob, ws=ws_full)

    def step_bwd():
        fab.backward(tq, tk, tv, td, scale, mask=tm, mode=mode, O=O, lse=lse, blob=blob, ws=ws_bwd)

    def step_fwd():
        fab.forward_lse(tq, tk, tv, scale, mask=tm, mode=mode, O=O, lse=lse, ws=ws_bwd)

    if args.calib_copy:
        a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # ---- timed region: the whole path, K steps with nothing but the launches
    st_step, st_bwd = {}, {}
    ms_step = time_loop(torch, step_full, args.steps, args.warmup, stream, args.min_warm_s, stats=st_step)
    # ---- the same K steps again with every kernel bracketed by HIP events on its
    # launch stream: per-kernel durations (the event records add gaps between the
    # kernels, so this pass is not the one `value` is taken from)
    fab.profile_reset()
    fab.profile_enable(True)
    ms_step_prof = time_loop(torch, step_full, args.steps, 0, stream, min_warm_s=0.0, repeats=1)
    prof = fab.profile_read()
    fab.profile_enable(False)
    fab.profile_reset()

    # ---- the backward alone (O, LSE from a prior forward) and the forward alone
    step_fwd()
    torch.cuda.synchronize()
    ms_bwd = time_loop(torch, step_bwd, args.steps, args.warmup, stream, args.min_warm_s, stats=st_bwd)
    # per-kernel durations of the backward alone (events around every launch, as above)
    fab.profile_reset()
    fab.profile_enable(True)
    time_loop(torch, step_bwd, args.steps, 0, stream, min_warm_s=0.0, repeats=1)
    prof_bwd = fab.profile_read()
    fab.profile_enable(False)
    fab.profile_reset()
    ms_fwd = time_loop(torch, step_fwd, args.steps, args.warmup, stream, args.min_warm_s)

    F_f, F_b = fwd_flops(s, causal), bwd_flops(s, causal)
    peak = PEAK_TFLOPS[mode]
    work = kernel_work(s, causal, mode, mask is not None)

    def per_kernel(pr, work):
        out = {}
        for name, (tot_ms, launches) in pr.items():
            if not launches:
                continue
            ms = tot_ms / args.steps                       # per step (all launches of the kernel)
            amount, kind = work[name]
            if kind == "flop":
                rate = amount / (ms * 1e-3) / 1e12
                out[name] = {"ms": round(ms, 4), "launches_per_step": launches // args.steps,
                             "achieved": round(rate, 2), "unit": "TFLOP/s", "frac": round(rate / peak, 4)}
            else:
                rate = amount / (ms * 1e-3) / 1e9
                out[name] = {"ms": round(ms, 4), "launches_per_step": launches // args.steps,
                             "achieved": round(rate, 1), "unit": "GB/s", "frac": round(rate / HBM_GBS, 4)}
        return out

    kernels = per_kernel(prof, work)
    # in the backward alone, "pack" is the launch that packs Q, K, V and builds the
    # block map together with the prep of the supplied O and LSE (bf16), and "prep"
    # is D alone (f32)
    kernels_bwd = per_kernel(prof_bwd, dict(work, pack=work["pack_prep"]))
    dom = max(kernels, key=lambda n: kernels[n]["ms"])
    dom_launch_ms = prof[dom][0] / prof[dom][1]
    dom_amount, dom_kind = work[dom]
    per_launch = dom_amount / max(prof[dom][1] // args.steps, 1)
    if dom_kind == "flop":
        ach = per_launch / (dom_launch_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": measured_traffic(dom, w.name), "per_launch_flops": per_launch,
                "avg_launch_ms": round(dom_launch_ms, 5)}
    else:
        ach = per_launch / (dom_launch_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_GBS, 4), "traffic": measured_traffic(dom, w.name), "per_launch_bytes": per_launch,
                "avg_launch_ms": round(dom_launch_ms, 5)}

    out = {
        "metric": METRIC,
        "value": round((F_f + F_b) / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_min": round(st_step["min"], 4),
        "ms_per_step_with_kernel_events": round(ms_step_prof, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mode,
        "data": "synthetic",
        "config": {"workload": w.name, "B": s.B, "H": s.H, "Hkv": s.Hkv, "N": s.N, "M": s.M,
                   "DK": s.DK, "DV": s.DV, "mask": w.mask, "mode": mode, "scale": scale,
                   "step": "fab_backward with internal forward (whole path)"},
        "frac_of_peak": round((F_f + F_b) / (ms_step * 1e-3) / 1e12 / peak, 4),
        "backward_only": {"ms": round(ms_bwd, 4), "ms_min": round(st_bwd["min"], 4),
                          "tflops": round(F_b / (ms_bwd * 1e-3) / 1e12, 3),
                          "frac_of_peak": round(F_b / (ms_bwd * 1e-3) / 1e12 / peak, 4),
                          "flops_counted": F_b, "kernels": kernels_bwd},
        "forward_only": {"ms": round(ms_fwd, 4), "tflops": round(F_f / (ms_fwd * 1e-3) / 1e12, 3),
                         "frac_of_peak": round(F_f / (ms_fwd * 1e-3) / 1e12 / peak, 4)},
        "kernels": kernels,
        "roofline": roof,
    }
    # ---- the same step with the causal rule given as a flag instead of the mask
    # tensor (identical result; no block map, no mask reads)
    mask_free = None
    if causal:
        ws_c, _ = fab.alloc_workspace(fs, mode, False, False, dev, causal=True)
        ms_c = time_loop(torch, lambda: fab.backward(tq, tk, tv, td, scale, mode=mode, blob=blob, ws=ws_c,
                                                     causal=True), args.steps, args.warmup, stream, args.min_warm_s)
        mask_free = {"ms_per_step": round(ms_c, 4), "value": round((F_f + F_b) / (ms_c * 1e-3) / 1e12, 3),
                     "frac_of_peak": round((F_f + F_b) / (ms_c * 1e-3) / 1e12 / peak, 4)}
        del ws_c

    # ---- the same step with q, k, v, d stored as bf16 (bf16 mode: the values the
    # matrix cores read; the f32 inputs rounded once beforehand, outside the timing)
    bf16_in = None
    if mode == "bf16":
        tb = [x.to(torch.bfloat16) for x in (tq, tk, tv, td)]
        ms_b = time_loop(torch, lambda: fab.backward(*tb, scale, mask=tm, mode=mode, blob=blob, ws=ws_full),
                         args.steps, args.warmup, stream, args.min_warm_s)
        bf16_in = {"ms_per_step": round(ms_b, 4), "value": round((F_f + F_b) / (ms_b * 1e-3) / 1e12, 3),
                   "frac_of_peak": round((F_f + F_b) / (ms_b * 1e-3) / 1e12 / peak, 4)}
        del tb

    # ---- the other arithmetic mode on the same workload (f32 operands on the f32
    # matrix cores, priced against the f32 peak), whole step and backward alone
    other_mode = None
    om = "f32" if mode == "bf16" else "bf16"
    if om in w.modes or om == "f32":
        ws_o, _ = fab.alloc_workspace(fs, om, tm is not None, False, dev)
        ws_ob, _ = fab.alloc_workspace(fs, om, tm is not None, True, dev)
        O_o, lse_o = fab.forward_lse(tq, tk, tv, scale, mask=tm, mode=om, ws=ws_ob)
        ms_o = time_loop(torch, lambda: fab.backward(tq, tk, tv, td, scale, mask=tm, mode=om, blob=blob, ws=ws_o),
                         args.steps, args.warmup, stream, args.min_warm_s)
        ms_ob = time_loop(torch, lambda: fab.backward(tq, tk, tv, td, scale, mask=tm, mode=om, O=O_o, lse=lse_o,
                                                      blob=blob, ws=ws_ob), args.steps, args.warmup, stream,
                          args.min_warm_s)
        pk = PEAK_TFLOPS[om]
        other_mode = {"mode": om, "ms_per_step": round(ms_o, 4),
                      "value": round((F_f + F_b) / (ms_o * 1e-3) / 1e12, 3),
                      "frac_of_peak": round((F_f + F_b) / (ms_o * 1e-3) / 1e12 / pk, 4), "peak": pk,
                      "backward_only": {"ms": round(ms_ob, 4), "tflops": round(F_b / (ms_ob * 1e-3) / 1e12, 3),
                                        "frac_of_peak": round(F_b / (ms_ob * 1e-3) / 1e12 / pk, 4)}}
        del ws_o, ws_ob, O_o, lse_o

    # ---- other workloads (e.g. the long-context one), same protocol, same mode
    also = {}
    for wid in [int(x) for x in args.also.split(",") if x.strip()]:
        if wid == args.workload:
            continue
        w2 = fi.WORKLOADS[wid]
        if mode not in w2.modes:
            continue
        s2, q2, k2, v2, d2, mask2, scale2 = fi.workload_inputs(wid)
        c2 = w2.mask == "causal"
        t2 = [torch.from_numpy(x).to(dev) for x in (q2, k2, v2, d2)]
        tm2 = None if mask2 is None else torch.from_numpy(mask2.view(np.int16)).to(dev)
        fs2 = fab.Shape(*s2.astuple())
        blob2 = torch.empty(fab.blob_layout(fs2)[3], dtype=torch.float32, device=dev)
        ws2, _ = fab.alloc_workspace(fs2, mode, tm2 is not None, False, dev)
        ws2b, _ = fab.alloc_workspace(fs2, mode, tm2 is not None, True, dev)
        O2, lse2 = fab.forward_lse(t2[0], t2[1], t2[2], scale2, mask=tm2, mode=mode, ws=ws2b)
        ms2 = time_loop(torch, lambda: fab.backward(*t2, scale2, mask=tm2, mode=mode, blob=blob2, ws=ws2),
                        args.steps, args.warmup, stream, args.min_warm_s)
        ms2b = time_loop(torch, lambda: fab.backward(*t2, scale2, mask=tm2, mode=mode, O=O2, lse=lse2, blob=blob2,
                                                     ws=ws2b), args.steps, args.warmup, stream, args.min_warm_s)
        ms2c = None
        if c2:
            ws2c, _ = fab.alloc_workspace(fs2, mode, False, False, dev, causal=True)
            ms2c = time_loop(torch, lambda: fab.backward(*t2, scale2, mode=mode, blob=blob2, ws=ws2c, causal=True),
                             args.steps, args.warmup, stream, args.min_warm_s)
            del ws2c
        Ff2, Fb2 = fwd_flops(s2, c2), bwd_flops(s2, c2)
        also[w2.name] = {"ms_per_step": round(ms2, 4), "value": round((Ff2 + Fb2) / (ms2 * 1e-3) / 1e12, 3),
                         "frac_of_peak": round((Ff2 + Fb2) / (ms2 * 1e-3) / 1e12 / peak, 4),
                         "backward_only": {"ms": round(ms2b, 4), "tflops": round(Fb2 / (ms2b * 1e-3) / 1e12, 3),
                                           "frac_of_peak": round(Fb2 / (ms2b * 1e-3) / 1e12 / peak, 4)}}
        if ms2c:
            also[w2.name]["causal_flag_instead_of_mask"] = {
                "ms_per_step": round(ms2c, 4), "value": round((Ff2 + Fb2) / (ms2c * 1e-3) / 1e12, 3)}
        del t2, tm2, blob2, ws2, ws2b, O2, lse2
    if mask_free:
        out["causal_flag_instead_of_mask"] = mask_free
    if bf16_in:
        out["bf16_inputs"] = bf16_in
    if other_mode:
        out["other_mode"] = other_mode
    if also:
        out["other_workloads"] = also
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(s, q, k, v, d, mask, scale, causal, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
