#!/usr/bin/env python3
"""Benchmark of the exact attention backward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 3] [--mode bf16]
    python bench.py --only backward|whole|forward ...   (one timed loop, for profilers)

A step is one fab_backward call over one batch of resident inputs with O and the
row LSE supplied by a prior fab_forward_lse (the usual training convention): the
pack of Q, K, V to bf16 tiles with the block map of the mask and the prep of d, O
and the LSE (D = rowsum(dO o O)), the key-block-outer dK/dV kernel, the dQ kernel,
the grouped-query reduction and the blob packing.  `value` counts the backward's
work, 10*N*M*(DK+DV)/2*H*B (halved under a causal mask), over K steps timed with
two HIP events on the launch stream and nothing else in between (after at least W
warm-up steps and 1 s of warm-up; the median of three such runs, the fastest run
beside it), and `frac_of_peak` prices it against the dense matrix-core peak of the
mode.  The same K steps are then run again with every kernel bracketed by HIP
events on its launch stream (which adds gaps between the kernels) for every
kernel's time and algorithmic rate (TFLOP/s for the matrix-core kernels, GB/s for
the memory-bound ones) and the `roofline` object of the dominant kernel.

Beside it: `whole_path`, the op's own semantics (O = lse = NULL: the forward runs
inside fab_backward, counted as forward plus backward flops); `forward_only`;
causal workloads with the causal rule passed as a flag instead of the mask tensor
(`causal_flag_instead_of_mask`); bf16 mode with q, k, v, d stored as bf16
(`bf16_inputs`), with O stored as bf16 as well (`bf16_storage`) and with the result
blob as bf16 too (`bf16_storage_and_blob`), or stored as f16 (`f16_inputs`); and `configs`: every other (workload, mode) pair of the five
workloads, each with its backward alone (and kernel split), whole path and
fraction of its mode's peak.  `mfma_loop_ceiling` (bf16 mode) is the rate of a
loop of dense bf16 products on every SIMD, with the shader clock it runs at: the
practical ceiling of the matrix cores, beside the published peak that `roofline`
and `frac_of_peak` use.  `cpu_baseline` times the f64 CPU oracle on a
bounded sample of the headline workload on this host's cores.

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
    dq_from_ds = bf16 and s.B * s.H * (np_ // 64) * math.ceil(s.M / 128) * 16384 < 4 << 30
    w = {
        # S = Q K^T and O = P V
        "forward": (2.0 * pairs * (s.DK + s.DV), "flop"),
        # bf16: S, dP, dV, dK; f32: also dQ (atomics)
        "backward": (2.0 * pairs * ((2 * s.DK + 2 * s.DV) if bf16 else (3 * s.DK + 2 * s.DV)), "flop"),
        # dQ: from the dS^T tiles the dK/dV kernel stores (tiles within 4 GiB, as the
        # library decides) a memory-bound
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
    ap.add_argument("--configs", default="all",
                    help="(workload:mode) pairs also timed, comma-separated, e.g. '2:f32,5:bf16'; "
                         "'all' for every pair the five workloads list, '' for none")
    ap.add_argument("--only", default=None, choices=["backward", "whole", "forward"],
                    help="run only the warm-up and K timed steps of one call (backward alone, whole path "
                         "or forward) and print its time: the command profilers wrap")
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
    Counted like `value`: the backward's flops of the (query, key) pairs attended
    (the oracle also recomputes the forward it needs, as the GPU path's supplied O
    and LSE spare it)."""
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
    flops = pairs * 5.0 * (s.DK + s.DV)   # the backward's count per attended pair, as `value`
    what = (f"{len(units)} of {len(units) if n_keep < s.N else s.B * s.Hkv} key/value groups" if n_keep == s.N
            else f"key/value group 0, queries 0..{n_keep - 1} of {s.N}")
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": round(dt, 3),
            "sample": f"{what} ({rk2} query heads each, all {s.M} keys); f64 forward recompute + backward, "
                      f"counted as `value` counts the backward: 10*(DK+DV)/2 flops per attended pair"}


def per_kernel(pr, work, steps, peak):
    out = {}
    for name, (tot_ms, launches) in pr.items():
        if not launches:
            continue
        ms = tot_ms / steps                            # per step (all launches of the kernel)
        amount, kind = work[name]
        if kind == "flop":
            rate = amount / (ms * 1e-3) / 1e12
            out[name] = {"ms": round(ms, 4), "launches_per_step": launches // steps,
                         "achieved": round(rate, 2), "unit": "TFLOP/s", "frac": round(rate / peak, 4)}
        else:
            rate = amount / (ms * 1e-3) / 1e9
            out[name] = {"ms": round(ms, 4), "launches_per_step": launches // steps,
                         "achieved": round(rate, 1), "unit": "GB/s", "frac": round(rate / HBM_GBS, 4)}
    return out


def profiled(torch, fab, fn, steps, stream):
    """The same steps once more with every kernel bracketed by HIP events on its
    launch stream: {kernel: (total_ms, launches)} and the step time of that pass."""
    fab.profile_reset()
    fab.profile_enable(True)
    ms = time_loop(torch, fn, steps, 0, stream, min_warm_s=0.0, repeats=1)
    pr = fab.profile_read()
    fab.profile_enable(False)
    fab.profile_reset()
    return pr, ms


class Case:
    """Device inputs and buffers of one (workload, mode) pair, and its three calls."""

    def __init__(self, torch, fab, dev, wid, mode):
        w = fi.WORKLOADS[wid]
        self.w, self.mode, self.causal = w, mode, w.mask == "causal"
        s, q, k, v, d, mask, scale = fi.workload_inputs(wid)
        self.s, self.scale, self.host = s, scale, (q, k, v, d, mask)
        self.t = [torch.from_numpy(x).to(dev) for x in (q, k, v, d)]
        self.tm = None if mask is None else torch.from_numpy(mask.view(np.int16)).to(dev)
        self.fs = fab.Shape(*s.astuple())
        self.blob = torch.empty(fab.blob_layout(self.fs)[3], dtype=torch.float32, device=dev)
        self.O = torch.empty((s.B, s.N, s.H, s.DV), dtype=torch.float32, device=dev)
        self.lse = torch.empty((s.B, s.H, s.N), dtype=torch.float32, device=dev)
        self.ws_full, _ = fab.alloc_workspace(self.fs, mode, self.tm is not None, False, dev)
        self.ws_bwd, _ = fab.alloc_workspace(self.fs, mode, self.tm is not None, True, dev)
        self.fab = fab
        self.fwd()

    def fwd(self):
        t = self.t
        self.fab.forward_lse(t[0], t[1], t[2], self.scale, mask=self.tm, mode=self.mode, O=self.O, lse=self.lse,
                             ws=self.ws_bwd)

    def bwd(self):
        self.fab.backward(*self.t, self.scale, mask=self.tm, mode=self.mode, O=self.O, lse=self.lse, blob=self.blob,
                          ws=self.ws_bwd)

    def whole(self):
        self.fab.backward(*self.t, self.scale, mask=self.tm, mode=self.mode, blob=self.blob, ws=self.ws_full)

    def flops(self):
        return fwd_flops(self.s, self.causal), bwd_flops(self.s, self.causal)


def pair_summary(torch, fab, c, args, stream):
    """Backward alone (with its kernel split), whole path and forward of one pair."""
    F_f, F_b = c.flops()
    peak = PEAK_TFLOPS[c.mode]
    ms_b = time_loop(torch, c.bwd, args.steps, args.warmup, stream, args.min_warm_s)
    pr, _ = profiled(torch, fab, c.bwd, args.steps, stream)
    ms_w = time_loop(torch, c.whole, args.steps, args.warmup, stream, args.min_warm_s)
    work = kernel_work(c.s, c.causal, c.mode, c.tm is not None)
    return {"workload": c.w.name, "mode": c.mode, "peak": peak,
            "backward_only": {"ms": round(ms_b, 4), "tflops": round(F_b / (ms_b * 1e-3) / 1e12, 3),
                              "frac_of_peak": round(F_b / (ms_b * 1e-3) / 1e12 / peak, 4),
                              "kernels": per_kernel(pr, dict(work, pack=work["pack_prep"]), args.steps, peak)},
            "whole_path": {"ms": round(ms_w, 4), "tflops": round((F_f + F_b) / (ms_w * 1e-3) / 1e12, 3),
                           "frac_of_peak": round((F_f + F_b) / (ms_w * 1e-3) / 1e12 / peak, 4)}}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the split of this path "
              f"over several GPUs (by key/value head group) is not built.", file=sys.stderr)
        sys.exit(2)
    import torch
    import exact_attention_backward_fab_amd as fab

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    w = fi.WORKLOADS[args.workload]
    mode = args.mode or ("bf16" if "bf16" in w.modes else w.modes[0])
    c = Case(torch, fab, dev, args.workload, mode)
    s, causal = c.s, c.causal
    F_f, F_b = c.flops()
    peak = PEAK_TFLOPS[mode]

    if args.calib_copy:
        a = torch.empty(64 << 20, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    if args.only:
        fn, flops = {"backward": (c.bwd, F_b), "whole": (c.whole, F_f + F_b), "forward": (c.fwd, F_f)}[args.only]
        ms = time_loop(torch, fn, args.steps, args.warmup, stream, args.min_warm_s, repeats=1)
        print(json.dumps({"only": args.only, "workload": w.name, "mode": mode, "steps": args.steps,
                          "ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 3)}),
              flush=True)
        return

    # ---- timed region: the backward alone, K steps with nothing but its launches
    st_bwd, st_whole = {}, {}
    ms_bwd = time_loop(torch, c.bwd, args.steps, args.warmup, stream, args.min_warm_s, stats=st_bwd)
    # ---- the same K steps with every kernel bracketed by HIP events (per-kernel times)
    prof_bwd, ms_bwd_prof = profiled(torch, fab, c.bwd, args.steps, stream)
    # ---- the whole path (forward inside the call) and the forward alone
    ms_whole = time_loop(torch, c.whole, args.steps, args.warmup, stream, args.min_warm_s, stats=st_whole)
    prof_whole, _ = profiled(torch, fab, c.whole, args.steps, stream)
    ms_fwd = time_loop(torch, c.fwd, args.steps, args.warmup, stream, args.min_warm_s)

    work = kernel_work(s, causal, mode, c.tm is not None)
    # in the backward alone "pack" is the launch that packs Q, K, V and builds the
    # block map together with the prep of the supplied O and LSE (bf16); "prep" is D
    # alone (f32)
    work_bwd = dict(work, pack=work["pack_prep"])
    kernels_bwd = per_kernel(prof_bwd, work_bwd, args.steps, peak)
    kernels_whole = per_kernel(prof_whole, work, args.steps, peak)
    dom = max(kernels_bwd, key=lambda n: kernels_bwd[n]["ms"])
    dom_launch_ms = prof_bwd[dom][0] / prof_bwd[dom][1]
    dom_amount, dom_kind = work_bwd[dom]
    per_launch = dom_amount / max(prof_bwd[dom][1] // args.steps, 1)
    if dom_kind == "flop":
        ach = per_launch / (dom_launch_ms * 1e-3) / 1e12
        roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 3), "peak": peak, "unit": "TFLOP/s",
                "frac": round(ach / peak, 4), "traffic": measured_traffic(dom, w.name), "per_launch_flops": per_launch,
                "avg_launch_ms": round(dom_launch_ms, 5)}
    else:
        ach = per_launch / (dom_launch_ms * 1e-3) / 1e9
        roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_GBS, 4), "traffic": measured_traffic(dom, w.name),
                "per_launch_bytes": per_launch, "avg_launch_ms": round(dom_launch_ms, 5)}

    value = F_b / (ms_bwd * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_bwd, 4),
        "ms_per_step_min": round(st_bwd["min"], 4),
        "ms_per_step_with_kernel_events": round(ms_bwd_prof, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": mode,
        "data": "synthetic",
        "config": {"workload": w.name, "B": s.B, "H": s.H, "Hkv": s.Hkv, "N": s.N, "M": s.M,
                   "DK": s.DK, "DV": s.DV, "mask": w.mask, "mode": mode, "scale": c.scale,
                   "step": "fab_backward with O and LSE supplied (the backward alone)",
                   "flops_counted": F_b},
        "frac_of_peak": round(value / peak, 4),
        "kernels": kernels_bwd,
        "roofline": roof,
        "whole_path": {"ms": round(ms_whole, 4), "ms_min": round(st_whole["min"], 4),
                       "tflops": round((F_f + F_b) / (ms_whole * 1e-3) / 1e12, 3),
                       "frac_of_peak": round((F_f + F_b) / (ms_whole * 1e-3) / 1e12 / peak, 4),
                       "flops_counted": F_f + F_b, "kernels": kernels_whole},
        "forward_only": {"ms": round(ms_fwd, 4), "tflops": round(F_f / (ms_fwd * 1e-3) / 1e12, 3),
                         "frac_of_peak": round(F_f / (ms_fwd * 1e-3) / 1e12 / peak, 4)},
    }
    # ---- the practical ceiling of the matrix cores: a loop of dense bf16 products on
    # every SIMD (the chip lowers its clock under this load); context for `roofline`
    if mode == "bf16":
        tf_loop, ghz_loop = fab.measure_mfma_loop(iters=20000)
        out["mfma_loop_ceiling"] = {"tflops": round(tf_loop, 1), "clock_ghz": round(ghz_loop, 3),
                                    "frac_of_published_peak": round(tf_loop / peak, 4),
                                    "dominant_kernel_frac_of_ceiling": round(roof["achieved"] / tf_loop, 4)
                                    if roof["unit"] == "TFLOP/s" else None}
    tq, tk, tv, td = c.t
    # ---- the causal rule given as a flag instead of the mask tensor (identical
    # result; no block map, no mask reads), backward alone and whole path
    if causal:
        ws_c, _ = fab.alloc_workspace(c.fs, mode, False, True, dev, causal=True)
        ws_cw, _ = fab.alloc_workspace(c.fs, mode, False, False, dev, causal=True)
        ms_c = time_loop(torch, lambda: fab.backward(tq, tk, tv, td, c.scale, mode=mode, O=c.O, lse=c.lse,
                                                     blob=c.blob, ws=ws_c, causal=True),
                         args.steps, args.warmup, stream, args.min_warm_s)
        ms_cw = time_loop(torch, lambda: fab.backward(tq, tk, tv, td, c.scale, mode=mode, blob=c.blob, ws=ws_cw,
                                                      causal=True), args.steps, args.warmup, stream, args.min_warm_s)
        out["causal_flag_instead_of_mask"] = {
            "backward_only": {"ms": round(ms_c, 4), "tflops": round(F_b / (ms_c * 1e-3) / 1e12, 3),
                              "frac_of_peak": round(F_b / (ms_c * 1e-3) / 1e12 / peak, 4)},
            "whole_path": {"ms": round(ms_cw, 4), "tflops": round((F_f + F_b) / (ms_cw * 1e-3) / 1e12, 3)}}
        del ws_c, ws_cw
        c.fwd()
    # ---- q, k, v, d stored as bf16 (bf16 mode: the values the matrix cores read; the
    # f32 inputs rounded once beforehand, outside the timing)
    if mode == "bf16":
        tb = [x.to(torch.bfloat16) for x in (tq, tk, tv, td)]
        ms_b = time_loop(torch, lambda: fab.backward(*tb, c.scale, mask=c.tm, mode=mode, O=c.O, lse=c.lse,
                                                     blob=c.blob, ws=c.ws_bwd),
                         args.steps, args.warmup, stream, args.min_warm_s)
        out["bf16_inputs"] = {"backward_only": {"ms": round(ms_b, 4), "tflops": round(F_b / (ms_b * 1e-3) / 1e12, 3),
                                                "frac_of_peak": round(F_b / (ms_b * 1e-3) / 1e12 / peak, 4)}}
        # ... and O stored as bf16 too (FAB_BF16_O, written so by the forward)
        O16, lse16 = fab.forward_lse(tb[0], tb[1], tb[2], c.scale, mask=c.tm, mode=mode, o_bf16=True, ws=c.ws_bwd)
        ms_o = time_loop(torch, lambda: fab.backward(*tb, c.scale, mask=c.tm, mode=mode, O=O16, lse=lse16,
                                                     blob=c.blob, ws=c.ws_bwd),
                         args.steps, args.warmup, stream, args.min_warm_s)
        out["bf16_storage"] = {"what": "q, k, v, d and O stored as bf16",
                               "backward_only": {"ms": round(ms_o, 4), "tflops": round(F_b / (ms_o * 1e-3) / 1e12, 3),
                                                 "frac_of_peak": round(F_b / (ms_o * 1e-3) / 1e12 / peak, 4)}}
        # ... and the result blob as bf16 too (FAB_BF16_BLOB: the f32 gradients rounded
        # once at the store): every tensor the backward reads or writes is 16-bit
        blob16 = torch.empty(fab.blob_layout(c.fs, torch.bfloat16)[3], dtype=torch.bfloat16, device=dev)
        ms_ob = time_loop(torch, lambda: fab.backward(*tb, c.scale, mask=c.tm, mode=mode, O=O16, lse=lse16,
                                                      blob=blob16, ws=c.ws_bwd),
                          args.steps, args.warmup, stream, args.min_warm_s)
        out["bf16_storage_and_blob"] = {
            "what": "q, k, v, d, O and the result blob stored as bf16",
            "backward_only": {"ms": round(ms_ob, 4), "tflops": round(F_b / (ms_ob * 1e-3) / 1e12, 3),
                              "frac_of_peak": round(F_b / (ms_ob * 1e-3) / 1e12 / peak, 4)}}
        del tb, O16, lse16, blob16
        # ... and q, k, v, d stored as f16 instead (FAB_F16_INPUTS: widened exactly, then
        # rounded to bf16 like f32 inputs)
        th = [x.to(torch.float16) for x in (tq, tk, tv, td)]
        ms_h = time_loop(torch, lambda: fab.backward(*th, c.scale, mask=c.tm, mode=mode, O=c.O, lse=c.lse,
                                                     blob=c.blob, ws=c.ws_bwd),
                         args.steps, args.warmup, stream, args.min_warm_s)
        out["f16_inputs"] = {"backward_only": {"ms": round(ms_h, 4), "tflops": round(F_b / (ms_h * 1e-3) / 1e12, 3),
                                               "frac_of_peak": round(F_b / (ms_h * 1e-3) / 1e12 / peak, 4)}}
        del th

    # ---- every other (workload, mode) pair, same protocol
    pairs = []
    if args.configs == "all":
        pairs = [(wid, m) for wid in sorted(fi.WORKLOADS) for m in fi.WORKLOADS[wid].modes]
        if (args.workload, "f32") not in pairs:
            pairs.append((args.workload, "f32"))   # the headline workload in the other mode too
    elif args.configs:
        pairs = [(int(x.split(":")[0]), x.split(":")[1]) for x in args.configs.split(",") if x.strip()]
    headline_host = c.host
    del c
    torch.cuda.empty_cache()
    configs = {}
    for wid, m in pairs:
        if (wid, m) == (args.workload, mode):
            continue
        c2 = Case(torch, fab, dev, wid, m)
        configs[f"{wid}:{m}"] = pair_summary(torch, fab, c2, args, stream)
        del c2
        torch.cuda.empty_cache()
    if configs:
        out["configs"] = configs
    if not args.no_cpu_baseline:
        q, k, v, d, mask = headline_host
        out["cpu_baseline"] = cpu_baseline(s, q, k, v, d, mask, c_scale(args.workload), causal, args.cpu_budget_s)
    print(json.dumps(out), flush=True)


def c_scale(wid):
    return fi.WORKLOADS[wid].scale_f32()


if __name__ == "__main__":
    main()
