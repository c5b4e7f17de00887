#!/usr/bin/env python3
"""Benchmark of the split-KV attention path on one MI355X.

Default (the headline line): decode, 1 query, 40 query heads / 8 KV heads, head_dim 128,
n_kv = 131072 cells fully device-resident, K q8_0 / V q4_0, Q f16 -- one rkv_attn_decode
call per step (window split-K segment kernel + LSE merge).  Inputs are seeded synthetic
draws (rkv_inputs); the KV cache is rotated over several independent device copies so the
256 MB last-level cache cannot serve repeats.

Other workloads (--workload 1..5) print a line of the same form for the small decode
split, the rolling window + pinned-host tail decode, the unified-pool rows decode and the
prefill chunk.

The JSON line carries:
  value       whole-call effective KV GB/s (algorithmic KV bytes / ms_per_step)
  roofline    the dominant segment kernel: algorithmic bytes (or flops) per launch over
              its average launch time, timed with HIP events on its own stream inside the
              timed region, against the MI355X peak
  cpu_baseline the fp64 oracle on the host cores over a bounded sample, scaled to the
              same unit
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense f16 MFMA, vendor figure
PROFILES = os.path.join(ROOT, "profiles")

LIFT_NAMES = {0: "bulk", 1: "uva", 2: "kernel", 4: "direct"}

METRIC = "decode attn effective KV GB/s (% HBM peak) + tok/s/layer at n_kv=128K"


KERNEL_SOURCES = {
    # sources whose change invalidates a committed traffic measurement of that kernel
    "decode": ("rkv_decode.hip", "rkv_decode_mma.hip", "rkv_decode_mma16.hip", "rkv_unpack.h", "rkv_wave.h", "rkv_internal.h", "rkv_runtime.cpp"),
    "prefill": ("rkv_prefill.hip", "rkv_unpack.h", "rkv_internal.h", "rkv_runtime.cpp"),
}


def kernel_source_hash(kind: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        p = os.path.join(ROOT, "tiered_kv_cache_split_amd", "csrc", f)
        if os.path.exists(p):
            h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profiles(name: str, kind: str):
    """HBM bytes per launch from the committed PMC summary, if it was taken on this kernel."""
    p = os.path.join(PROFILES, f"{name}_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return d.get("hbm_bytes_per_launch")


def physical_cores() -> int:
    """Physical cores of this host from lscpu (cores per socket x sockets); the logical CPU
    count if lscpu is unavailable."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        kv = {}
        for line in out.splitlines():
            if ":" in line:
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
        n = int(kv["Core(s) per socket"]) * int(kv.get("Socket(s)", "1"))
        # a container may see fewer CPUs than the host has cores
        return max(1, min(n, len(os.sched_getaffinity(0))))
    except Exception:
        return os.cpu_count() or 1


# ------------------------------------------------------------------ workloads on device
_DRAWN = {}


def setup(num: int, sets: int, head_dim: int = 128, f16: bool = False):
    import numpy as np
    import torch

    import rkv_inputs as gen

    key = (num, head_dim, f16)
    if key not in _DRAWN:  # the tail-read contrasts of one workload reuse its draw
        _DRAWN.clear()
        over = {} if head_dim == 128 else {"d": head_dim, "dv": 512 if head_dim == 576 else head_dim}
        if f16:  # binary16 K and V in place of the workload's own types
            over.update(k_type=gen.TYPE_F16, v_type=gen.TYPE_F16)
        w = gen.make_workload(num, **over)
        if f16:
            w["name"] = w["name"].replace("q8q4", "f16")
        _DRAWN[key] = w
    w = _DRAWN[key]
    dv = w.get("dv", w["d"])
    rb = lambda t, dd=w["d"]: gen.row_bytes(t, dd)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()

    def pinned(a):
        src = torch.from_numpy(np.ascontiguousarray(a))
        t = torch.empty(src.shape, dtype=src.dtype, pin_memory=True)
        t.copy_(src)
        return t

    st = {"w": w, "q": dev(w["q"])}
    if w["kind"] == "rows":
        k0, v0 = dev(w["k"]), dev(w["v"])
        st["sets"] = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(sets - 1)]
        st["rows"] = dev(w["kv_rows"].astype(np.int32))
        st["mask"] = dev(w["mask"])
        n_seq, n_head, n_q, _ = w["q"].shape
        st["o"] = torch.empty((n_seq, n_q, n_head, dv), dtype=torch.float32, device="cuda")
        st["lse"] = torch.empty((n_seq, n_q, n_head), dtype=torch.float32, device="cuda")
        kv_bytes = int((w["kv_rows"] >= 0).sum()) * w["n_head_kv"] * (rb(w["k_type"]) + rb(w["v_type"], dv))
        st["kv_bytes"] = kv_bytes
        st["tail_bytes"] = 0
        return st
    wc = w["wc"]
    kw, vw = dev(w["k"][:wc]), dev(w["v"][:wc])
    st["sets"] = [(kw, vw)] + [(kw.clone(), vw.clone()) for _ in range(sets - 1)]
    st["tail"] = None
    if w["n_kv"] > wc:
        st["tail"] = (pinned(w["k"][wc:]), pinned(w["v"][wc:]))
    n_head, n_q = w["n_head"], w["q"].shape[1]
    st["o"] = torch.empty((n_q, n_head, dv), dtype=torch.float32, device="cuda")
    st["lse"] = torch.empty((n_q, n_head), dtype=torch.float32, device="cuda")
    per_cell = w["n_head_kv"] * (rb(w["k_type"]) + rb(w["v_type"], dv))
    st["kv_bytes"] = w["n_kv"] * per_cell
    st["tail_bytes"] = (w["n_kv"] - wc) * per_cell
    st["window_bytes"] = wc * per_cell
    return st


# kernel families reported in the context's stats (enum rkv_kernel_variant)
DECODE_KERNELS = {0: "decode_seg_kernel", 2: "decode_cell_kernel", 3: "decode_mma_kernel", 4: "decode_mma16_kernel",
                  5: "decode_hd_kernel"}


def call(ctx, st, i):
    import tiered_kv_cache_split_amd as rkv
    w = st["w"]
    k, v = st["sets"][i % len(st["sets"])]
    if w["kind"] == "rows":
        ctx.attn_rows(rkv.q_desc(st["q"]), rkv.kv_desc(k, w["k_type"]), rkv.kv_desc(v, w["v_type"]), st["rows"],
                      w["n_kv"], rkv.mask_desc(st["mask"]), w["scale"], st["o"], st["lse"])
        return
    kt = vt = None
    if st["tail"] is not None:
        kt = rkv.kv_desc(st["tail"][0], w["k_type"])
        vt = rkv.kv_desc(st["tail"][1], w["v_type"])
    args = (rkv.q_desc(st["q"]), rkv.kv_desc(k, w["k_type"]), rkv.kv_desc(v, w["v_type"]), kt, vt, None,
            w["wc"], w["tile_kv"], w["scale"])
    if w["kind"] == "prefill":
        ctx.attn_prefill(*args, w["q_pos0"], st["o"], st["lse"])
    else:
        ctx.attn_decode(*args, st["o"], st["lse"])


def prefill_flops(w) -> float:
    """QK^T and PV flops over the visible (query, key) pairs of a causal chunk at the end:
    2 dk + 2 dv per pair and query head."""
    n_q, n_kv, q0 = w["q"].shape[1], w["n_kv"], w["q_pos0"]
    pairs = sum(min(n_kv, q0 + i + 1) for i in range(n_q))
    return 2.0 * (w["d"] + w.get("dv", w["d"])) * pairs * w["n_head"]


def measured_h2d_gbs(nbytes=256 << 20, reps=10) -> float:
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    ts = []
    for _ in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dst.copy_(src, non_blocking=True)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts = sorted(ts[2:])
    return nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9


def measured_copy_gbs(nbytes=1 << 30, reps=10) -> float:
    """Device-to-device copy kernel, counting read + write bytes."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    ts = []
    for _ in range(reps + 2):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        e1.synchronize()
        ts.append(e0.elapsed_time(e1))
    ts = sorted(ts[2:])
    return 2 * nbytes / (ts[len(ts) // 2] * 1e-3) / 1e9


# ------------------------------------------------------------------ CPU baseline (oracle)
def cpu_baseline(num: int, budget_s: float = 12.0, w=None, softcap: float = 0.0):
    """Time the fp64 oracle on a bounded sample of the same workload and scale to GB/s of the
    full workload's algorithmic KV bytes.  BLAS threads = the physical cores (lscpu); one
    warm-up run (which also sizes the sample to about budget_s / 8), then the median of three;
    then the same sample on one thread (median of three, or one run if that would exceed the
    budget)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import rkv_inputs as gen

    w = gen.make_workload(num) if w is None else w
    cores = physical_cores()
    n_kv = w["n_kv"]
    target = budget_s / 8
    if w["kind"] == "rows":
        per_cell = w["n_head_kv"] * (gen.row_bytes(w["k_type"], w["d"]) + gen.row_bytes(w["v_type"], w.get("dv", w["d"])))
        total_cells = int((w["kv_rows"] >= 0).sum())
        q = np.stack([oracle.q_values(w["q"][b]) for b in range(w["q"].shape[0])])

        def run_sample(cells):
            rows = w["kv_rows"][:, :cells]
            k = oracle.kv_values(w["k_type"], w["k"])
            v = oracle.kv_values(w["v_type"], w["v"])
            oracle.attention_rows(q, k, v, rows, w["scale"], None, softcap)
            return int((rows >= 0).sum())
        full_units, unit_bytes = total_cells, per_cell
    else:
        per_cell = w["n_head_kv"] * (gen.row_bytes(w["k_type"], w["d"]) + gen.row_bytes(w["v_type"], w.get("dv", w["d"])))
        q = oracle.q_values(w["q"])
        n_q = w["q"].shape[1]
        if w["kind"] == "prefill":
            q = q[:, -min(n_q, 64):]
        q_scale = (n_q / q.shape[1]) if w["kind"] == "prefill" else 1.0

        def run_sample(cells):
            k = oracle.kv_values(w["k_type"], w["k"][:cells])
            v = oracle.kv_values(w["v_type"], w["v"][:cells])
            oracle.attention(q, k, v, w["scale"], None, softcap)
            return cells / q_scale
        full_units, unit_bytes = n_kv, per_cell

    def timed(cells):
        t0 = time.perf_counter()
        done = run_sample(cells)
        return time.perf_counter() - t0, done

    with threadpool_limits(limits=cores, user_api="blas"):
        cells = 1024
        while True:  # warm-up and sizing
            dt, done = timed(cells)
            if dt >= target or cells >= n_kv:
                break
            cells = min(n_kv, cells * 2)
        runs = [timed(cells) for _ in range(3)]
    med = sorted(r[0] for r in runs)[1]
    done = runs[0][1]
    with threadpool_limits(limits=1, user_api="blas"):
        t1, _ = timed(cells)
        one = [t1]
        if 3 * t1 < budget_s / 2:
            one += [timed(cells)[0] for _ in range(2)]
    med1 = sorted(one)[len(one) // 2]
    full_s = med * full_units / max(1e-9, done)
    full_s1 = med1 * full_units / max(1e-9, done)
    if w["kind"] == "rows":
        sample = f"row lists cut to their first {cells} entries ({done} pool rows of {total_cells})"
    else:
        sample = f"first {cells} of {n_kv} cells"
        if w["kind"] == "prefill":
            sample += f", last {q.shape[1]} of {w['q'].shape[1]} queries (unmasked)"
    sample += "; median of 3 after one warm-up, time scaled linearly to the full workload"
    gbs = full_units * unit_bytes / full_s / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": cores, "kind": "oracle", "sample": sample,
            "oracle_s_full_extrapolated": round(full_s, 2), "sample_s_median": round(med, 3),
            "single_core": {"value": round(full_units * unit_bytes / full_s1 / 1e9, 4), "unit": "GB/s",
                            "sample_s_median": round(med1, 3), "runs": len(one)}}


# ------------------------------------------------------------------ main
def measure(args, num):
    """One workload: warm-up, the timed calls, then an instrumented pass; returns the JSON fields
    and the workload's host arrays."""
    import torch

    import rkv_inputs as gen
    import tiered_kv_cache_split_amd as rkv

    print(f"[bench] workload {num}: {gen.WORKLOADS[num]['name']} setup", file=sys.stderr, flush=True)
    st = setup(num, args.sets, args.head_dim, args.kv_types == "f16")
    w = st["w"]
    ctx = rkv.Context(0)
    if args.splits:
        ctx.set_splits(args.splits)
    ctx.set_lift_mode(args.lift_mode)
    if args.softcap:
        ctx.set_softcap(args.softcap)
    tail_choice = None
    if args.tail_mode == "auto" and st.get("tail_bytes"):
        # rates on this machine: pinned H2D copies, and two calls with the host partial
        h2d = measured_h2d_gbs()
        ctx.set_tail_mode(rkv.RKV_TAIL_HOST, args.host_threads)
        host_ms = []
        for i in range(2):
            call(ctx, st, i)
            host_ms.append(ctx.stats()["host_tail_ms"])
        torch.cuda.synchronize()
        host_gbs = st["tail_bytes"] / (min(host_ms) * 1e-3) / 1e9
        mode = rkv.choose_tail_mode(st["tail_bytes"], h2d, host_gbs)
        tail_choice = {"h2d_GBps": round(h2d, 2), "host_GBps": round(host_gbs, 2),
                       "chosen": "host" if mode == rkv.RKV_TAIL_HOST else "lift"}
        ctx.set_tail_mode(rkv.RKV_TAIL_LIFT)
        args.tail_mode = tail_choice["chosen"]
    host_tail = args.tail_mode == "host" and bool(st.get("tail_bytes"))
    if host_tail:
        ctx.set_tail_mode(rkv.RKV_TAIL_HOST, args.host_threads)
    for i in range(args.warmup):
        call(ctx, st, i)
    torch.cuda.synchronize()
    print(f"[bench] workload {num}: warmup done, timing {args.steps} steps", file=sys.stderr, flush=True)

    # timed region: whole calls only, nothing else on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        call(ctx, st, i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stats = ctx.stats()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    assert torch.isfinite(st["o"]).all()

    # instrumented pass over the same calls: the segment kernels bracketed by events recorded
    # in their own dispatches (roofline), and the tail lifts timed on the copy stream
    n_inst = min(args.steps, 50)
    ctx.set_kernel_timing(True)
    lift_totals, host_ms = [], []
    if st.get("tail_bytes") and not host_tail:
        ctx.set_lift_timing(True)
    torch.cuda.synchronize()
    for i in range(n_inst):
        call(ctx, st, i)
        if st.get("tail_bytes") and not host_tail:
            tot, span, n = ctx.lift_timing_ms()  # waits for this call's lifts
            lift_totals.append((tot, span, n))
        if host_tail:
            host_ms.append(ctx.stats()["host_tail_ms"])
    torch.cuda.synchronize()
    k_ms, k_n = ctx.kernel_timing_ms()
    ctx.set_kernel_timing(False)
    ctx.set_lift_timing(False)

    launches_per_step = max(1, k_n // n_inst)
    kern_ms = k_ms / max(1, k_n)  # average segment-kernel launch
    kv_bytes = st["kv_bytes"]
    out = {
        "metric": METRIC,
        "value": round(kv_bytes / (ms_per_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",  # matrix-core operands (q8_0/q4_0 codes as exact binary16 integers)
        "accum_dtype": "f32",  # accumulation, softmax and partials
        "data": "synthetic",
        "config": {"workload": w["name"], "n_head": w["n_head"], "n_head_kv": w["n_head_kv"], "head_dim": w["d"], **({"head_dim_v": w["dv"]} if w.get("dv", w["d"]) != w["d"] else {}),
                   "n_q": int(w["q"].shape[-2]), "n_kv": int(w["n_kv"]),
                   "k_type": gen.TYPE_NAMES[w["k_type"]], "v_type": gen.TYPE_NAMES[w["v_type"]],
                   "kv_sets_rotated": args.sets, "parallelism": "single GPU",
                   **({"tail_mode": "host"} if host_tail else {}),
                   **({"softcap": args.softcap} if args.softcap else {})},
        "tok_per_s_per_layer": round(1e3 / ms_per_step, 1),
        "pct_hbm_peak_whole_call": round(100 * kv_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
        "segment_launches_per_step": launches_per_step,
        "stats": stats,
    }
    if w["kind"] == "prefill":
        flops = prefill_flops(w)
        kern_total_ms = k_ms / n_inst
        achieved = flops / (kern_total_ms * 1e-3) / 1e12
        out["roofline"] = {"bound": "mfma", "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                           "traffic": traffic_from_profiles("prefill_seg_q8q4_nq512_nkv106496", "prefill")
                           if w["d"] == 128 and args.kv_types == "own" else None,
                           "kernel": ("prefill_seg_kernel" if stats.get("kernel_variant") == 1 else
                                      DECODE_KERNELS.get(stats.get("kernel_variant"), "segment kernel"))
                           + " (all segments of a step)",
                           "kernel_ms_per_step": round(kern_total_ms, 4)}
    else:
        name = {2: "decode_seg_q8q4_nkv131072", 4: "decode_seg_rows_f16_pool65536"}.get(num, "")
        label = DECODE_KERNELS.get(stats.get("kernel_variant"), "decode segment kernel")
        gpu_bytes = kv_bytes - (st["tail_bytes"] if host_tail else 0)  # a host tail partial reads no HBM
        if launches_per_step == 1:
            # one segment launch per step (resident window or pool): bytes of one launch / its time
            achieved = gpu_bytes / (kern_ms * 1e-3) / 1e9
        else:
            # window plus tail tiles: all KV bytes over the step's total segment-kernel time
            achieved = gpu_bytes / ((k_ms / n_inst) * 1e-3) / 1e9
            label += " (all segments of a step)"
        out["roofline"] = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": round(achieved / HBM_PEAK_GBS, 4),
                           "traffic": traffic_from_profiles(name, "decode")
                           if name and w["d"] == 128 and args.kv_types == "own" else None,
                           "kernel": label, "kernel_avg_ms": round(kern_ms, 5)}
    if lift_totals:
        tot = sum(t[0] for t in lift_totals) / len(lift_totals)
        span = sum(t[1] for t in lift_totals) / len(lift_totals)
        h2d = measured_h2d_gbs()
        lift_gbs = st["tail_bytes"] / (tot * 1e-3) / 1e9 if tot > 0 else None
        out["lift"] = {"mode": LIFT_NAMES[stats["lift_mode"]], "tail_bytes": st["tail_bytes"],
                       "lift_ms_sum": round(tot, 4), "lift_span_ms": round(span, 4),
                       "lift_GBps_overlapped": round(lift_gbs, 2) if lift_gbs else None,
                       "measured_h2d_GBps": round(h2d, 2),
                       "frac_of_measured_h2d": round(lift_gbs / h2d, 4) if lift_gbs else None}
    if stats.get("lift_mode") == 4 and st.get("tail_bytes"):
        # no lift: the segment kernels read the pinned tail through its device view; the tail's
        # own read rate is at least its bytes over all segment-kernel time of a step
        seg_ms = k_ms / n_inst
        out["direct_tail"] = {"tail_bytes": st["tail_bytes"], "segment_kernel_ms_per_step": round(seg_ms, 4),
                              "tail_GBps_at_least": round(st["tail_bytes"] / (seg_ms * 1e-3) / 1e9, 2)}
    if host_tail:
        hm = sorted(host_ms)[len(host_ms) // 2]
        out["host_tail"] = {"tail_bytes": st["tail_bytes"], "threads": args.host_threads, "host_ms_median": round(hm, 4),
                            "host_GBps": round(st["tail_bytes"] / (hm * 1e-3) / 1e9, 2),
                            "partial_bytes_uploaded": int(w["n_head"] * w["q"].shape[-2] * (2 + w["d"]) * 4)}
    if tail_choice:
        out["tail_choice"] = tail_choice
    ctx.close()
    w = st["w"]
    del st
    torch.cuda.empty_cache()
    return out, w


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--sets", type=int, default=4, help="independent device copies of the KV cache")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--softcap", type=float, default=0.0, help="logit soft-cap c (0: none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--head-dim", type=int, default=128, choices=[64, 128, 256, 512, 576],
                    help="head dim of Q and K; V takes the same, or 512 with 576")
    ap.add_argument("--kv-types", choices=["own", "f16"], default="own",
                    help="K / V types: the workload's own, or binary16 for both")
    ap.add_argument("--lift-mode", type=int, default=3,
                    help="0 bulk DMA, 1 word-granularity UVA read, 2 bulk copy kernel on the copy stream, "
                         "3 automatic (decode: copy kernel, prefill: DMA)")
    ap.add_argument("--tail-mode", choices=["lift", "host", "auto"], default="lift",
                    help="host tail: lifted to the GPU in tiles, its partial computed on the host cores, or "
                         "whichever the measured link and host rates make faster")
    ap.add_argument("--host-threads", type=int, default=16, help="host threads of the host tail partial")
    ap.add_argument("--no-secondary", dest="secondary", action="store_false",
                    help="headline workload only (default: workloads 1, 3, 4 and 5 and the tail-read contrasts "
                         "of workload 3 follow in the same run, under \"secondary\")")
    ap.add_argument("--secondary-steps", type=int, default=30)
    ap.add_argument("--copy-only", action="store_true",
                    help="only run a plain 1 GiB device copy (calibrates HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import rkv_inputs as gen
    import tiered_kv_cache_split_amd as rkv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.copy_only:
        gbs = measured_copy_gbs(1 << 30, reps=5)
        print(json.dumps({"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "copy_GBps": round(gbs, 1)}))
        return
    out, w = measure(args, args.workload)
    if args.secondary and args.workload == 2 and args.head_dim == 128 and not args.softcap and args.kv_types == "own":
        # the other configurations, timed in the same run (fewer steps; the headline stays config 2)
        sec = {}
        base = dict(vars(args))
        for num, over, key in ((1, {}, None), (3, {}, None), (3, {"lift_mode": 0}, "lift_dma"),
                               (3, {"lift_mode": 4}, "direct_tail_read"), (4, {}, None), (5, {}, None)):
            a2 = argparse.Namespace(**{**base, "steps": args.secondary_steps, "warmup": 5, "sets": 2, **over})
            r, _ = measure(a2, num)
            name = gen.WORKLOADS[num]["name"] + (f"_{key}" if key else "")
            sec[name] = {k: r[k] for k in ("value", "unit", "ms_per_step", "tok_per_s_per_layer", "config", "roofline",
                                           "lift", "direct_tail", "segment_launches_per_step") if k in r}
            sec[name]["steps"] = a2.steps
        out["secondary"] = sec
    out["measured_copy_GBps"] = round(measured_copy_gbs(), 1)
    if not args.no_cpu_baseline:
        print("[bench] timing the oracle on the host cores", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(args.workload, w=w, softcap=args.softcap)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
