#!/usr/bin/env python3
"""Benchmark of exact tiled attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward (fa_fwd: O and lse) and the backward (fa_bwd's three stages: D,
the key-tile kernel, dQ conversion) of causal attention at the training-step
shape [4, 16, 2048, 64] in bf16.  Inputs are resident in HBM before timing.

Prints ONE JSON line.  Throughput counts 4*N^2*d FLOP per (batch, head) for
the forward, halved when causal, and 2.5x that for the backward.

Extra modes (each prints its own JSON):
  --copy-calibration MIB   time a plain device copy of MIB MiB (used to scale
                           rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --pmc-summary FETCH_CSV WRITE_CSV
                           turn two rocprofv3 --pmc counter CSVs into
                           profiles/traffic.json (HBM bytes per launch of the
                           dominant kernel, scaled by the copy calibration)
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at N=1k-32k, d=64/128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# sources each kernel is built from: counter-derived traffic is used only while
# they are unchanged
KERNEL_SOURCES = {
    "bwd_main_kernel": ["exact_tiled_attention_10_amd/csrc/fa_bwd.hip",
                        "exact_tiled_attention_10_amd/csrc/fa_common.h"],
    "fwd_bf16_kernel": ["exact_tiled_attention_10_amd/csrc/fa_fwd.hip",
                        "exact_tiled_attention_10_amd/csrc/fa_common.h"],
}
STEP_WORKLOAD = "train_step_n2048"
SWEEP = [("gpt2_medium_n1024", False), ("gpt2_medium_n1024", True),
         ("llama8b_n4096", True), ("long_context_n16384", True),
         ("long_context_n32768", True)]


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def run_step_bench(steps: int, warmup: int):
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[STEP_WORKLOAD]
    causal = True
    q, k, v, do = (t.cuda() for t in workload_inputs(w, with_do=True))
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd(q, k, v, o, lse, causal, w.scale)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd_preprocess(o, do, lse, ws)
        if ev is not None:
            ev[2].record(stream)
        fa.fa_bwd_main(q, k, v, do, dk, dv, ws, causal, w.scale)
        if ev is not None:
            ev[3].record(stream)
        fa.fa_bwd_finalize(dq, ws, q, k, v, do, causal, w.scale)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    # the timed steps carry no events of their own: an event recorded between
    # two launches holds the next one until the previous has drained (four per
    # step added ~12 us to a ~195 us step)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms = total_ms / steps
    # then the same number of steps again with events around each kernel on
    # its launch stream: the forward and key-tile kernel durations
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        step(evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    inst_ms = t0.elapsed_time(t1) / steps
    fwd_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    main_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    ff = fwd_flops(B, H, N, d, causal)
    bf = 2.5 * ff
    return dict(workload=w, ms_per_step=ms, step_flops=ff + bf, fwd_ms=fwd_ms, main_ms=main_ms,
                fwd_flops=ff, bwd_flops=bf, instrumented_ms_per_step=inst_ms)


def run_fwd_sweep(reps: int = 20, warm_s: float = 0.05):
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import WORKLOADS, workload_inputs

    out = {}
    for name, causal in SWEEP:
        w = WORKLOADS[name]
        q, k, v = (t.cuda() for t in workload_inputs(w, with_do=False))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        t_end = time.perf_counter() + warm_s
        n_warm = 0
        while n_warm < 3 or time.perf_counter() < t_end:
            fa.fa_fwd(q, k, v, o, lse, causal, w.scale)
            n_warm += 1
            if n_warm % 16 == 0:
                torch.cuda.synchronize()
        s = torch.cuda.Event(enable_timing=True)
        e = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        for _ in range(reps):
            fa.fa_fwd(q, k, v, o, lse, causal, w.scale)
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        tf = fwd_flops(w.B, w.H, w.N, w.d, causal) / (ms * 1e-3) / 1e12
        out[f"{name}{'_causal' if causal else ''}"] = dict(
            fwd_ms=round(ms, 4), tflops=round(tf, 1),
            pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def _time_launches(fn, reps: int = 20, warm_s: float = 0.05):
    """Mean ms per call of ``fn`` (HIP events on the current stream) after
    ``warm_s`` seconds of warm-up."""
    import torch
    t_end = time.perf_counter() + warm_s
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / reps


def run_extra_sweep():
    """Grouped-query, head-dimension-256 and different-length shapes:
    Llama-3.1-8B's real head sharing (32 query heads over 8 key/value heads)
    for the causal N = 4096 forward and backward, the d = 256 causal forward at
    [1, 16, 4096, 256], the e4m3 forward at [1, 32, 4096, 128] causal (against
    the fp8 peak), and decode -- one new token per sequence against a
    32k-token cache, split across workgroups by key range -- whose bound is
    HBM (every key and value byte is read once per key/value head)."""
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import make_gqa_inputs

    out = {}
    B, H, Hkv, N, d = 1, 32, 8, 4096, 128
    q, k, v, do = (t.cuda() for t in make_gqa_inputs(B, H, Hkv, N, d, seed=6, with_do=True))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    sc = 1 / math.sqrt(d)
    ms = _time_launches(lambda: fa.fa_fwd_gqa(q, k, v, o, lse, True, sc))
    tf = fwd_flops(B, H, N, d, True) / (ms * 1e-3) / 1e12
    out["llama8b_gqa32x8_n4096_causal_fwd"] = dict(
        ms=round(ms, 4), tflops=round(tf, 1), pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(fa.fa_bwd_kv_workspace_size(B, H, Hkv, N, N, d), dtype=torch.uint8,
                     device="cuda")
    ms = _time_launches(lambda: fa.fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, True, sc))
    tf = 2.5 * fwd_flops(B, H, N, d, True) / (ms * 1e-3) / 1e12
    out["llama8b_gqa32x8_n4096_causal_bwd"] = dict(
        ms=round(ms, 4), tflops=round(tf, 1), pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
    del q, k, v, do, o, lse, dq, dk, dv, ws

    B, H2, N2, d2 = 1, 16, 4096, 256
    q, k, v = (t.cuda() for t in make_gqa_inputs(B, H2, H2, N2, d2, seed=9))
    o = torch.empty_like(q)
    lse = torch.empty((B, H2, N2), dtype=torch.float32, device="cuda")
    ms = _time_launches(lambda: fa.fa_fwd(q, k, v, o, lse, True, 1 / 16.0))
    tf = fwd_flops(B, H2, N2, d2, True) / (ms * 1e-3) / 1e12
    out["d256_n4096_causal_fwd"] = dict(
        ms=round(ms, 4), tflops=round(tf, 1), pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
    del q, k, v, o, lse

    from workloads import make_fp8_inputs
    q8, k8, v8, sq, sk, sv = make_fp8_inputs(1, 32, 4096, 128, seed=10)
    q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
    o = torch.empty((1, 32, 4096, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 32, 4096), dtype=torch.float32, device="cuda")
    ms = _time_launches(lambda: fa.fa_fwd_fp8(q8, k8, v8, o, lse, sq, sk, sv, True, sc))
    tf = fwd_flops(1, 32, 4096, 128, True) / (ms * 1e-3) / 1e12
    out["fp8_llama8b_n4096_causal_fwd"] = dict(
        ms=round(ms, 4), tflops=round(tf, 1), pct_of_fp8_peak=round(100 * tf / PEAK_FP8_TFLOPS, 1),
        pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
    del q8, k8, v8, o, lse

    B, Nk = 8, 32768
    q = make_gqa_inputs(B, H, Hkv, 1, d, seed=7)[0].cuda()
    k, v = (t.cuda() for t in make_gqa_inputs(B, H, Hkv, Nk, d, seed=8)[1:])
    o = torch.empty_like(q)
    lse = torch.empty((B, H, 1), dtype=torch.float32, device="cuda")
    nb = fa.fa_fwd_kv_workspace_size(B, H, Hkv, 1, Nk, d)
    ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
    ms = _time_launches(lambda: fa.fa_fwd_kv(q, k, v, o, lse, ws, True, sc), reps=50)
    nbytes = 2 * B * Hkv * Nk * d * 2 + 2 * B * H * d * 2 + B * H * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["llama8b_decode_b8_gqa32x8_nk32768"] = dict(
        ms=round(ms, 4), algorithmic_bytes=nbytes, gbs=round(gbs, 1),
        frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4), workspace_bytes=nb)
    del q, k, v, o, lse, ws
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------
# oracle on the host cores
# ---------------------------------------------------------------------------

def _blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # noqa: BLE001
        pass
    return 1


def run_cpu_baseline(budget_s: float):
    """The float64 oracle (plain forward + Jacobian backward) on whole heads of
    the step workload until ``budget_s`` of wall time is spent (at least one
    head); throughput in the same counted-FLOP units as the GPU value."""
    import numpy as np
    from oracle import naive_bwd, naive_fwd
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[STEP_WORKLOAD]
    q, k, v, do = workload_inputs(w, with_do=True)
    f64 = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for (b, h) in heads:
        qq, kk, vv, gg = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
        naive_fwd(qq, kk, vv, w.scale, True)
        naive_bwd(qq, kk, vv, gg, w.scale, True)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, done, w.N, w.d, True)
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=_blas_threads(),
                kind="oracle",
                sample=f"{done} of {len(heads)} (batch, head) slices of {w.name}, float64 "
                       f"forward + backward, {dt:.1f} s wall",
                host_cpu=platform.processor() or platform.machine(),
                host_logical_cpus=os.cpu_count())


# ---------------------------------------------------------------------------
# traffic (rocprofv3 counters) bookkeeping
# ---------------------------------------------------------------------------

def load_traffic(kernel_name: str):
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel") != kernel_name or t.get("source_hash") != source_hash(kernel_name):
        return None
    return t.get("bytes_per_launch")


def _read_counter_csv(path, counter):
    """{kernel-name-substring -> list of per-dispatch values} from a rocprofv3
    counter_collection.csv."""
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return rows


def pmc_summary(fetch_csv: str, write_csv: str, copy_mib: float) -> dict:
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")

    def pick(table, needle):
        ks = [k for k in table if needle in k]
        if not ks:
            raise SystemExit(f"no kernel matching {needle!r} in counters")
        vals = table[ks[0]]
        return ks[0], sum(vals) / len(vals)

    copy_bytes = copy_mib * 2 ** 20
    _, cf = pick(fetch, "copy")           # KiB read by the copy kernel
    _, cw = pick(write, "copy")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    name, kf = pick(fetch, "bwd_main_kernel")
    _, kw = pick(write, "bwd_main_kernel")
    bytes_per_launch = kf * 1024.0 * f_scale + kw * 1024.0 * w_scale
    out = dict(kernel="bwd_main_kernel", kernel_symbol=name,
               source_hash=source_hash("bwd_main_kernel"),
               fetch_kib_raw=kf, write_kib_raw=kw, copy_mib=copy_mib,
               copy_fetch_kib_raw=cf, copy_write_kib_raw=cw,
               fetch_scale=f_scale, write_scale=w_scale,
               bytes_per_launch=bytes_per_launch)
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    return out


def copy_calibration(mib: float):
    import torch
    n = int(mib * 2 ** 20)
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    return dict(copy_mib=mib, bytes=n)


# ---------------------------------------------------------------------------

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # The clock settles only after ~0.1 s of sustained matrix-core load, so the
    # default warm-up is long enough to time the steady state.
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--copy-calibration", type=float, default=None, metavar="MIB")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--copy-mib", type=float, default=256.0)
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); run with --gpus 1.",
              file=sys.stderr, flush=True)
        return 2

    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1],
                                     args.copy_mib)))
        return 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration)), flush=True)

    r = run_step_bench(args.steps, args.warmup)
    w = r["workload"]
    ms = r["ms_per_step"]
    value = r["step_flops"] / (ms * 1e-3) / 1e12

    # dominant kernel of the step: the longer of the forward and backward main kernels
    if r["main_ms"] >= r["fwd_ms"]:
        kname, kms, kflops = "bwd_main_kernel", r["main_ms"], r["bwd_flops"]
    else:
        kname, kms, kflops = "fwd_bf16_kernel", r["fwd_ms"], r["fwd_flops"]
    achieved = kflops / (kms * 1e-3) / 1e12
    roofline = dict(bound="mfma", achieved=round(achieved, 1), peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=round(achieved / PEAK_BF16_TFLOPS, 4),
                    traffic=load_traffic(kname), kernel=kname,
                    kernel_ms=round(kms, 5))

    line = dict(
        metric=METRIC, value=round(value, 2), unit="TFLOP/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=round(ms, 5),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic",
        config=dict(workload=w.name, B=w.B, H=w.H, N=w.N, d=w.d, causal=True,
                    step="fa_fwd + fa_bwd (preprocess, main, finalize)",
                    pct_of_bf16_peak=round(100 * value / PEAK_BF16_TFLOPS, 2),
                    fwd_ms=round(r["fwd_ms"], 5), bwd_main_ms=round(r["main_ms"], 5),
                    kernel_timing="HIP events around each kernel in a second pass of the "
                                  "same steps (the timed steps carry no events)",
                    instrumented_ms_per_step=round(r["instrumented_ms_per_step"], 5)),
        roofline=roofline,
    )
    if not args.no_sweep:
        line["fwd_sweep"] = run_fwd_sweep()
        line["extra_sweep"] = run_extra_sweep()
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = run_cpu_baseline(args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
