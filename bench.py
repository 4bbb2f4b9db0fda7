#!/usr/bin/env python3
"""Benchmark of exact tiled attention on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
the forward (fa_fwd: O and lse) and the backward (fa_bwd's three stages: D,
the key-tile kernel, dQ) of causal attention at the training-step shape
[4, 16, 2048, 64] in bf16.  Inputs are resident in HBM before timing.

Timing protocol (every figure is a steady-state one): a time-based settle
phase of untimed steps first (the shader clock takes a fraction of a second
of sustained matrix-core load to settle), then the counted warm-up steps,
then repeats of exactly --steps steps, each repeat bracketed by device
synchronisation and HIP events, until at least --min-timed-ms of GPU time is
covered; ms_per_step is the median repeat, with the minimum beside it.  A
second pass of the same kind records HIP events around every kernel of the
step on its launch stream, for the per-kernel durations of the roofline.

Prints ONE JSON line.  Throughput counts 4*N^2*d FLOP per (batch, head) for
the forward, halved when causal, and 2.5x that for the backward.

With --cold every timed repeat is one call (one step, one forward) and a
512 MiB device buffer -- more than the eight 4 MiB L2s and the 256 MiB
last-level cache together -- is written before it, outside the timed region,
so the inputs come from HBM; the default keeps caches warm.

Extra modes (each prints its own JSON):
  --only NAME              run just one workload: the step (--launches steps
                           after --only-settle-s seconds of untimed ones), or
                           one forward or extra shape timed as in the full run
                           (settle phase, then >= 150 ms of repeats): the
                           target of per-shape rocprofv3 runs
  --copy-calibration MIB   time a plain device copy of MIB MiB (used to scale
                           rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --pmc-summary FETCH_CSV WRITE_CSV --kernel K --workload W
                           turn two rocprofv3 --pmc counter CSVs into an entry
                           of profiles/traffic.json (HBM bytes per launch of
                           kernel K on workload W, scaled by the copy
                           calibration)
"""

from __future__ import annotations

import argparse
import csv
import hashlib
import json
import math
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd/bwd TFLOP/s and % of bf16 MFMA peak at N=1k-32k, d=64/128"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3       # MI355X dense fp32 (matrix and vector), published
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense fp8 MFMA, published
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = "exact_tiled_attention_10_amd/csrc/"
# sources each kernel is built from: counter-derived traffic is used only while
# they are unchanged
KERNEL_SOURCES = {
    "bwd_main_kernel": [CSRC + "fa_bwd.hip", CSRC + "fa_common.h"],
    "bwd_dq_direct_kernel": [CSRC + "fa_bwd.hip", CSRC + "fa_common.h"],
    "fwd_bf16_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
    "fwd_inorder_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
    "fwd_fp8_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
    "fwd_d256_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
    "fwd_d256_pair_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
    "fwd_decode_kernel": [CSRC + "fa_fwd.hip", CSRC + "fa_common.h"],
}


def fwd_kernel(d: int) -> str:
    """The forward kernel fa_fwd launches for bf16 inputs of head dimension d."""
    return {64: "fwd_inorder_kernel", 128: "fwd_bf16_kernel", 256: "fwd_d256_kernel"}[d]
STEP_WORKLOAD = "train_step_n2048"
# The pages' own figures for this path, printed beside the measurements as
# context only: other hardware, other precisions, other workloads.
PAGES_CONTEXT = {
    "note": "figures the pages quote, measured on other hardware: context, not targets",
    # "FlashAttention from scratch", "Measured on a real GPU" (the FlashAttention
    # paper's forward + backward on an A100)
    "flashattention_vs_standard_fwd_bwd": dict(
        workload="GPT-2 medium, N=1024, d=64, 16 heads, batch 64; A100",
        runtime_ms=[41.7, 7.3], speedup=5.7, hbm_gb=[40.3, 4.4], hbm_reduction=9.2),
    # "LLM Architecture Refresh [3]", section 8, the wall-clock table of naive
    # attention against the fused scaled-dot-product kernel
    "fused_vs_naive_wall_clock": dict(
        workload="causal, 8 heads, d=64, fp32; M-series Mac",
        n=[512, 1024, 2048, 4096], speedup=[3.45, 4.52, 6.40, 8.16]),
    # "Flash Attention, From First Principles", "Honesty time -- the
    # confession list", item 7
    "flashattention2_fraction_of_peak": dict(hardware="A100", fraction=[0.50, 0.73]),
}
# forward shapes: (key, workload, causal)
SWEEP = [("single_head_fp32_n256", "single_head_fp32_n256", False),
         ("gpt2_medium_n1024", "gpt2_medium_n1024", False),
         ("gpt2_medium_n1024_causal", "gpt2_medium_n1024", True),
         ("llama8b_n4096_causal", "llama8b_n4096", True),
         ("long_context_n16384_causal", "long_context_n16384", True),
         ("long_context_n32768_causal", "long_context_n32768", True)]


def fwd_flops(B, H, N, d, causal):
    f = 4.0 * N * N * d * B * H
    return f / 2 if causal else f


def fwd_algorithmic_bytes(B, H, N, d, elem=2):
    """Read Q, K, V; write O and the float32 lse."""
    return 4 * B * H * N * d * elem + B * H * N * 4


def bwd_algorithmic_bytes(B, H, N, d, elem=2):
    """Read Q, K, V, O, dO and lse; write dQ, dK, dV."""
    return 8 * B * H * N * d * elem + B * H * N * 4


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ---------------------------------------------------------------------------
# GPU timing
# ---------------------------------------------------------------------------

def make_step(workload: str = STEP_WORKLOAD):
    """Device tensors of the training-step workload and ``step(ev=None)``, one
    pass of fa_fwd -> fa_bwd_preprocess -> fa_bwd_main -> fa_bwd_finalize on
    the current stream.  ``ev``, a list of five HIP events, brackets the four
    launches.  Returns (step, tensors); the parity tests call this same step."""
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[workload]
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
        if ev is not None:
            ev[4].record(stream)

    tensors = dict(q=q, k=k, v=v, do=do, o=o, lse=lse, dq=dq, dk=dk, dv=dv, ws=ws,
                   workload=w, causal=causal)
    return step, tensors


def _settle(fn, seconds: float) -> int:
    """Run ``fn`` untimed for at least ``seconds`` of wall time (synchronising
    every 16 calls so the queue stays short); returns the call count."""
    import torch
    t_end = time.perf_counter() + seconds
    n = 0
    while n < 3 or time.perf_counter() < t_end:
        fn()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


# --cold: the buffer written before every timed repeat (None: warm caches)
COLD_MIB = 512
_cold_buf = None


def set_cold(on: bool):
    global _cold_buf
    import torch
    _cold_buf = torch.empty(COLD_MIB << 20, dtype=torch.uint8, device="cuda") if on else None


def _flush_caches(i: int):
    """Cold mode: write the whole buffer (a value that changes per repeat) and
    wait for it, so the next timed call finds no input in any cache."""
    if _cold_buf is not None:
        import torch
        _cold_buf.fill_(i & 0xFF)
        torch.cuda.synchronize()


def _per_repeat(n: int) -> int:
    return 1 if _cold_buf is not None else n


def _repeats(fn, per_repeat: int, min_ms: float, min_repeats: int = 5):
    """Per-call ms of repeats of ``per_repeat`` calls of ``fn`` (HIP events on
    the current stream, device synchronised around each repeat) until at
    least ``min_ms`` of GPU time is covered.  Cold mode: one call per repeat,
    caches flushed before each."""
    import torch
    per_repeat = _per_repeat(per_repeat)
    stream = torch.cuda.current_stream()
    s = torch.cuda.Event(enable_timing=True)
    e = torch.cuda.Event(enable_timing=True)
    out, total = [], 0.0
    while len(out) < min_repeats or total < min_ms:
        torch.cuda.synchronize()
        _flush_caches(len(out))
        s.record(stream)
        for _ in range(per_repeat):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        ms = s.elapsed_time(e)
        total += ms
        out.append(ms / per_repeat)
    return out


def run_step_bench(steps: int, warmup: int, settle_s: float, min_timed_ms: float):
    import torch

    step, t = make_step()
    w = t["workload"]
    B, H, N, d = t["q"].shape
    n_settle = _settle(step, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps carry no events of their own: an event recorded between
    # two launches holds the next one until the previous has drained
    reps = _repeats(step, steps, min_timed_ms)
    # then repeats with events around each kernel on its launch stream
    kernel_ms = {"fwd": [], "pre": [], "main": [], "fin": []}
    inst = []
    timed = 0.0
    per = _per_repeat(steps)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(per)]
    while len(inst) < 5 or timed < min_timed_ms:
        torch.cuda.synchronize()
        _flush_caches(len(inst))
        for i in range(per):
            step(evs[i])
        torch.cuda.synchronize()
        span = evs[0][0].elapsed_time(evs[-1][4])
        timed += span
        inst.append(span / per)
        for e in evs:
            for j, key in enumerate(("fwd", "pre", "main", "fin")):
                kernel_ms[key].append(e[j].elapsed_time(e[j + 1]))
    ff = fwd_flops(B, H, N, d, True)
    bf = 2.5 * ff
    med = {k: statistics.median(v) for k, v in kernel_ms.items()}
    return dict(workload=w, ms_per_step=statistics.median(reps), ms_min=min(reps),
                ms_mean=statistics.fmean(reps), repeats=len(reps), steps_per_repeat=per,
                timed_ms=sum(reps) * per, settle_steps=n_settle, settle_s=settle_s,
                step_flops=ff + bf, fwd_flops=ff, bwd_flops=bf,
                instrumented_ms_per_step=statistics.median(inst), kernel_ms=med)


def _roofline_mfma(flops, ms, kernel, workload, peak=PEAK_BF16_TFLOPS, unit_bytes=None):
    achieved = flops / (ms * 1e-3) / 1e12
    r = dict(bound="mfma", achieved=round(achieved, 1), peak=peak, unit="TFLOP/s",
             frac=round(achieved / peak, 4), traffic=load_traffic(kernel, workload),
             kernel=kernel, kernel_ms=round(ms, 5))
    if unit_bytes is not None:
        r["algorithmic_bytes"] = unit_bytes
    return r


def run_fwd_sweep(settle_s: float = 0.2, min_ms: float = 150.0, only: str = None):
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import WORKLOADS, workload_inputs

    out = {}
    for key, name, causal in SWEEP:
        if only is not None and key != only:
            continue
        w = WORKLOADS[name]
        q, k, v = (t.cuda() for t in workload_inputs(w, with_do=False))
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device="cuda")
        f32 = w.dtype == "f32"
        call = (lambda: fa.fa_fwd_f32(q, k, v, o, lse, causal, w.scale)) if f32 else \
               (lambda: fa.fa_fwd(q, k, v, o, lse, causal, w.scale))
        _settle(call, settle_s)
        reps = _repeats(call, 10, min_ms)
        ms = statistics.median(reps)
        flops = fwd_flops(w.B, w.H, w.N, w.d, causal)
        tf = flops / (ms * 1e-3) / 1e12
        ent = dict(B=w.B, H=w.H, N=w.N, d=w.d, causal=causal, dtype=w.dtype,
                   fwd_ms=round(ms, 5), fwd_ms_min=round(min(reps), 5),
                   repeats=len(reps), launches_per_repeat=_per_repeat(10), tflops=round(tf, 1))
        if f32:
            # two workgroups: a latency-bound correctness shape, no roofline claim
            ent["pct_of_fp32_peak"] = round(100 * tf / PEAK_FP32_TFLOPS, 2)
            ent["roofline"] = None
            ent["note"] = "2 workgroups on 256 CUs: launch- and latency-bound"
        else:
            ent["pct_of_bf16_peak"] = round(100 * tf / PEAK_BF16_TFLOPS, 1)
            ent["roofline"] = _roofline_mfma(
                flops, ms, fwd_kernel(w.d), key,
                unit_bytes=fwd_algorithmic_bytes(w.B, w.H, w.N, w.d))
        out[key] = ent
        del q, k, v, o, lse
    torch.cuda.empty_cache()
    return out


def _time_launches(fn, settle_s: float = 0.2, min_ms: float = 150.0, per_repeat: int = 10):
    """(median, min) ms per call of ``fn`` after a settle phase."""
    _settle(fn, settle_s)
    reps = _repeats(fn, per_repeat, min_ms)
    return statistics.median(reps), min(reps)


def run_extra_sweep(only: str = None):
    """Grouped-query, head-dimension-256 and different-length shapes:
    Llama-3.1-8B's real head sharing (32 query heads over 8 key/value heads)
    for the causal N = 4096 forward and backward, the d = 256 causal forward at
    [1, 16, 4096, 256], the e4m3 forward at [1, 32, 4096, 128] causal (against
    the fp8 peak), the d = 256 causal backward (fa_bwd: preprocess, key-tile
    kernel, query-tile dQ kernel), and decode -- one new token per sequence against a
    32k-token cache, split across workgroups by key range -- whose bound is
    HBM (every key and value byte is read once per key/value head)."""
    import torch
    import exact_tiled_attention_10_amd as fa
    from workloads import make_fp8_inputs, make_gqa_inputs

    def want(key):
        return only is None or only == key

    def entry(ms, ms_min, flops, peak=PEAK_BF16_TFLOPS, extra=None, kernel=None, key=None,
              unit_bytes=None):
        tf = flops / (ms * 1e-3) / 1e12
        e = dict(ms=round(ms, 5), ms_min=round(ms_min, 5), tflops=round(tf, 1),
                 pct_of_bf16_peak=round(100 * tf / PEAK_BF16_TFLOPS, 1))
        if peak != PEAK_BF16_TFLOPS:
            e["pct_of_fp8_peak"] = round(100 * tf / peak, 1)
        if kernel is not None:
            # one kernel per call: the call's time is the kernel's
            e["roofline"] = _roofline_mfma(flops, ms, kernel, key, peak=peak,
                                           unit_bytes=unit_bytes)
        e.update(extra or {})
        return e

    out = {}
    B, H, Hkv, N, d = 1, 32, 8, 4096, 128
    sc = 1 / math.sqrt(d)
    if want("llama8b_gqa32x8_n4096_causal_fwd") or want("llama8b_gqa32x8_n4096_causal_bwd"):
        q, k, v, do = (t.cuda() for t in make_gqa_inputs(B, H, Hkv, N, d, seed=6, with_do=True))
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
        fa.fa_fwd_gqa(q, k, v, o, lse, True, sc)
        if want("llama8b_gqa32x8_n4096_causal_fwd"):
            ms, mn = _time_launches(lambda: fa.fa_fwd_gqa(q, k, v, o, lse, True, sc))
            out["llama8b_gqa32x8_n4096_causal_fwd"] = entry(
                ms, mn, fwd_flops(B, H, N, d, True), kernel="fwd_bf16_kernel",
                key="llama8b_gqa32x8_n4096_causal_fwd",
                unit_bytes=2 * B * (H + Hkv) * N * d * 2 + B * H * N * 4)
        if want("llama8b_gqa32x8_n4096_causal_bwd"):
            dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
            ws = torch.empty(fa.fa_bwd_kv_workspace_size(B, H, Hkv, N, N, d),
                             dtype=torch.uint8, device="cuda")
            ms, mn = _time_launches(
                lambda: fa.fa_bwd_gqa(q, k, v, o, do, lse, dq, dk, dv, ws, True, sc),
                per_repeat=4)
            out["llama8b_gqa32x8_n4096_causal_bwd"] = entry(
                ms, mn, 2.5 * fwd_flops(B, H, N, d, True))
            del dq, dk, dv, ws
        del q, k, v, do, o, lse

    if want("d256_n4096_causal_bwd"):
        B2, H2, N2, d2 = 1, 16, 4096, 256
        q, k, v, do = (t.cuda() for t in make_gqa_inputs(B2, H2, H2, N2, d2, seed=9, with_do=True))
        o = torch.empty_like(q)
        lse = torch.empty((B2, H2, N2), dtype=torch.float32, device="cuda")
        fa.fa_fwd(q, k, v, o, lse, True, 1 / 16.0)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(fa.fa_bwd_workspace_size(B2, H2, N2, d2), dtype=torch.uint8,
                         device="cuda")
        ms, mn = _time_launches(
            lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, ws, True, 1 / 16.0),
            per_repeat=4)
        out["d256_n4096_causal_bwd"] = entry(ms, mn, 2.5 * fwd_flops(B2, H2, N2, d2, True))
        del q, k, v, do, o, lse, dq, dk, dv, ws

    if want("d256_n4096_causal_fwd"):
        B2, H2, N2, d2 = 1, 16, 4096, 256
        q, k, v = (t.cuda() for t in make_gqa_inputs(B2, H2, H2, N2, d2, seed=9))
        o = torch.empty_like(q)
        lse = torch.empty((B2, H2, N2), dtype=torch.float32, device="cuda")
        ms, mn = _time_launches(lambda: fa.fa_fwd(q, k, v, o, lse, True, 1 / 16.0))
        # one wave of workgroups under causal masking: the balanced-pair kernel
        out["d256_n4096_causal_fwd"] = entry(ms, mn, fwd_flops(B2, H2, N2, d2, True),
                                             kernel="fwd_d256_pair_kernel",
                                             key="d256_n4096_causal_fwd",
                                             unit_bytes=fwd_algorithmic_bytes(B2, H2, N2, d2))
        del q, k, v, o, lse

    if want("fp8_llama8b_n4096_causal_fwd"):
        q8, k8, v8, sq, sk, sv = make_fp8_inputs(1, 32, 4096, 128, seed=10)
        q8, k8, v8 = q8.cuda(), k8.cuda(), v8.cuda()
        o = torch.empty((1, 32, 4096, 128), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, 32, 4096), dtype=torch.float32, device="cuda")
        ms, mn = _time_launches(lambda: fa.fa_fwd_fp8(q8, k8, v8, o, lse, sq, sk, sv, True, sc))
        out["fp8_llama8b_n4096_causal_fwd"] = entry(
            ms, mn, fwd_flops(1, 32, 4096, 128, True), peak=PEAK_FP8_TFLOPS,
            kernel="fwd_fp8_kernel", key="fp8_llama8b_n4096_causal_fwd",
            unit_bytes=3 * 32 * 4096 * 128 + 32 * 4096 * 128 * 2 + 32 * 4096 * 4)
        del q8, k8, v8, o, lse

    if want("llama8b_decode_b8_gqa32x8_nk32768"):
        Bd, Nk = 8, 32768
        q = make_gqa_inputs(Bd, H, Hkv, 1, d, seed=7)[0].cuda()
        k, v = (t.cuda() for t in make_gqa_inputs(Bd, H, Hkv, Nk, d, seed=8)[1:])
        o = torch.empty_like(q)
        lse = torch.empty((Bd, H, 1), dtype=torch.float32, device="cuda")
        nb = fa.fa_fwd_kv_workspace_size(Bd, H, Hkv, 1, Nk, d)
        ws = torch.empty(max(nb, 1), dtype=torch.uint8, device="cuda")
        ms, mn = _time_launches(lambda: fa.fa_fwd_kv(q, k, v, o, lse, ws, True, sc),
                                per_repeat=20)
        nbytes = 2 * Bd * Hkv * Nk * d * 2 + 2 * Bd * H * d * 2 + Bd * H * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        out["llama8b_decode_b8_gqa32x8_nk32768"] = dict(
            ms=round(ms, 5), ms_min=round(mn, 5), algorithmic_bytes=nbytes, gbs=round(gbs, 1),
            frac_of_hbm_peak=round(gbs / PEAK_HBM_GBS, 4), workspace_bytes=nb,
            roofline=dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                          frac=round(gbs / PEAK_HBM_GBS, 4),
                          traffic=load_traffic("fwd_decode_kernel",
                                               "llama8b_decode_b8_gqa32x8_nk32768"),
                          kernel="fwd_decode_kernel + split merge", kernel_ms=round(ms, 5),
                          algorithmic_bytes=nbytes))
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
    head); throughput in the same counted-FLOP units as the GPU value.  Outside
    the timed loop, the heads it computed are compared with one GPU step (the
    bench's own step function): the largest absolute differences of O, lse,
    dQ, dK and dV, beside the stated tolerances."""
    import numpy as np
    import torch
    from oracle import naive_bwd, naive_fwd
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[STEP_WORKLOAD]
    q, k, v, do = workload_inputs(w, with_do=True)
    f64 = lambda t: t.float().numpy().astype(np.float64)  # noqa: E731
    sc = float(np.float32(w.scale))   # the scale as the kernels receive it
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    results = []
    t0 = time.perf_counter()
    for (b, h) in heads:
        qq, kk, vv, gg = f64(q[b, h]), f64(k[b, h]), f64(v[b, h]), f64(do[b, h])
        fo = naive_fwd(qq, kk, vv, sc, True)
        bo = naive_bwd(qq, kk, vv, gg, sc, True)
        results.append(((b, h), fo, bo))
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 3.5 * fwd_flops(1, done, w.N, w.d, True)

    step, t = make_step()
    step()
    torch.cuda.synchronize()
    err = dict(o=0.0, lse=0.0, dq=0.0, dk=0.0, dv=0.0)
    for (b, h), (o_ref, lse_ref), (dq_ref, dk_ref, dv_ref) in results:
        for key, ref in (("o", o_ref), ("lse", lse_ref), ("dq", dq_ref), ("dk", dk_ref),
                         ("dv", dv_ref)):
            got = t[key][b, h].float().cpu().numpy().astype(np.float64)
            err[key] = max(err[key], float(np.max(np.abs(got - ref))))
    del step, t
    torch.cuda.empty_cache()
    return dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s", cores=_blas_threads(),
                kind="oracle",
                sample=f"{done} of {len(heads)} (batch, head) slices of {w.name}, float64 "
                       f"forward + backward, {dt:.1f} s wall",
                host_cpu=platform.processor() or platform.machine(),
                host_logical_cpus=os.cpu_count(),
                max_abs_err_vs_gpu={key: float(f"{e:.3e}") for key, e in err.items()},
                tolerance=dict(o=2e-2, dq=2e-2, dk=2e-2, dv=2e-2, lse=1e-3))


def run_cpu_sweep(budget_s: float, rows: int = 256, only: str = None):
    """The float64 oracle timed beside each forward shape: query rows of head
    (0, 0), ``rows`` at a time spread evenly over the sequence, until
    ``budget_s`` of wall time per shape; counted FLOP pro rata (each row of a
    causal head counts 2*N*d, of a non-causal one 4*N*d, the convention's
    average), so the figure scales to the whole workload."""
    import numpy as np
    from oracle import naive_fwd_rows
    from workloads import WORKLOADS, workload_inputs

    out = {}
    for key, name, causal in SWEEP:
        if only is not None and key != only:
            continue
        w = WORKLOADS[name]
        q, k, v = workload_inputs(w, with_do=False)
        qq = q[0, 0].float().numpy().astype(np.float64)
        kk = k[0, 0].float().numpy().astype(np.float64)
        vv = v[0, 0].float().numpy().astype(np.float64)
        sc = float(np.float32(w.scale))   # the scale as the kernels receive it
        r = min(rows, w.N)
        done = 0
        start = 0
        first = None
        t0 = time.perf_counter()
        while True:
            pos = (np.arange(r) * (w.N // r) + start) % w.N
            res = naive_fwd_rows(qq[pos], kk, vv, sc, causal, pos)
            if first is None:
                first = (pos, res)
            done += r
            start += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        flops = fwd_flops(1, 1, w.N, w.d, causal) * done / w.N
        # outside the timed loop: the first rows against one GPU forward
        err_o, err_lse = _gpu_rows_err(w, causal, q, k, v, first[0], first[1])
        f32 = w.dtype == "f32"
        out[key] = dict(value=round(flops / dt / 1e12, 6), unit="TFLOP/s",
                        cores=_blas_threads(), kind="oracle",
                        sample=f"{done} query rows of head (0, 0) of {w.name} "
                               f"({'causal' if causal else 'non-causal'}), float64, "
                               f"{dt:.1f} s wall; counted FLOP pro rata",
                        rows_checked=int(len(first[0])),
                        max_abs_err_vs_gpu=dict(o=float(f"{err_o:.3e}"),
                                                lse=float(f"{err_lse:.3e}")),
                        tolerance=dict(o=1e-5 if f32 else 2e-2, lse=1e-5 if f32 else 1e-3))
    return out


def _gpu_rows_err(w, causal, q, k, v, pos, ref):
    """Largest |GPU - oracle| of O and lse over query rows ``pos`` of head
    (0, 0), from one GPU forward of the whole workload."""
    import numpy as np
    import torch
    import exact_tiled_attention_10_amd as fa
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    o = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    if w.dtype == "f32":
        fa.fa_fwd_f32(qd, kd, vd, o, lse, causal, w.scale)
    else:
        fa.fa_fwd(qd, kd, vd, o, lse, causal, w.scale)
    torch.cuda.synchronize()
    idx = torch.as_tensor(pos, dtype=torch.long, device="cuda")
    got_o = o[0, 0].index_select(0, idx).float().cpu().numpy().astype(np.float64)
    got_l = lse[0, 0].index_select(0, idx).cpu().numpy().astype(np.float64)
    del qd, kd, vd, o, lse
    torch.cuda.empty_cache()
    return float(np.max(np.abs(got_o - ref[0]))), float(np.max(np.abs(got_l - ref[1])))


# ---------------------------------------------------------------------------
# traffic (rocprofv3 counters) bookkeeping
# ---------------------------------------------------------------------------

def _load_traffic_file():
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return {"entries": []}
    return t if isinstance(t, dict) and "entries" in t else {"entries": []}


def load_traffic(kernel: str, workload: str):
    """Counter-derived HBM bytes per launch of ``kernel`` on ``workload``, or
    None when none were taken or the kernel's sources changed since."""
    for e in _load_traffic_file()["entries"]:
        if e.get("kernel") == kernel and e.get("workload") == workload:
            if e.get("source_hash") != source_hash(kernel):
                return None
            return e.get("bytes_per_launch")
    return None


def _read_counter_csv(path, counter):
    """{kernel name -> list of per-dispatch values} from a rocprofv3
    counter_collection.csv."""
    rows = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if r.get("Counter_Name") != counter:
                continue
            rows.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return rows


def pmc_summary(fetch_csv: str, write_csv: str, copy_mib: float, kernel: str,
                workload: str, algorithmic_bytes: float = None) -> dict:
    fetch = _read_counter_csv(fetch_csv, "FETCH_SIZE")
    write = _read_counter_csv(write_csv, "WRITE_SIZE")

    def pick(table, needle):
        ks = [k for k in table if needle in k]
        if not ks:
            raise SystemExit(f"no kernel matching {needle!r} in counters")
        vals = [x for k in ks for x in table[k]]
        return ks[0], sum(vals) / len(vals), len(vals)

    copy_bytes = copy_mib * 2 ** 20
    _, cf, _ = pick(fetch, "copy")           # KiB read by the copy kernel
    _, cw, _ = pick(write, "copy")
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    name, kf, nd = pick(fetch, kernel)
    _, kw, _ = pick(write, kernel)
    bytes_per_launch = kf * 1024.0 * f_scale + kw * 1024.0 * w_scale
    ent = dict(kernel=kernel, workload=workload, kernel_symbol=name,
               source_hash=source_hash(kernel), dispatches=nd,
               fetch_kib_raw=kf, write_kib_raw=kw, copy_mib=copy_mib,
               copy_fetch_kib_raw=cf, copy_write_kib_raw=cw,
               fetch_scale=f_scale, write_scale=w_scale,
               fetch_bytes=kf * 1024.0 * f_scale, write_bytes=kw * 1024.0 * w_scale,
               bytes_per_launch=bytes_per_launch)
    if algorithmic_bytes:
        ent["algorithmic_bytes"] = algorithmic_bytes
        ent["traffic_over_algorithmic"] = bytes_per_launch / algorithmic_bytes
    t = _load_traffic_file()
    t["entries"] = [e for e in t["entries"]
                    if not (e.get("kernel") == kernel and e.get("workload") == workload)]
    t["entries"].append(ent)
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
    return ent


def copy_calibration(mib: float):
    import torch
    n = int(mib * 2 ** 20)
    x = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    return dict(copy_mib=mib, bytes=n)


def run_only(name: str, launches: int, settle_s: float = 0.0):
    """One workload, nothing else, so each kernel's dispatches in a profiler
    run belong to one shape: the step (``settle_s`` of untimed steps, then
    ``launches`` more), or one sweep shape timed as the full run times it
    (a settle phase, then repeats covering at least 150 ms)."""
    import torch
    if name == "step":
        step, _ = make_step()
        if settle_s > 0:
            _settle(step, settle_s)
        for _ in range(launches):
            step()
        torch.cuda.synchronize()
        return dict(only=name, launches=launches, settle_s=settle_s)
    if name in {k for k, _, _ in SWEEP}:
        r = run_fwd_sweep(only=name)
    else:
        r = run_extra_sweep(only=name)
        if not r:
            raise SystemExit(f"unknown workload {name!r}")
    return dict(only=name, result=r)


# ---------------------------------------------------------------------------

def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-s", type=float, default=0.5,
                    help="seconds of untimed steps before the counted warm-up")
    ap.add_argument("--min-timed-ms", type=float, default=250.0,
                    help="GPU time the timed repeats must cover")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="wall-time budget of the oracle CPU baseline")
    ap.add_argument("--cpu-sweep-seconds", type=float, default=2.0,
                    help="wall-time budget of the oracle beside each forward shape")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--only", default=None, metavar="NAME")
    ap.add_argument("--launches", type=int, default=5)
    ap.add_argument("--only-settle-s", type=float, default=0.0,
                    help="with --only step: seconds of untimed steps before the launches")
    ap.add_argument("--copy-calibration", type=float, default=None, metavar="MIB")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"))
    ap.add_argument("--kernel", default="bwd_main_kernel")
    ap.add_argument("--workload", default=STEP_WORKLOAD)
    ap.add_argument("--algorithmic-bytes", type=float, default=None)
    ap.add_argument("--copy-mib", type=float, default=256.0)
    ap.add_argument("--cold", action="store_true",
                    help=f"write a {COLD_MIB} MiB buffer before every timed repeat of one call")
    args = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}); run with --gpus 1.",
              file=sys.stderr, flush=True)
        return 2

    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1],
                                     args.copy_mib, args.kernel, args.workload,
                                     args.algorithmic_bytes)))
        return 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    set_cold(args.cold)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(args.copy_calibration)), flush=True)
    if args.only:
        print(json.dumps(run_only(args.only, args.launches, args.only_settle_s)), flush=True)
        return 0

    r = run_step_bench(args.steps, args.warmup, args.settle_s, args.min_timed_ms)
    w = r["workload"]
    ms = r["ms_per_step"]
    value = r["step_flops"] / (ms * 1e-3) / 1e12
    km = r["kernel_ms"]

    # dominant kernel of the step: the longer of the forward and backward main kernels
    if km["main"] >= km["fwd"]:
        roofline = _roofline_mfma(r["bwd_flops"], km["main"], "bwd_main_kernel", STEP_WORKLOAD)
    else:
        roofline = _roofline_mfma(r["fwd_flops"], km["fwd"], fwd_kernel(w.d), STEP_WORKLOAD)
    roofline["algorithmic_bytes_whole_backward"] = bwd_algorithmic_bytes(w.B, w.H, w.N, w.d)

    line = dict(
        metric=METRIC, value=round(value, 2), unit="TFLOP/s", n_gpus=1,
        steps=args.steps, warmup=args.warmup, ms_per_step=round(ms, 5),
        higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic",
        config=dict(workload=w.name, B=w.B, H=w.H, N=w.N, d=w.d, causal=True,
                    step="fa_fwd + fa_bwd (preprocess, main, finalize)",
                    pct_of_bf16_peak=round(100 * value / PEAK_BF16_TFLOPS, 2)),
        timing=dict(settle_s=r["settle_s"], settle_steps=r["settle_steps"],
                    repeats=r["repeats"], steps_per_repeat=r["steps_per_repeat"],
                    caches=(f"cold: {COLD_MIB} MiB written before every timed step"
                            if args.cold else "warm"),
                    timed_ms=round(r["timed_ms"], 2),
                    ms_per_step_median=round(ms, 5), ms_per_step_min=round(r["ms_min"], 5),
                    ms_per_step_mean=round(r["ms_mean"], 5),
                    value_at_min=round(r["step_flops"] / (r["ms_min"] * 1e-3) / 1e12, 2),
                    instrumented_ms_per_step=round(r["instrumented_ms_per_step"], 5),
                    kernel_ms_median={k: round(v, 5) for k, v in km.items()},
                    kernel_timing="HIP events around each kernel on its launch stream, in "
                                  "a second pass of the same repeats (the timed steps "
                                  "carry no events)"),
        roofline=roofline,
        context=PAGES_CONTEXT,
    )
    if not args.no_sweep:
        line["fwd_sweep"] = run_fwd_sweep()
        line["extra_sweep"] = run_extra_sweep()
    if not args.no_cpu_baseline:
        cb = run_cpu_baseline(args.cpu_seconds)
        cb["gpu_over_oracle"] = round(value / cb["value"], 1) if cb["value"] > 0 else None
        line["cpu_baseline"] = cb
        if not args.no_sweep:
            cs = run_cpu_sweep(args.cpu_sweep_seconds)
            for key, ent in cs.items():
                gpu = line["fwd_sweep"][key]["tflops"]
                ent["gpu_over_oracle"] = round(gpu / ent["value"], 1) if ent["value"] > 0 else None
                line["fwd_sweep"][key]["cpu_baseline"] = ent
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
