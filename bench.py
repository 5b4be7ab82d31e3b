#!/usr/bin/env python3
"""Benchmark of the fused attention forward on one MI355X.

One step is one pass of the whole path over synthetic inputs already resident
in HBM:
  * the compute-bound causal prefill, B=4, Hq=Hkv=16, Sq=Sk=4096, D=128, bf16
    (one fa_fwd call: the persistent prefill kernel), and
  * the memory-bound decode, B=32, Hq=32, Hkv=8, Sq=1, Sk=8192, D=128, bf16
    (one fa_fwd call: the split-key kernel and the log-sum-exp merge), and
  * the same decode over a paged K/V cache (16-key pages scattered over the
    cache): every sequence at 8192 keys, then lengths drawn from [1, 16384]
    (one fa_fwd_paged call each: paged split kernel and merge), and
  * head dim 256: a causal prefill, B=2, H=16, S=4096, and the decode shape
    (one fa_fwd call each), and
  * the causal prefill's shape on FP8 E4M3 inputs (one fa_fwd_fp8 call), and
  * the backward of the causal prefill (one fa_bwd call: delta, dK/dV, dQ
    kernels) on the prefill's own O and LSE and a seeded dO, and
  * the other three shapes of the suite, one fa_fwd call each: the
    single-head B=1 H=1 S=128 D=64 (fp32 O), the small causal prefill
    B=2 H=8 S=1024 D=64 and the long non-causal GQA prefill B=1 Hq=32 Hkv=8
    S=16384 D=128.
All go to the same stream; HIP events recorded on that stream around each
call give the per-call durations.

Printed: one JSON line.  `value` is the prefill's algorithmic TFLOP/s (4*D
flops per allowed query-key pair); `decode` holds the decode's algorithmic
GB/s (Q, K, V read once, O and LSE written once), `paged_decode` and
`paged_decode_ragged` the paged calls' (plus the block-table entries read),
`d256_prefill` / `d256_decode` the head-dim-256 calls' TFLOP/s and GB/s,
`fp8_prefill` the FP8 call's TFLOP/s against the dense FP8 MFMA peak,
`backward` the backward's TFLOP/s (algorithmic: 5 products, 2.5x the
forward's FLOPs) against the bf16 peak, `single_head`, `causal_small` and
`gqa_long` the other shapes' TFLOP/s.  `ceilings` are same-machine loops (HBM
streaming read, MFMA issue and the clock it runs at, LDS and VALU rates) that
the datasheet peaks are read against; `conditions` the GPU, ROCm, power cap
and the shader/memory clocks sampled while the step ran without pause;
`host` the CPU the baseline ran on.
`roofline` is the prefill kernel against the dense bf16 MFMA peak; the decode
entries' `roofline` their call against HBM.  `cpu_baseline` times the fp64 oracle on a bounded sample of the
prefill workload's rows and also compares those rows with the timed output.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]

The default warm-up is 100 steps (about 50 ms of GPU work): from idle the
shader clock takes about 30 ms of load to reach its steady level, and steps
timed before that run up to 30 % slower.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("attention fwd TFLOP/s + % bf16 MFMA peak (causal S=4096 D=128); "
          "decode HBM GB/s")
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA (datasheet)
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E (datasheet)
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (datasheet)
PREFILL = "causal_b4_h16_s4096_d128"
DECODE = "decode_b32_hq32_hkv8_sk8192_d128"
PAGED = "paged_decode_b32_hq32_hkv8_len8192_ps16_d128"
PAGED_RAGGED = "paged_decode_b32_hq32_hkv8_ragged16384_ps16_d128"
PREFILL_D256 = "causal_b2_h16_s4096_d256"
DECODE_D256 = "decode_b32_hq32_hkv8_sk8192_d256"
PREFILL_FP8 = "causal_b4_h16_s4096_d128_fp8"
SINGLE = "single_head_s128_d64"
SMALL = "causal_b2_h8_s1024_d64"
GQA = "gqa_b1_hq32_hkv8_s16384_d128"
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")
DEVICE_SHA = os.path.join(ROOT, "attention_fwd_02_amd", "libfa.so.device-sha256")


def log(msg):
    """Progress on stderr (stdout carries only the JSON line)."""
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def roofline(achieved, peak, unit, bound, traffic=None):
    return {"bound": bound, "achieved": round(achieved, 3), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic}


def device_code_hash():
    """sha256 of the built kernels' gfx950 assembly (written by the build)."""
    try:
        with open(DEVICE_SHA) as f:
            return f.read().strip()
    except OSError:
        return None


def measured_traffic(key):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when the kernels' device code changed since they were taken."""
    try:
        with open(COUNTERS) as f:
            c = json.load(f)[key]
    except (OSError, KeyError, ValueError):
        return None
    h = device_code_hash()
    if h is None or c.get("device_code_sha256") != h:
        return None
    return int(c["hbm_bytes_per_launch"])


def cpu_baseline_leg(w, q, k, v, o_gpu, lse_gpu, seconds):
    """The oracle as it stands, on a bounded sample of the workload's rows,
    timed on this host's cores; the sampled rows of the timed GPU output are
    compared with it on the way."""
    import numpy as np
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from tests.helpers import check

    threads = oracle.default_threads()
    rng = np.random.default_rng(1234)

    def rows_of(n):
        idx = rng.choice(w.B * w.Hq * w.Sq, size=n, replace=False)
        b = idx // (w.Hq * w.Sq)
        h = (idx // w.Sq) % w.Hq
        i = idx % w.Sq
        return np.stack([b, h, i], axis=1).astype(np.int64)

    def flops_of(rows):
        off = w.Sk - w.Sq
        keys = np.clip(rows[:, 2] + off + 1, 0, w.Sk) if w.causal else np.full(len(rows), w.Sk)
        return int(4 * w.D * keys.sum())

    cal = rows_of(4 * threads)
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, w.causal, w.scale, rows=cal, nthreads=threads)
    t_cal = max(time.perf_counter() - t0, 1e-3)
    n = int(min(w.B * w.Hq * w.Sq, max(len(cal), len(cal) * seconds / t_cal)))
    rows = rows_of(n)
    t0 = time.perf_counter()
    o_ref, lse_ref = oracle.attn_fwd(q, k, v, w.causal, w.scale, rows=rows, nthreads=threads)
    dt = time.perf_counter() - t0
    fl = flops_of(rows)

    og = o_gpu.float().cpu().numpy().astype(np.float64)
    lg = lse_gpu.float().cpu().numpy().astype(np.float64)
    o_s = np.stack([og[b, i, h] for b, h, i in rows])
    l_s = np.array([lg[b, h, i] for b, h, i in rows])
    eo, el = check(o_s, l_s, o_ref, lse_ref, w.o_dtype, "timed output")
    err = np.abs(o_s - o_ref)
    over = err > 1e-2
    return {
        "value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} random query rows of the {PREFILL} workload "
                   f"({fl / 1e9:.1f} GFLOP algorithmic, {dt:.1f} s, fp64, "
                   f"{threads} threads)"),
        "parity_on_timed_output": {
            "rows": n, "max_abs_dO": eo, "max_abs_dLSE": el,
            "elements": int(err.size),
            "elements_over_flat_1e-2": int(over.sum()),
            "abs_O_range_of_those": ([float(np.abs(o_ref[over]).min()),
                                      float(np.abs(o_ref[over]).max())] if over.any() else None),
            "rule": ("|dO| <= 1e-2 + half a bf16 ulp of the oracle's value (the output's own "
                     "rounding), |dLSE| <= 1e-3"),
        },
    }


def host_facts():
    """The CPU the baseline ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        aff = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        aff = None
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            quota = f.read().strip()
    except OSError:
        pass
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "affinity_cpus": aff,
            "cgroup_cpu_max": quota}


def _smi(args, timeout=20):
    """Output of rocm-smi with `args` (JSON), or None."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", *args, "--json"], capture_output=True, text=True,
                           timeout=timeout)
        return json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip() else None
    except (OSError, ValueError, subprocess.SubprocessError):
        return None


def _pick(d, words):
    """Values of `d` (card entries of a rocm-smi JSON) whose key holds all of `words`."""
    out = {}
    if isinstance(d, dict):
        for card, ent in d.items():
            if isinstance(ent, dict):
                for k, v in ent.items():
                    if all(w in k.lower() for w in words):
                        out[k] = v
    return out


def sustained_clocks(run_for, seconds):
    """Keep the step running back to back for `seconds` while a thread samples
    rocm-smi's current clocks; returns the samples and the steps' own pace."""
    import threading
    samples, stop = [], threading.Event()

    def sampler():
        while not stop.is_set():
            c = _smi(["--showclocks"])
            if c is not None:
                samples.append({**_pick(c, ["sclk"]), **_pick(c, ["mclk"])})

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    ms = run_for(seconds)
    stop.set()
    th.join(timeout=30)

    def mhz(word):
        vals = []
        for smp in samples:
            for k, v in smp.items():
                m = re.search(r"(\d+)\s*mhz", str(v).lower())
                if word in k.lower() and "speed" in k.lower() and m:
                    vals.append(int(m.group(1)))
        vals.sort()
        return ({"min": vals[0], "median": vals[len(vals) // 2], "max": vals[-1], "n": len(vals)}
                if vals else None)

    return {"seconds": seconds, "ms_per_step": ms, "sclk_MHz": mhz("sclk"),
            "mclk_MHz": mhz("mclk"), "source": "rocm-smi --showclocks, sampled back to back"}


def profile_one(args):
    """Run one call `warmup + steps` times on its own (for rocprofv3 --pmc)."""
    import torch
    from attention_fwd_02_amd import _binding as fa
    from attention_fwd_02_amd.inputs import WORKLOADS, make_inputs
    dev = "cuda:0"
    from attention_fwd_02_amd.inputs import PAGED_WORKLOADS, make_paged_inputs
    if args.profile_kernel == "copy":
        n = 1 << 30
        x = torch.empty(n // 2, dtype=torch.bfloat16, device=dev).fill_(1.0)
        y = torch.empty_like(x)
        fn = lambda: y.copy_(x)  # noqa: E731
        label = f"copy of {n} bytes"
    elif args.profile_kernel in ("paged", "paged_ragged"):
        w = PAGED_WORKLOADS[PAGED if args.profile_kernel == "paged" else PAGED_RAGGED]
        q, kc, vc, table, lens = (t.to(dev) for t in make_paged_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        fn = lambda: fa.fa_fwd_paged(q, kc, vc, table, lens, o, lse, w.causal, w.scale)  # noqa: E731
        label = w.name
    elif args.profile_kernel == "prefill_fp8":
        from attention_fwd_02_amd.inputs import FP8_WORKLOADS, make_fp8_inputs
        w = FP8_WORKLOADS[PREFILL_FP8]
        q, k, v, dq, dk, dv = make_fp8_inputs(w, device=dev)
        o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        fn = lambda: fa.fa_fwd_fp8(q, k, v, o, lse, w.causal, w.scale, dq, dk, dv)  # noqa: E731
        label = w.name
    elif args.profile_kernel == "bwd":
        w = WORKLOADS[PREFILL]
        q, k, v = (t.to(dev) for t in make_inputs(w))
        do = torch.randn(q.shape, generator=torch.Generator().manual_seed(65)).to(
            torch.bfloat16).to(dev)
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        fa.fa_fwd(q, k, v, o, lse, w.causal, w.scale)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        fn = lambda: fa.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, w.causal, w.scale)  # noqa: E731
        label = w.name + " backward"
    elif args.profile_kernel in ("prefill_d256", "decode_d256"):
        from attention_fwd_02_amd.inputs import HEADDIM_WORKLOADS
        w = HEADDIM_WORKLOADS[PREFILL_D256 if args.profile_kernel == "prefill_d256"
                              else DECODE_D256]
        q, k, v = (t.to(dev) for t in make_inputs(w))
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        fn = lambda: fa.fa_fwd(q, k, v, o, lse, w.causal, w.scale)  # noqa: E731
        label = w.name
    else:
        w = WORKLOADS[{"prefill": PREFILL, "decode": DECODE, "single_head": SINGLE,
                       "causal_small": SMALL, "gqa_long": GQA}[args.profile_kernel]]
        q, k, v = (t.to(dev) for t in make_inputs(w))
        o = torch.empty(q.shape, dtype=torch.float32 if w.o_dtype == "f32" else torch.bfloat16,
                        device=dev)
        lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev)
        fn = lambda: fa.fa_fwd_ex(q, k, v, o, lse, w.causal, w.scale)  # noqa: E731
        label = w.name
    for _ in range(args.warmup + args.steps):
        fn()
    torch.cuda.synchronize()
    print(f"profiled {label}: {args.warmup + args.steps} calls", flush=True)
    return 0


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=25.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true")
    ap.add_argument("--settle-seconds", type=float, default=2.0,
                    help="back-to-back steps after the warm-up while the clocks are sampled")
    ap.add_argument("--profile-kernel",
                    choices=["prefill", "decode", "paged", "paged_ragged", "prefill_d256",
                             "decode_d256", "prefill_fp8", "bwd", "single_head", "causal_small",
                             "gqa_long", "copy"],
                    help="run only this call (warmup + steps) for counter collection; "
                         "'copy' is a plain 1 GiB device-to-device copy that calibrates "
                         "the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU sharding is a design note only).", file=sys.stderr)
        return 2

    import torch
    from attention_fwd_02_amd import _binding as fa
    from attention_fwd_02_amd.inputs import (FP8_WORKLOADS, HEADDIM_WORKLOADS, PAGED_WORKLOADS,
                                             WORKLOADS, make_fp8_inputs, make_inputs,
                                             make_paged_inputs)

    dev = "cuda:0"
    torch.cuda.set_device(0)
    if args.profile_kernel:
        return profile_one(args)
    wp, wd = WORKLOADS[PREFILL], WORKLOADS[DECODE]
    qp_h, kp_h, vp_h = make_inputs(wp)
    qp, kp, vp = (t.to(dev) for t in (qp_h, kp_h, vp_h))
    op = torch.empty_like(qp)
    lp = torch.empty((wp.B, wp.Hq, wp.Sq), dtype=torch.float32, device=dev)
    qd, kd, vd = (t.to(dev) for t in make_inputs(wd))
    od = torch.empty_like(qd)
    ld = torch.empty((wd.B, wd.Hq, wd.Sq), dtype=torch.float32, device=dev)

    paged = {}
    for key in (PAGED, PAGED_RAGGED):
        w = PAGED_WORKLOADS[key]
        q, kc, vc, table, lens = make_paged_inputs(w)
        paged[key] = (w, lens.tolist(), tuple(t.to(dev) for t in (q, kc, vc, table, lens)),
                      torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device=dev),
                      torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev))

    d256 = {}
    for key in (PREFILL_D256, DECODE_D256):
        w = HEADDIM_WORKLOADS[key]
        q, k, v = (t.to(dev) for t in make_inputs(w))
        d256[key] = (w, q, k, v, torch.empty_like(q),
                     torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev))

    wf = FP8_WORKLOADS[PREFILL_FP8]
    qf8, kf8, vf8, dqf, dkf, dvf = make_fp8_inputs(wf, device=dev)
    of8 = torch.empty(qf8.shape, dtype=torch.bfloat16, device=dev)
    lf8 = torch.empty((wf.B, wf.Hq, wf.Sq), dtype=torch.float32, device=dev)

    dop = torch.randn(qp.shape, generator=torch.Generator().manual_seed(65)).to(
        torch.bfloat16).to(dev)
    dqp, dkp, dvp = torch.empty_like(qp), torch.empty_like(kp), torch.empty_like(vp)

    suite = {}
    for key in (SINGLE, SMALL, GQA):
        w = WORKLOADS[key]
        q, k, v = (t.to(dev) for t in make_inputs(w))
        o = torch.empty(q.shape, dtype=torch.float32 if w.o_dtype == "f32" else torch.bfloat16,
                        device=dev)
        suite[key] = (w, q, k, v, o,
                      torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device=dev))

    stream = torch.cuda.current_stream()

    def prefill():
        fa.fa_fwd(qp, kp, vp, op, lp, wp.causal, wp.scale, stream=stream)

    def decode():
        fa.fa_fwd(qd, kd, vd, od, ld, wd.causal, wd.scale, stream=stream)

    def paged_call(key):
        w, _, (q, kc, vc, table, lens), o, lse = paged[key]
        fa.fa_fwd_paged(q, kc, vc, table, lens, o, lse, w.causal, w.scale, stream=stream)

    def d256_call(key):
        w, q, k, v, o, lse = d256[key]
        fa.fa_fwd(q, k, v, o, lse, w.causal, w.scale, stream=stream)

    def fp8_call():
        fa.fa_fwd_fp8(qf8, kf8, vf8, of8, lf8, wf.causal, wf.scale, dqf, dkf, dvf, stream=stream)

    def bwd_call():
        fa.fa_bwd(qp, kp, vp, op, dop, lp, dqp, dkp, dvp, wp.causal, wp.scale, stream=stream)

    def suite_call(key):
        w, q, k, v, o, lse = suite[key]
        fa.fa_fwd_ex(q, k, v, o, lse, w.causal, w.scale, stream=stream)

    calls = (prefill, decode, lambda: paged_call(PAGED), lambda: paged_call(PAGED_RAGGED),
             lambda: d256_call(PREFILL_D256), lambda: d256_call(DECODE_D256), fp8_call,
             bwd_call, lambda: suite_call(SINGLE), lambda: suite_call(SMALL),
             lambda: suite_call(GQA))

    def step(evs=None):
        for i, call in enumerate(calls):
            if evs:
                evs[i].record(stream)
            call()
        if evs:
            evs[len(calls)].record(stream)

    log("inputs resident; warm-up")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"{args.warmup} warm-up steps done")

    def run_for(seconds):
        t0, n = time.perf_counter(), 0
        while time.perf_counter() - t0 < seconds:
            for _ in range(10):
                step()
            torch.cuda.synchronize()
            n += 10
        return round((time.perf_counter() - t0) * 1e3 / max(n, 1), 4)

    clocks = sustained_clocks(run_for, args.settle_seconds) if args.settle_seconds > 0 else None

    log("clocks sampled; timed steps")
    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
           for _ in range(K)]
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for s in range(K):
        step(evs[s])
    stop.record(stream)
    torch.cuda.synchronize()

    total_ms = start.elapsed_time(stop)
    p_ms = sorted(e[0].elapsed_time(e[1]) for e in evs)
    d_ms = sorted(e[1].elapsed_time(e[2]) for e in evs)
    p_avg = sum(p_ms) / K
    d_avg = sum(d_ms) / K

    def paged_entry(key, i):
        w, lens, (_, kc, _, table, _), _, _ = paged[key]
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        avg = sum(ms) / K
        nbytes = w.hbm_bytes(lens)
        gb = nbytes / (avg * 1e-3) / 1e9
        return {
            "workload": key, "value": round(gb, 1), "unit": "GB/s",
            "config": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "D": w.D,
                       "page_size": w.page_size, "max_len": w.max_len, "lengths": w.lengths,
                       "total_keys": sum(lens), "algorithmic_bytes": nbytes,
                       "plan": fa.fa_plan_paged(w.B, w.Hq, w.Hkv, w.Sq, w.D, kc.shape[0],
                                                w.page_size, table.shape[1], 0)},
            "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4), "min": round(ms[0], 4)},
            "roofline": roofline(gb, PEAK_HBM_GBPS, "GB/s", "hbm",
                                 measured_traffic("paged" if key == PAGED else "paged_ragged")),
        }

    def d256_entry(key, i):
        w = d256[key][0]
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        avg = sum(ms) / K
        plan = fa.fa_plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.causal, 0)
        cfg = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk, "D": w.D,
               "causal": w.causal, "plan": plan}
        if w.Sq > 1:
            tf = w.flops() / (avg * 1e-3) / 1e12
            cfg["algorithmic_flops"] = w.flops()
            return {"workload": key, "value": round(tf, 3), "unit": "TFLOP/s", "config": cfg,
                    "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4),
                           "min": round(ms[0], 4)},
                    "roofline": roofline(tf, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                                         measured_traffic("prefill_d256"))}
        gb = w.hbm_bytes() / (avg * 1e-3) / 1e9
        cfg["algorithmic_bytes"] = w.hbm_bytes()
        return {"workload": key, "value": round(gb, 1), "unit": "GB/s", "config": cfg,
                "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4),
                       "min": round(ms[0], 4)},
                "roofline": roofline(gb, PEAK_HBM_GBPS, "GB/s", "hbm",
                                     measured_traffic("decode_d256"))}

    def fp8_entry(i):
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        avg = sum(ms) / K
        tf = wf.flops() / (avg * 1e-3) / 1e12
        return {"workload": PREFILL_FP8, "value": round(tf, 3), "unit": "TFLOP/s",
                "config": {"B": wf.B, "Hq": wf.Hq, "Hkv": wf.Hkv, "Sq": wf.Sq, "Sk": wf.Sk,
                           "D": wf.D, "causal": wf.causal, "inputs": "FP8 E4M3, per-tensor descale",
                           "algorithmic_flops": wf.flops()},
                "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4),
                       "min": round(ms[0], 4)},
                "roofline": roofline(tf, PEAK_FP8_TFLOPS, "TFLOP/s", "mfma",
                                     measured_traffic("prefill_fp8"))}

    def suite_entry(key, i):
        w = suite[key][0]
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        avg = sum(ms) / K
        tf = w.flops() / (avg * 1e-3) / 1e12
        return {"workload": key, "value": round(tf, 3), "unit": "TFLOP/s",
                "config": {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Sq": w.Sq, "Sk": w.Sk,
                           "D": w.D, "causal": w.causal, "o_dtype": w.o_dtype,
                           "algorithmic_flops": w.flops(),
                           "plan": fa.fa_plan(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.causal, 0)},
                "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4),
                       "min": round(ms[0], 4)},
                "roofline": roofline(tf, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                                     measured_traffic({SINGLE: "single_head", SMALL: "causal_small",
                                                       GQA: "gqa_long"}[key]))}

    def bwd_entry(i):
        ms = sorted(e[i].elapsed_time(e[i + 1]) for e in evs)
        avg = sum(ms) / K
        fl = 5 * wp.flops() // 2
        tf = fl / (avg * 1e-3) / 1e12
        return {"workload": PREFILL + " backward", "value": round(tf, 3), "unit": "TFLOP/s",
                "config": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Sq": wp.Sq, "Sk": wp.Sk,
                           "D": wp.D, "causal": wp.causal, "algorithmic_flops": fl,
                           "flops_rule": "5 products (S, dP, dV, dK, dQ) of 2*D per allowed pair"},
                "ms": {"avg": round(avg, 4), "median": round(ms[K // 2], 4),
                       "min": round(ms[0], 4)},
                "roofline": roofline(tf, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                                     measured_traffic("bwd"))}

    flops = wp.flops()
    tflops = flops / (p_avg * 1e-3) / 1e12
    dbytes = wd.hbm_bytes()
    gbps = dbytes / (d_avg * 1e-3) / 1e9

    plan_p = fa.fa_plan(wp.B, wp.Hq, wp.Hkv, wp.Sq, wp.Sk, wp.D, wp.causal, 0)
    plan_d = fa.fa_plan(wd.B, wd.Hq, wd.Hkv, wd.Sq, wd.Sk, wd.D, wd.causal, 0)
    props = torch.cuda.get_device_properties(0)

    out = {
        "metric": METRIC,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (f"{PREFILL} (causal prefill B=4 Hq=Hkv=16 Sq=Sk=4096 D=128) + "
                         f"{DECODE} (decode B=32 Hq=32 Hkv=8 Sq=1 Sk=8192 D=128) + "
                         f"{PAGED} and {PAGED_RAGGED} (the decode over 16-key pages; "
                         "8192 keys each, then lengths drawn from [1, 16384]) + "
                         f"{PREFILL_D256} and {DECODE_D256} (head dim 256) + "
                         f"{PREFILL_FP8} (the causal prefill on FP8 E4M3 inputs) + "
                         f"the backward of {PREFILL} + {SINGLE}, {SMALL} and {GQA}"),
            "prefill": {"B": wp.B, "Hq": wp.Hq, "Hkv": wp.Hkv, "Sq": wp.Sq, "Sk": wp.Sk,
                        "D": wp.D, "causal": wp.causal, "algorithmic_flops": flops,
                        "plan": plan_p},
            "decode": {"B": wd.B, "Hq": wd.Hq, "Hkv": wd.Hkv, "Sq": wd.Sq, "Sk": wd.Sk,
                       "D": wd.D, "causal": wd.causal, "algorithmic_bytes": dbytes,
                       "plan": plan_d},
            "device": props.name, "cus": props.multi_processor_count,
        },
        "pct_bf16_mfma_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "prefill_ms": {"avg": round(p_avg, 4), "median": round(p_ms[K // 2], 4),
                       "min": round(p_ms[0], 4)},
        "decode": {
            "value": round(gbps, 1), "unit": "GB/s",
            "ms": {"avg": round(d_avg, 4), "median": round(d_ms[K // 2], 4),
                   "min": round(d_ms[0], 4)},
            "roofline": roofline(gbps, PEAK_HBM_GBPS, "GB/s", "hbm",
                                 measured_traffic("decode")),
        },
        "paged_decode": paged_entry(PAGED, 2),
        "paged_decode_ragged": paged_entry(PAGED_RAGGED, 3),
        "d256_prefill": d256_entry(PREFILL_D256, 4),
        "d256_decode": d256_entry(DECODE_D256, 5),
        "fp8_prefill": fp8_entry(6),
        "backward": bwd_entry(7),
        "single_head": suite_entry(SINGLE, 8),
        "causal_small": suite_entry(SMALL, 9),
        "gqa_long": suite_entry(GQA, 10),
        "roofline": roofline(tflops, PEAK_BF16_TFLOPS, "TFLOP/s", "mfma",
                             measured_traffic("prefill")),
        "cpu_baseline": None,
        "conditions": None,
        "ceilings": None,
        "host": host_facts(),
    }
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        rocm = None
    power = _smi(["--showmaxpower"])
    out["conditions"] = {
        "gcn_arch": getattr(props, "gcnArchName", None), "rocm": rocm,
        "torch": torch.__version__, "hip": torch.version.hip,
        "power_cap": _pick(power, ["power"]) or None,
        "clocks_while_stepping": clocks,
    }
    if not args.no_ceilings:
        log("timed steps done; ceilings")
        from attention_fwd_02_amd import ceilings
        c = ceilings.measure_all(torch, dev)
        c["prefill_frac_of_mfma_loop"] = round(tflops / c["mfma_bf16_TFLOPs"], 4)
        c["decode_frac_of_read_loop"] = round(gbps / c["hbm_read_GBps"], 4)
        out["ceilings"] = c
    if not args.no_cpu_baseline:
        log("cpu baseline (the oracle on a sample of the prefill's rows)")
        out["cpu_baseline"] = cpu_baseline_leg(wp, qp_h, kp_h, vp_h, op, lp, args.cpu_seconds)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
