"""Measure the HBM bytes each bench.py call moves, with rocprofv3 counters.

    python3 -m attention_fwd_02_amd.profile_counters [--out DIR] [--keys k1,k2]

For every call (`bench.py --profile-kernel KEY`, 2 warm-up + 5 timed calls)
two rocprofv3 passes run, one counter each: FETCH_SIZE, then WRITE_SIZE
(KiB per dispatch).  A plain 1 GiB device-to-device copy calibrates them: the
ratio of its known bytes to what each counter reads scales the attention
kernels' readings.  The per-dispatch mean of every attention kernel of the
call (names holding `fa_`, or `fa_bwd` for the backward) is summed.  Writes
`profiles/counters.json` with the hash of the kernels' device code the
figures were taken with (`libfa.so.device-sha256`, written by the build);
bench.py reports them as `traffic` only while that hash matches.
`--from-csv` assembles the file from the CSVs of an earlier run.

This process never touches the GPU: each pass is a child rocprofv3 process
with its own time limit.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import shutil
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEVICE_SHA = os.path.join(ROOT, "attention_fwd_02_amd", "libfa.so.device-sha256")
COPY_BYTES = 1 << 30

# key -> (workload, kernel-name filter)
CALLS = {
    "prefill": ("causal_b4_h16_s4096_d128", "fa_"),
    "decode": ("decode_b32_hq32_hkv8_sk8192_d128", "fa_"),
    "paged": ("paged_decode_b32_hq32_hkv8_len8192_ps16_d128", "fa_"),
    "paged_ragged": ("paged_decode_b32_hq32_hkv8_ragged16384_ps16_d128", "fa_"),
    "prefill_d256": ("causal_b2_h16_s4096_d256", "fa_"),
    "decode_d256": ("decode_b32_hq32_hkv8_sk8192_d256", "fa_"),
    "prefill_fp8": ("causal_b4_h16_s4096_d128_fp8", "fa_"),
    "bwd": ("causal_b4_h16_s4096_d128 backward", "fa_bwd"),
    "single_head": ("single_head_s128_d64", "fa_"),
    "causal_small": ("causal_b2_h8_s1024_d64", "fa_"),
    "gqa_long": ("gqa_b1_hq32_hkv8_s16384_d128", "fa_"),
}


def command(key, counter, out_dir):
    return ["timeout", "-s", "KILL", "120", "rocprofv3", "--pmc", counter, "--output-format",
            "csv", "-d", os.path.join(out_dir, f"pmc_{key}_{counter}"), "-o", "pmc", "--",
            sys.executable, os.path.join(ROOT, "bench.py"), "--profile-kernel", key,
            "--warmup", "2", "--steps", "5"]


def per_kernel_means(out_dir, key, counter, name_filter):
    files = glob.glob(os.path.join(out_dir, f"pmc_{key}_{counter}", "**",
                                   "*counter_collection.csv"), recursive=True)
    if not files:
        raise RuntimeError(f"no counter CSV for {key} {counter}")
    vals = {}
    with open(files[0]) as f:
        for r in csv.DictReader(f):
            if name_filter in r["Kernel_Name"] and r.get("Counter_Name", counter) == counter:
                vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    if not vals:
        raise RuntimeError(f"no {name_filter!r} kernel in the {key} {counter} CSV")
    return {k: sum(v) / len(v) for k, v in vals.items()}


def short(name):
    name = name.replace("void ", "").replace("fa::kern::", "")
    return name[:name.index("(")] if "(" in name else name


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=os.path.join(ROOT, "gpurun_out", "pmc"))
    ap.add_argument("--keys", default=",".join(CALLS))
    ap.add_argument("--json", default=os.path.join(ROOT, "profiles", "counters.json"))
    ap.add_argument("--from-csv", action="store_true",
                    help="skip the rocprofv3 passes; read the CSVs already under --out")
    args = ap.parse_args()
    keys = [k for k in args.keys.split(",") if k]
    os.makedirs(args.out, exist_ok=True)
    for key in [] if args.from_csv else ["copy", *keys]:
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            d = os.path.join(args.out, f"pmc_{key}_{counter}")
            shutil.rmtree(d, ignore_errors=True)
            print(f"counter pass: {key} {counter}", flush=True)
            r = subprocess.run(command(key, counter, args.out), cwd=ROOT)
            if r.returncode != 0:
                print(f"rocprofv3 pass {key} {counter} ended with {r.returncode}", flush=True)
                return r.returncode
    cf = sum(per_kernel_means(args.out, "copy", "FETCH_SIZE", "copyBuffer").values())
    cw = sum(per_kernel_means(args.out, "copy", "WRITE_SIZE", "copyBuffer").values())
    fs, ws = COPY_BYTES / 1024 / cf, COPY_BYTES / 1024 / cw
    with open(DEVICE_SHA) as f:
        sha = f.read().strip()
    try:
        with open(args.json) as f:
            out = json.load(f)
    except (OSError, ValueError):
        out = {}
    out["calibration"] = {"copy_bytes": COPY_BYTES, "FETCH_SIZE_KiB": cf, "WRITE_SIZE_KiB": cw,
                          "fetch_scale": fs, "write_scale": ws}
    cmds = {"copy": " ".join(command("copy", "FETCH_SIZE", "gpurun_out/pmc")[4:]).replace(
        sys.executable, "python3").replace(ROOT + "/", "") + " (then WRITE_SIZE)"}
    for key in keys:
        wl, filt = CALLS[key]
        fm = per_kernel_means(args.out, key, "FETCH_SIZE", filt)
        wm = per_kernel_means(args.out, key, "WRITE_SIZE", filt)
        a, b = sum(fm.values()), sum(wm.values())
        out[key] = {"kernel": " + ".join(short(n) for n in fm), "workload": wl,
                    "FETCH_SIZE_KiB": a, "WRITE_SIZE_KiB": b,
                    "hbm_bytes_per_launch": int(round((a * fs + b * ws) * 1024)),
                    "device_code_sha256": sha}
        cmds[key] = " ".join(command(key, "FETCH_SIZE", "gpurun_out/pmc")[4:]).replace(
            sys.executable, "python3").replace(ROOT + "/", "") + " (then WRITE_SIZE)"
        print(key, json.dumps(out[key]), flush=True)
    out.setdefault("commands", {}).update(cmds)
    out["commands"]["all"] = "python3 -m attention_fwd_02_amd.profile_counters"
    with open(args.json, "w") as f:
        json.dump(out, f, indent=1)
    print(f"wrote {args.json}", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
