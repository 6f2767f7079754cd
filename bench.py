#!/usr/bin/env python3
"""Benchmark of the grouped-query attention forward on one MI355X.

Prints ONE JSON line.  The headline is the Mistral-7B-shaped decode step
(B16, 32 query heads, 8 KV heads, M 4096 cached keys, D 128, bf16): achieved
HBM bandwidth = algorithmic KV bytes / time.  The same run also measures the
Llama-2-70B-shaped decode (M 32768) and the causal bf16 prefill
(B4, 32/8 heads, N = M = 4096, D 128; TFLOP/s over the visible pairs), which
appear under "secondary".

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-secondary]
                    [--no-cpu-baseline] [--only WORKLOAD]

A step is one call of the path over one batch of synthetic input already
resident in HBM.  Decode inputs rotate over enough copies that the working
set exceeds the 256 MB last-level cache, so the bytes really come from HBM.

--profile-run WORKLOAD runs a few steps of one workload plus a 1 GiB torch
copy (the calibration kernel for the HBM byte counters) and prints nothing
else; it is the program that rocprofv3 wraps.  --summarize-pmc DIR turns the
counter output of such runs into the traffic summary read back here.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA, published
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 (vector and matrix), published
METRIC = "GQA decode achieved HBM GB/s (% of peak); prefill TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "decode": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "decode.hip"),
    "prefill": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "prefill.hip"),
}
KERNEL_NAMES = {"decode": "decode_kernel", "prefill": "prefill_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kind):
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES[kind],
              os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "gqa_device.h")):
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- workloads
def setup(name, torch, copies=1):
    import workloads
    from grouped_query_attention_fwd_amd import accounting
    w = workloads.by_name(name)
    q, k, v, mask, causal = workloads.make_inputs(w)
    sets = []
    for c in range(copies):
        if c == 0:
            sets.append([t.cuda() if t is not None else None for t in (q, k, v, mask)])
        else:   # distinct buffers with the same contents
            sets.append([t.cuda().clone() if t is not None else None for t in (q, k, v, mask)])
    elt = 2 if w.dtype == "bf16" else 4
    info = {"w": w, "cpu": (q, k, v, mask, causal), "sets": sets}
    if w.kind == "decode":
        info["units"] = accounting.decode_bytes(w.B, w.H, w.H_kv, w.M, w.D, elt)
    else:
        lengths = None
        if mask is not None:
            lengths = mask[:, 0, :].sum(dim=1).tolist()
        info["units"] = accounting.prefill_flops(w.B, w.H, w.N, w.M, w.D, causal, lengths)
    return info


def make_call(info, torch):
    import grouped_query_attention_fwd_amd as gqa
    w = info["w"]
    outs = []
    if w.kind == "decode":
        ws = torch.zeros(max(1, gqa.decode_workspace_size(w.B, w.H, w.H_kv, w.M, w.D)),
                         dtype=torch.uint8, device="cuda")
        for (q, k, v, m) in info["sets"]:
            outs.append(torch.empty_like(q))

        def call(i):
            q, k, v, m = info["sets"][i % len(info["sets"])]
            gqa.decode(q, k, v, m, out=outs[i % len(outs)], workspace=ws)
    else:
        for (q, k, v, m) in info["sets"]:
            outs.append(torch.empty_like(q))

        def call(i):
            q, k, v, m = info["sets"][i % len(info["sets"])]
            gqa.prefill(q, k, v, m, causal=info["cpu"][4], out=outs[i % len(outs)])
    return call


def time_workload(info, steps, warmup, torch):
    call = make_call(info, torch)
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for i in range(steps):
        starts[i].record()
        call(warmup + i)
        ends[i].record()
    t_all1.record()
    torch.cuda.synchronize()
    per = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    total_ms = t_all0.elapsed_time(t_all1)
    return {
        "ms_per_step": total_ms / steps,
        "launch_ms_avg": sum(per) / len(per),
        "launch_ms_p10": per[max(0, int(0.1 * len(per)) - 0)],
        "launch_ms_p50": per[len(per) // 2],
        "launch_ms_p90": per[min(len(per) - 1, int(0.9 * len(per)))],
    }


def traffic_for(kind, workload, launch_units):
    """HBM bytes per launch from the stored counter summary, or None when
    there is none for this workload or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    ent = data.get(workload)
    if not ent or ent.get("source_sha") != source_sha(kind):
        return None
    return ent.get("bytes_per_launch")


def result_for(info, timing):
    w = info["w"]
    kind = w.kind
    avg_s = timing["launch_ms_avg"] * 1e-3
    whole_s = timing["ms_per_step"] * 1e-3
    if kind == "decode":
        achieved = info["units"] / avg_s / 1e9
        value = info["units"] / whole_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        unit = "GB/s"
    else:
        peak = BF16_PEAK_TFLOPS if w.dtype == "bf16" else FP32_PEAK_TFLOPS
        achieved = info["units"] / avg_s / 1e12
        value = info["units"] / whole_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        unit = "TFLOP/s"
    roof["traffic"] = traffic_for(kind, w.name, info["units"])
    roof["kernel"] = KERNEL_NAMES[kind]
    return {
        "workload": w.name, "value": round(value, 3 if unit == "TFLOP/s" else 1), "unit": unit,
        "ms_per_step": round(timing["ms_per_step"], 5),
        "launch_us": {k[len("launch_ms_"):]: round(v * 1e3, 2) for k, v in timing.items()
                      if k.startswith("launch_ms_")},
        "algorithmic_units_per_launch": info["units"],
        "roofline": roof,
        "config": {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "M": w.M,
                   "D": w.D, "dtype": w.dtype, "causal": w.causal, "padded_mask": w.padded},
    }


# ------------------------------------------------------------- cpu baseline
def cpu_baseline(info, budget_s=15.0):
    """Time the fp64 oracle on a bounded sample of the same workload (whole
    batch rows, first rows first) and scale to the metric's unit."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:   # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    q, k, v, mask, causal = info["cpu"]
    w = info["w"]
    done_units, t_used, rows = 0, 0.0, 0
    for b in range(w.B):
        qb = q[b:b + 1].float().numpy().astype(np.float64)
        kb = k[b:b + 1].float().numpy().astype(np.float64)
        vb = v[b:b + 1].float().numpy().astype(np.float64)
        mb = None if mask is None else mask[b:b + 1].numpy()
        t0 = time.perf_counter()
        oracle.gqa(qb, kb, vb, mb, causal)
        t_used += time.perf_counter() - t0
        rows += 1
        done_units += info["units"] / w.B
        if t_used >= budget_s:
            break
    if w.kind == "decode":
        val, unit = done_units / t_used / 1e9, "GB/s"
    else:
        val, unit = done_units / t_used / 1e12, "TFLOP/s"
    return {"value": round(val, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{rows} of {w.B} batch rows of {w.name} ({t_used:.1f} s of fp64 numpy)"}


# ---------------------------------------------------------- counter support
def profile_run(name, steps=3):
    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)                      # calibration: reads and writes exactly 1 GiB
    torch.cuda.synchronize()
    info = setup(name, torch, copies=1)
    call = make_call(info, torch)
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()


def summarize_pmc(fetch_dir, write_dir, out_path=TRAFFIC_FILE):
    """Read two rocprofv3 --pmc counter_collection.csv outputs (FETCH_SIZE and
    WRITE_SIZE, KiB per dispatch), calibrate with the 1 GiB copy kernel and
    store bytes per launch per workload."""
    def load(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = load(d, counter)
        copy = [v for n, v in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        known_kib = (1 << 30) / 1024.0
        factor = known_kib / max(copy) if copy else 1.0
        for kind, kname in KERNEL_NAMES.items():
            vals = [v for n, v in rows if kname in n]
            if vals:
                res.setdefault(kind, {})[counter] = {"kib_per_dispatch": sum(vals) / len(vals),
                                                     "copy_factor": factor}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None)
    ap.add_argument("--profile-run", default=None)
    ap.add_argument("--summarize-pmc", nargs=2, default=None, metavar=("FETCH_DIR", "WRITE_DIR"))
    args = ap.parse_args()

    if args.summarize_pmc:
        print(json.dumps(summarize_pmc(*args.summarize_pmc), indent=1))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this grouped-query attention forward runs on a "
              "single MI355X (no collectives); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    import grouped_query_attention_fwd_amd as gqa
    gqa.load_library()   # fail loudly if the HIP library is missing

    if args.profile_run:
        profile_run(args.profile_run)
        return 0

    primary = args.only or "decode_mistral7b_m4096"
    names = [primary]
    if not args.skip_secondary and not args.only:
        names += ["decode_llama70b_m32768", "prefill_causal_n4096"]
    copies = {"decode_mistral7b_m4096": 4, "decode_llama70b_m32768": 1}
    results = {}
    primary_info = None
    for name in names:
        log(f"[bench] setting up {name}")
        info = setup(name, torch, copies=copies.get(name, 1))
        steps = args.steps if name == primary else max(10, args.steps // 2)
        log(f"[bench] timing {name}: warmup {args.warmup}, steps {steps}")
        timing = time_workload(info, steps, args.warmup, torch)
        results[name] = result_for(info, timing)
        results[name]["steps"] = steps
        log(f"[bench] {name}: {results[name]['value']} {results[name]['unit']} "
            f"(launch avg {results[name]['launch_us']['avg']} us)")
        if name == primary:
            primary_info = info
        else:
            del info
            torch.cuda.empty_cache()

    p = results[primary]
    line = {
        "metric": METRIC,
        "value": p["value"],
        "unit": p["unit"],
        "n_gpus": 1,
        "steps": p["steps"],
        "warmup": args.warmup,
        "ms_per_step": p["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if primary_info["w"].dtype == "bf16" else "f32",
        "data": "synthetic: seeded i.i.d. N(0,1) q/k/v at the workload's shapes",
        "config": p["config"],
        "roofline": p["roofline"],
        "launch_us": p["launch_us"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a CPU sample")
        line["cpu_baseline"] = cpu_baseline(primary_info)
    else:
        line["cpu_baseline"] = None
    sec = [results[n] for n in names if n != primary]
    if sec:
        line["secondary"] = [{k: r[k] for k in ("workload", "value", "unit", "ms_per_step",
                                                "launch_us", "roofline")} for r in sec]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
