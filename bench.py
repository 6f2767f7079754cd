#!/usr/bin/env python3
"""Benchmark of the grouped-query attention forward on one MI355X.

Prints ONE JSON line.  The headline is the Mistral-7B-shaped decode step
(B16, 32 query heads, 8 KV heads, M 4096 cached keys, D 128, bf16): achieved
HBM bandwidth = algorithmic KV bytes / time.  The same run also measures the
Llama-2-70B-shaped decode (M 32768), the causal bf16 prefill (B4, 32/8 heads,
N = M = 4096, D 128; TFLOP/s over the visible pairs) and the paged decode of
the Mistral-shaped batch (blocks of 16 keys scattered over a pool; mixed
lengths, and all lengths 4096; GB/s over each sequence's own keys) and two
banded prefills (a 4096-key sliding window over N = M = 16384, and a
512-query chunk after 3584 cached keys, bottom-right causal) and the
headline decode and causal prefill with fp16 inputs, which appear under
"secondary".

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
WARMUP_S = 0.3                   # minimum warm-up time per workload
METRIC = "GQA decode achieved HBM GB/s (% of peak); prefill TFLOP/s (% MFMA peak)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# calls in the per-call timing pass (event pair around each), for its
# median, p10 and p90
PER_CALL_SAMPLES = 100
KERNEL_SOURCES = {
    "decode": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "decode.hip"),
    "decode_paged": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "decode.hip"),
    "decode_wide": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "prefill.hip"),
    "prefill": os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "prefill.hip"),
}
# the kernel one call launches (the decode merges its key splits inside the
# kernel); a decode with more than WIDE_MIN_G heads per KV head runs as a
# prefill over the group's heads whose splits merge in the same launch, or
# with a second merge kernel (the library's plan)
WIDE_MIN_G = 32
KERNEL_NAMES = {"decode": "decode_kernel", "decode_paged": "decode_kernel",
                "decode_wide": "prefill_kernel", "prefill": "prefill_kernel"}
KERNEL_PATTERNS = {"decode": ("decode_kernel",), "decode_paged": ("decode_kernel",),
                   "decode_wide": ("prefill_kernel", "prefill_merge_kernel"),
                   "prefill": ("prefill_kernel",)}
DECODE_KINDS = ("decode", "decode_paged", "decode_wide")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_only(text):
    """C/HIP source with comments removed and whitespace runs collapsed, so
    that a comment edit does not count as a kernel change."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"' or c == "'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_sha(kind):
    h = hashlib.sha256()
    for p in (KERNEL_SOURCES[kind],
              os.path.join(ROOT, "grouped_query_attention_fwd_amd", "csrc", "gqa_device.h")):
        with open(p, encoding="utf-8") as f:
            h.update(code_only(f.read()).encode())
    return h.hexdigest()[:16]


# ----------------------------------------------------------------- workloads
def kind_of(name):
    """decode, decode_paged, decode_wide or prefill: which kernels a call of
    the named workload launches."""
    import workloads
    if name.startswith("decode_paged"):
        return "decode_paged"
    w = workloads.by_name(name)
    if w.kind == "decode" and w.H // w.H_kv > WIDE_MIN_G:
        return "decode_wide"
    return w.kind


def sweep_copies(name):
    """Input copies for a group-sweep decode: enough that the rotating set
    exceeds the 256 MB last-level cache (at least 640 MB); 1 otherwise."""
    import workloads
    from grouped_query_attention_fwd_amd import accounting
    if not name.startswith("decode_h64_"):
        return 1
    w = workloads.by_name(name)
    kv = accounting.decode_bytes(w.B, w.H, w.H_kv, w.M, w.D, 2)
    return max(1, -(-(640 << 20) // kv))


def setup_paged(name, torch, copies=1):
    import workloads
    from grouped_query_attention_fwd_amd import accounting
    w = workloads.paged_by_name(name)
    cpu = workloads.make_paged_inputs(w)
    sets = [[t.cuda() if c == 0 else t.cuda().clone() for t in cpu] for c in range(copies)]
    elt = 4 if w.dtype == "fp32" else 2
    info = {"w": w, "kind": "decode_paged", "cpu": cpu, "sets": sets,
            "units": accounting.paged_decode_bytes(cpu[4].tolist(), w.H_kv, w.D, elt)}
    return info


def setup(name, torch, copies=1):
    import workloads
    from grouped_query_attention_fwd_amd import accounting
    if name.startswith("decode_paged"):
        return setup_paged(name, torch, copies)
    w = workloads.by_name(name)
    q, k, v, mask, causal = workloads.make_inputs(w)
    sets = []
    for c in range(copies):
        if c == 0:
            sets.append([t.cuda() if t is not None else None for t in (q, k, v, mask)])
        else:   # distinct buffers with the same contents
            sets.append([t.cuda().clone() if t is not None else None for t in (q, k, v, mask)])
    elt = 4 if w.dtype == "fp32" else 2
    info = {"w": w, "kind": kind_of(name), "cpu": (q, k, v, mask, causal), "sets": sets}
    if w.kind == "decode":
        info["units"] = accounting.decode_bytes(w.B, w.H, w.H_kv, w.M, w.D, elt)
    elif w.band is not None:
        info["units"] = accounting.band_flops(w.B, w.H, w.N, w.M, w.D, *w.band)
    else:
        lengths = None
        if mask is not None:
            lengths = mask[:, 0, :].sum(dim=1).tolist()
        info["units"] = accounting.prefill_flops(w.B, w.H, w.N, w.M, w.D, causal, lengths)
    return info


def make_call(info, torch):
    """One prepared op per input copy; call(i) enqueues step i."""
    import grouped_query_attention_fwd_amd as gqa
    w = info["w"]
    ops = []
    if info["kind"] == "decode_paged":
        mb = info["sets"][0][3].shape[1]
        ws = torch.zeros(max(1, gqa.decode_paged_workspace_size(w.B, w.H, w.H_kv, mb,
                                                                w.block_size, w.D)),
                         dtype=torch.uint8, device="cuda")
        for (q, kp, vp, bt, kl) in info["sets"]:
            ops.append(gqa.decode_paged_op(q, kp, vp, bt, kl, workspace=ws))
    elif w.kind == "decode":
        ws = torch.zeros(max(1, gqa.decode_workspace_size(w.B, w.H, w.H_kv, w.M, w.D)),
                         dtype=torch.uint8, device="cuda")
        for (q, k, v, m) in info["sets"]:
            ops.append(gqa.decode_op(q, k, v, m, workspace=ws))
    elif w.band is not None:
        for (q, k, v, m) in info["sets"]:
            ops.append(gqa.prefill_band_op(q, k, v, m, *w.band))
    else:
        for (q, k, v, m) in info["sets"]:
            ops.append(gqa.prefill_op(q, k, v, m, causal=info["cpu"][4]))

    def call(i):
        ops[i % len(ops)]()
    return call


def time_workload(info, steps, warmup, torch):
    """Eager timing on the launch stream: HIP events around K back-to-back
    steps (throughput and the average launch duration), then around every
    step of a second pass (the per-call spread, which also carries the
    events' own packets)."""
    call = make_call(info, torch)
    # warm-up: at least `warmup` steps and at least WARMUP_S seconds of work,
    # so the GPU clocks have settled before the timed region
    t0 = time.perf_counter()
    done = 0
    while done < warmup or time.perf_counter() - t0 < WARMUP_S:
        call(done)
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    warmup = done
    # whole job: K back-to-back steps between two events
    t_all0 = torch.cuda.Event(enable_timing=True)
    t_all1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_all0.record()
    for i in range(steps):
        call(warmup + i)
    t_all1.record()
    torch.cuda.synchronize()
    total_ms = t_all0.elapsed_time(t_all1)
    # per launch: an event pair around every call of a second timed pass of
    # at least PER_CALL_SAMPLES calls (median, p10 and p90 of the spread)
    n_per = max(steps, PER_CALL_SAMPLES)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_per)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_per)]
    torch.cuda.synchronize()
    for i in range(n_per):
        starts[i].record()
        call(warmup + steps + i)
        ends[i].record()
    torch.cuda.synchronize()
    per = sorted(s_.elapsed_time(e) for s_, e in zip(starts, ends))
    res = {
        "warmup_steps_done": done,
        "per_call_samples": n_per,
        "ms_per_step": total_ms / steps,
        "launch_ms_avg": sum(per) / len(per),
        "launch_ms_p10": per[int(0.1 * (len(per) - 1))],
        "launch_ms_p50": per[len(per) // 2],
        "launch_ms_p90": per[int(0.9 * (len(per) - 1))],
    }
    # cross-check without host launch overhead: the same calls replayed
    # from a captured HIP graph
    try:
        reps = min(steps, 20)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            call(0)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=side):
                for i in range(reps):
                    call(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        best = None
        for _ in range(3):
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            best = t if best is None else min(best, t)
        res["graph_ms_per_launch"] = best
    except Exception as exc:   # noqa: BLE001 - report, keep the eager numbers
        log(f"[bench] graph replay unavailable: {exc}")
        res["graph_ms_per_launch"] = None
    return res


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
    kind = info["kind"]
    # average launch duration: two HIP events around K back-to-back launches
    # on the launching stream, divided by K (an event pair around every
    # single call, reported as launch_us, adds the events' own packets)
    avg_s = timing["ms_per_step"] * 1e-3
    whole_s = timing["ms_per_step"] * 1e-3
    if kind in DECODE_KINDS:
        achieved = info["units"] / avg_s / 1e9
        value = info["units"] / whole_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
        unit = "GB/s"
    else:
        peak = FP32_PEAK_TFLOPS if w.dtype == "fp32" else BF16_PEAK_TFLOPS  # fp16 = bf16 rate
        achieved = info["units"] / avg_s / 1e12
        value = info["units"] / whole_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4)}
        unit = "TFLOP/s"
    roof["traffic"] = traffic_for(kind, w.name, info["units"])
    roof["kernel"] = KERNEL_NAMES[kind]
    if kind == "decode_paged":
        config = {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv,
                  "max_len": w.max_len, "block_size": w.block_size, "D": w.D,
                  "dtype": w.dtype, "lengths": w.lengths,
                  "kv_len_sum": int(sum(info["cpu"][4].tolist()))}
    else:
        config = {"workload": w.name, "B": w.B, "H": w.H, "H_kv": w.H_kv, "N": w.N, "M": w.M,
                  "D": w.D, "dtype": w.dtype, "causal": w.causal, "padded_mask": w.padded}
        if w.band is not None:
            config["band"] = {"q_offset": w.q_offset, "window_left": w.window_left,
                              "window_right": w.window_right}
    roof["duration_us"] = round(timing["ms_per_step"] * 1e3, 2)
    return {
        "workload": w.name, "value": round(value, 3 if unit == "TFLOP/s" else 1), "unit": unit,
        "ms_per_step": round(timing["ms_per_step"], 5),
        "warmup_steps_done": timing["warmup_steps_done"],
        "launch_us": {**{k[len("launch_ms_"):]: round(v * 1e3, 2) for k, v in timing.items()
                         if k.startswith("launch_ms_")},
                      "calls": timing["per_call_samples"]},
        "graph_us_per_launch": (None if timing.get("graph_ms_per_launch") is None
                                else round(timing["graph_ms_per_launch"] * 1e3, 2)),
        "algorithmic_units_per_launch": info["units"],
        "roofline": roof,
        "config": config,
    }


# ------------------------------------------------------------- cpu baseline
def cpu_baseline(info, budget_s=12.0, max_rows=None):
    """Time the fp64 oracle on a bounded sample of the same workload: whole
    batch rows in order (wrapping round, so a small workload is repeated)
    until about budget_s seconds of CPU work, scaled to the metric's unit."""
    import numpy as np

    import oracle
    threads = blas_threads()
    if info["kind"] == "decode_paged":
        return cpu_baseline_paged(info, budget_s, threads)
    q, k, v, mask, causal = info["cpu"]
    w = info["w"]
    if w.kind == "prefill":
        # fewer rows per call where one call would take seconds (N x M above 2^26)
        return cpu_baseline_prefill(info, budget_s, threads,
                                    rows_per_call=64 if w.N * w.M > (1 << 26) else 256)
    done_units, t_used, rows = 0, 0.0, 0
    while t_used < budget_s and (max_rows is None or rows < max_rows):
        b = rows % w.B
        qb = q[b:b + 1].float().numpy().astype(np.float64)
        kb = k[b:b + 1].float().numpy().astype(np.float64)
        vb = v[b:b + 1].float().numpy().astype(np.float64)
        mb = None if mask is None else mask[b:b + 1].numpy()
        t0 = time.perf_counter()
        oracle.gqa(qb, kb, vb, mb, causal)
        t_used += time.perf_counter() - t0
        rows += 1
        done_units += info["units"] / w.B
    if w.kind == "decode":
        val, unit = done_units / t_used / 1e9, "GB/s"
    else:
        val, unit = done_units / t_used / 1e12, "TFLOP/s"
    return {"value": round(val, 6), "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{rows} batch rows of {w.name} ({rows / w.B:.2f} x the workload; "
                      f"{t_used:.1f} s of fp64 numpy on the host)",
            "blas": blas_info()}


def cpu_baseline_paged(info, budget_s, threads):
    """The fp64 oracle's paged decode (gather the cache through the block
    table, then attention) on whole sequences in order, wrapping round,
    until about budget_s seconds; throughput counts each sequence's own K/V
    bytes, as for the GPU.  The pool is widened to float64 once, outside
    the timed calls."""
    import numpy as np

    import oracle
    q, kp, vp, table, lens = info["cpu"]
    w = info["w"]
    elt = 4 if w.dtype == "fp32" else 2
    kp64 = kp.float().numpy().astype(np.float64)
    vp64 = vp.float().numpy().astype(np.float64)
    done, t_used, rows = 0, 0.0, 0
    while t_used < budget_s:
        b = rows % w.B
        qb = q[b:b + 1].float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.gqa_paged(qb, kp64, vp64, table[b:b + 1].numpy(), lens[b:b + 1].numpy())
        t_used += time.perf_counter() - t0
        done += 2 * int(lens[b]) * w.H_kv * w.D * elt
        rows += 1
    return {"value": round(done / t_used / 1e9, 6), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{rows} sequences of {w.name} ({rows / w.B:.2f} x the workload; "
                      f"{t_used:.1f} s of fp64 numpy on the host)",
            "blas": blas_info()}


def cpu_baseline_prefill(info, budget_s, threads, rows_per_call=256):
    """The fp64 oracle on sampled query rows of a prefill workload: for one
    batch row at a time, rows_per_call query rows spread evenly over N (a
    different offset each call), with their band or causal visibility given
    to the oracle as an explicit [1, rows, M] mask; repeated over batch rows
    until about budget_s seconds.  Throughput counts 4 D flop per visible
    (query, key) pair and head, as for the GPU."""
    import numpy as np

    import oracle
    q, k, v, mask, causal = info["cpu"]
    w = info["w"]
    band = w.band if w.band is not None else (0, -1, 0 if causal else -1)
    q_off, wl, wr = band
    step = max(1, w.N // rows_per_call)
    flops, t_used, calls = 0, 0.0, 0
    while t_used < budget_s:
        b = calls % w.B
        rows = np.arange((calls // w.B) % step, w.N, step)[:rows_per_call]
        pos = rows[:, None] + q_off
        j = np.arange(w.M)[None, :]
        vis = np.ones((len(rows), w.M), dtype=bool)
        if wl >= 0:
            vis &= j >= pos - wl
        if wr >= 0:
            vis &= j <= pos + wr
        if mask is not None:
            vis &= mask[b, rows].numpy()
        qb = q[b:b + 1, :, rows].float().numpy().astype(np.float64)
        kb = k[b:b + 1].float().numpy().astype(np.float64)
        vb = v[b:b + 1].float().numpy().astype(np.float64)
        t0 = time.perf_counter()
        oracle.gqa(qb, kb, vb, vis[None])
        t_used += time.perf_counter() - t0
        flops += 4 * w.D * w.H * int(vis.sum())
        calls += 1
    return {"value": round(flops / t_used / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{calls} calls of {rows_per_call} query rows x all {w.H} heads of one "
                      f"batch row of {w.name} ({flops / info['units']:.5f} x the workload's "
                      f"flops; {t_used:.1f} s of fp64 numpy on the host)",
            "blas": blas_info()}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:   # noqa: BLE001
        return len(os.sched_getaffinity(0))


def blas_info():
    """The thread pools numpy's fp64 products ran on (threadpoolctl), and
    the cores this process may use."""
    info = {"affinity_cores": len(os.sched_getaffinity(0))}
    try:
        from threadpoolctl import threadpool_info
        info["pools"] = [{k: d.get(k) for k in ("user_api", "internal_api", "num_threads")}
                         for d in threadpool_info()]
    except Exception:   # noqa: BLE001
        info["pools"] = None
    return info


# ------------------------------------------------------ calibration probes
def hbm_read_probe(torch, steps=30):
    """The read rate plain streaming kernels reach on this GPU, for
    comparison with the decode: over 268,435,456 bytes (four rotating copies,
    so that no call finds its data in the 256 MB last-level cache) and over
    2 GiB, the read-only kernels of libgqa_probe.so (one contiguous slab per
    workgroup, or all workgroups sweeping together; 256 to 1024 workgroups;
    8 or 16 16-byte loads in flight per thread; normal or non-temporal
    loads), and torch's sum of a bf16 tensor for reference.  Times are HIP
    events around `steps` back-to-back calls on the launching stream."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "grouped_query_attention_fwd_amd", "libgqa_probe.so"))
    lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.gqa_probe_read.restype = ctypes.c_int
    sink = torch.empty(1024 * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    res = {}
    for nbytes, copies in ((268435456, 4), (2 << 30, 1)):
        bufs = [torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda") for _ in range(copies)]
        variants = [("torch_sum", None)]
        for mode in (0, 1):
            for wgs in (256, 512, 1024):
                for unroll in (8, 16):
                    for nt in (0, 1):
                        variants.append((f"{'slabs' if mode == 0 else 'sweep'}_wg{wgs}_u{unroll}"
                                         f"{'_nt' if nt else ''}", (wgs, mode, unroll, nt)))
        rows = []
        for name, cfg in variants:
            def call(i, cfg=cfg):
                b = bufs[i % copies]
                if cfg is None:
                    b.sum(dtype=torch.float32)
                else:
                    rc = lib.gqa_probe_read(b.data_ptr(), nbytes, cfg[0], cfg[1], cfg[2], cfg[3],
                                            sink.data_ptr(), stream)
                    if rc != 0:
                        raise RuntimeError(f"read probe {name}: status {rc}")
            for i in range(8):
                call(i)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for i in range(steps):
                call(i)
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / steps
            rows.append({"variant": name, "us_per_call": round(us, 2),
                         "GB_per_s": round(nbytes / us / 1e3, 1)})
        best = max((r_ for r_ in rows if r_["variant"] != "torch_sum"), key=lambda r_: r_["GB_per_s"])
        res[str(nbytes)] = {"copies": copies, "best": best, "variants": rows}
        del bufs
        torch.cuda.empty_cache()
    return res


def decode_size_sweep(torch, steps=30, warmup=5):
    """The Mistral-7B-shaped decode (B16, 32 / 8 heads, D 128, bf16) over
    M = 1024 ... 32768 cached keys, timed like the benchmark; a least-squares
    line t = t0 + bytes / rate through the points splits each call into a
    fixed cost t0 and a streaming rate."""
    import workloads
    from grouped_query_attention_fwd_amd import accounting
    pts = []
    for M in (1024, 2048, 4096, 8192, 16384, 32768):
        w = workloads.Workload(f"decode_mistral7b_m{M}", 2, 16, 32, 8, 1, M, 128, "bf16")
        q, k, v, mask, causal = workloads.make_inputs(w)
        kv = accounting.decode_bytes(w.B, w.H, w.H_kv, w.M, w.D, 2)
        copies = max(1, -(-(640 << 20) // kv))
        sets = [[t.cuda().clone() for t in (q, k, v)] for _ in range(copies)]
        info = {"w": w, "kind": "decode", "sets": [s_ + [None] for s_ in sets], "cpu": None}
        timing = time_workload(info, steps, warmup, torch)
        us = timing["ms_per_step"] * 1e3
        pts.append({"M": M, "kv_bytes": kv, "us_per_launch": round(us, 2),
                    "GB_per_s": round(kv / us / 1e3, 1)})
        del sets, info
        torch.cuda.empty_cache()
    import numpy as np
    x = np.array([p_["kv_bytes"] for p_ in pts], dtype=np.float64)
    y = np.array([p_["us_per_launch"] for p_ in pts], dtype=np.float64)
    slope, t0 = np.polyfit(x, y, 1)
    return {"points": pts, "fit": {"fixed_us": round(float(t0), 2),
                                   "stream_GB_per_s": round(1e-3 / float(slope), 1)}}


def decode_trace(name, torch, reps=20):
    """Per-workgroup phase budget of one decode workload from the timing
    build (libgqa_trace.so, `python -m grouped_query_attention_fwd_amd._build
    --trace`): each workgroup records wall-clock ticks at its start, when its
    waves have finished their keys, after its arrival ticket and at its end,
    plus its XCD and CU.  Per call: how far apart the workgroups start, when
    the key phase ends (median / slowest workgroup, per XCD), what the split
    merge adds, and the whole span; medians over `reps` calls."""
    import ctypes

    import numpy as np

    import grouped_query_attention_fwd_amd as gqa
    path = os.path.join(ROOT, "grouped_query_attention_fwd_amd", "libgqa_trace.so")
    lib = gqa.load_library(path)
    lib.gqa_debug_decode_trace.argtypes = [ctypes.c_void_p]
    lib.gqa_debug_wall_clock_khz.restype = ctypes.c_int
    khz = lib.gqa_debug_wall_clock_khz()
    if khz <= 0:
        raise RuntimeError("wall clock rate unavailable")
    records = 8192
    buf = torch.zeros(records * 8, dtype=torch.int64, device="cuda")
    lib.gqa_debug_decode_trace(ctypes.c_void_p(buf.data_ptr()))
    copies = 4 if name.startswith(("decode_mistral", "decode_paged")) else 1
    info = setup(name, torch, copies=copies)
    call = make_call(info, torch)
    for i in range(10):
        call(i)
    torch.cuda.synchronize()
    per_call = []
    for r in range(reps):
        buf.zero_()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        call(r)
        e1.record()
        torch.cuda.synchronize()
        rec = buf.view(records, 8).cpu().numpy()
        rec = rec[rec[:, 0] != 0]
        us = lambda t: t * 1e3 / khz   # noqa: E731 - ticks to microseconds
        t0 = rec[:, 0].min()
        start = us(rec[:, 0] - t0)
        keys = us(rec[:, 1] - t0)
        end = us(rec[:, 3] - t0)
        xcd = (rec[:, 4] >> 16) & 0xF
        merged = rec[:, 7] == 1
        split = rec[:, 2] != 0
        per_xcd = [float(np.median(keys[xcd == x])) for x in range(8) if (xcd == x).any()]
        per_call.append({
            "event_us": e0.elapsed_time(e1) * 1e3,
            "workgroups": int(len(rec)),
            "start_spread_us": float(start.max()),
            "plan_median_us": float(np.median(us(rec[:, 5] - rec[:, 0]))),
            "keys_done_median_us": float(np.median(keys)),
            "keys_done_max_us": float(keys.max()),
            "key_phase_median_us": float(np.median(keys - start)),
            "xcd_keys_done_median_min_us": min(per_xcd),
            "xcd_keys_done_median_max_us": max(per_xcd),
            "ticket_after_keys_median_us": (float(np.median(us(rec[split, 2] - rec[split, 1])))
                                            if split.any() else 0.0),
            "merge_us_median": (float(np.median(us(rec[merged, 3] - rec[merged, 2])))
                                if merged.any() else 0.0),
            "span_us": float(end.max()),
            "last_end_minus_last_keys_us": float(end.max() - keys.max()),
        })
    lib.gqa_debug_decode_trace(None)
    keys_ = per_call[0].keys()
    summary = {k: round(float(np.median([c[k] for c in per_call])), 2) for k in keys_}
    return {"workload": name, "wall_clock_khz": khz, "calls": reps,
            "median_over_calls": summary}


# ---------------------------------------------------------- counter support
PROBE_CAL_BYTES = 256 << 20


def profile_run(name, steps=3):
    import ctypes

    import torch
    n = (1 << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    y.copy_(x)                      # calibration: reads and writes exactly 1 GiB
    torch.cuda.synchronize()
    del x, y
    # second calibration: the read probe (read_sweep) reads exactly 256 MiB
    lib = ctypes.CDLL(os.path.join(ROOT, "grouped_query_attention_fwd_amd", "libgqa_probe.so"))
    lib.gqa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    buf = torch.ones(PROBE_CAL_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.empty(256 * 256, dtype=torch.int32, device="cuda")
    rc = lib.gqa_probe_read(buf.data_ptr(), PROBE_CAL_BYTES, 256, 1, 8, 1, sink.data_ptr(),
                            torch.cuda.current_stream().cuda_stream)
    if rc != 0:
        raise RuntimeError(f"read probe status {rc}")
    torch.cuda.synchronize()
    del buf, sink
    info = setup(name, torch, copies=1)
    call = make_call(info, torch)
    for i in range(steps):
        call(i)
    torch.cuda.synchronize()


def summarize_pmc(workload, fetch_dir, write_dir):
    """Traffic per call from two rocprofv3 --pmc runs of --profile-run
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch).  Each counter is scaled
    by what it reads for the 1 GiB copy in the same run (factor = true bytes
    / counted bytes), then summed over the kernels of one call."""
    kind = kind_of(workload)

    def load(d, counter):
        rows = []
        for p in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(p) as f:
                for r in csv.DictReader(f):
                    if r.get("Counter_Name") == counter:
                        rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
        return rows

    out = {"workload": workload, "kernel": KERNEL_NAMES[kind], "source_sha": source_sha(kind)}
    total = 0.0
    for counter, d, copy_bytes in (("FETCH_SIZE", fetch_dir, 1 << 30), ("WRITE_SIZE", write_dir, 1 << 30)):
        rows = load(d, counter)
        copy = [val for n, val in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        factor = (copy_bytes / 1024.0) / max(copy) if copy and max(copy) > 0 else None
        if counter == "FETCH_SIZE":
            # cross-check: the read probe's 256 MiB, counted by the same counter
            probe = [val for n, val in rows if "read_sweep" in n]
            out["probe_read_check"] = {
                "probe_kib_counted": max(probe) if probe else None,
                "probe_factor": (round((PROBE_CAL_BYTES / 1024.0) / max(probe), 4)
                                 if probe and max(probe) > 0 else None)}
        per_call = 0.0
        for pat in KERNEL_PATTERNS[kind]:
            vals = [val for n, val in rows if (pat + "<") in n or n.endswith(pat)]
            if vals:
                per_call += sum(vals) / len(vals)
        out[counter] = {"kib_per_call": round(per_call, 1),
                        "copy_kib_counted": max(copy) if copy else None,
                        "copy_factor": None if factor is None else round(factor, 4)}
        total += per_call * 1024.0 * (factor if factor else 1.0)
    out["bytes_per_launch"] = int(total)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default=None)
    ap.add_argument("--profile-run", default=None)
    ap.add_argument("--summarize-pmc", nargs=3, default=None,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR"))
    ap.add_argument("--hbm-read-probe", action="store_true",
                    help="time the HBM read probe kernels and a torch reduction over 268 MB and 2 GiB")
    ap.add_argument("--decode-size-sweep", action="store_true",
                    help="time the Mistral-7B-shaped decode over M = 1024 ... 32768")
    ap.add_argument("--decode-trace", default=None, metavar="WORKLOAD",
                    help="per-workgroup phase budget of a decode workload (timing build)")
    args = ap.parse_args()

    if args.summarize_pmc:
        ent = summarize_pmc(*args.summarize_pmc)
        try:
            with open(TRAFFIC_FILE) as f:
                data = json.load(f)
        except (OSError, ValueError):
            data = {}
        data[ent["workload"]] = ent
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
        print(json.dumps(ent, indent=1))
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
    if args.decode_trace:
        print(json.dumps({"decode_trace": decode_trace(args.decode_trace, torch)}), flush=True)
        return 0
    gqa.load_library()   # fail loudly if the HIP library is missing

    if args.profile_run:
        profile_run(args.profile_run)
        return 0
    if args.hbm_read_probe:
        print(json.dumps({"hbm_read_probe": hbm_read_probe(torch)}), flush=True)
        return 0
    if args.decode_size_sweep:
        print(json.dumps({"decode_size_sweep": decode_size_sweep(torch)}), flush=True)
        return 0

    primary = args.only or "decode_mistral7b_m4096"
    names = [primary]
    if not args.skip_secondary and not args.only:
        names += ["decode_llama70b_m32768", "prefill_causal_n4096",
                  "decode_paged_mistral7b_varlen", "decode_paged_mistral7b_full",
                  "prefill_window4096_n16384", "prefill_chunk512_m4096",
                  "decode_mistral7b_m4096_fp16", "prefill_causal_n4096_fp16",
                  "prefill_causal_n4096_d256"]
    copies = {"decode_mistral7b_m4096_fp16": 4, "decode_mistral7b_m4096": 4, "decode_llama70b_m32768": 1,
              "decode_paged_mistral7b_varlen": 4, "decode_paged_mistral7b_full": 4}
    results = {}
    primary_info = None
    # the oracle timed beside the prefill half of the metric, the long
    # decode, the paged decode and the sliding window as well
    cpu_side = ({"prefill_causal_n4096", "decode_llama70b_m32768",
                 "decode_paged_mistral7b_varlen", "prefill_window4096_n16384"}
                if not args.no_cpu_baseline else set())
    for name in names:
        log(f"[bench] setting up {name}")
        info = setup(name, torch, copies=copies.get(name, sweep_copies(name)))
        steps = args.steps if name == primary else max(10, args.steps // 2)
        log(f"[bench] timing {name}: warmup {args.warmup}, steps {steps}")
        timing = time_workload(info, steps, args.warmup, torch)
        results[name] = result_for(info, timing)
        results[name]["steps"] = steps
        log(f"[bench] {name}: {results[name]['value']} {results[name]['unit']} "
            f"({results[name]['roofline']['duration_us']} us per launch; with an event pair "
            f"around each call {results[name]['launch_us']['avg']} us)")
        if name == primary:
            primary_info = info
        else:
            if name in cpu_side:
                log(f"[bench] timing the fp64 oracle on a CPU sample of {name}")
                results[name]["cpu_baseline"] = cpu_baseline(info, budget_s=10.0)
            del info
            torch.cuda.empty_cache()

    # group-size sweep: the same decode step with 64 query heads and
    # g = 1 ... 64; enough rotating copies that each point streams from HBM
    sweep = []
    if not args.skip_secondary and not args.only:
        import workloads
        from grouped_query_attention_fwd_amd import accounting
        for w in workloads.GROUP_SWEEP:
            kv = accounting.decode_bytes(w.B, w.H, w.H_kv, w.M, w.D, 2)
            copies_g = sweep_copies(w.name)
            log(f"[bench] group sweep {w.name} ({copies_g} copies)")
            info = setup(w.name, torch, copies=copies_g)
            timing = time_workload(info, max(10, args.steps // 2), args.warmup, torch)
            r = result_for(info, timing)
            sweep.append({"g": w.H // w.H_kv, "H_kv": w.H_kv, "value": r["value"],
                          "unit": r["unit"], "us_per_launch": r["roofline"]["duration_us"],
                          "frac": r["roofline"]["frac"], "kv_bytes": kv,
                          "kernel": r["roofline"]["kernel"],
                          "traffic": r["roofline"]["traffic"]})
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
        "dtype": {"bf16": "bf16", "fp16": "f16", "fp32": "f32"}[primary_info["w"].dtype],
        "data": "synthetic: seeded i.i.d. N(0,1) q/k/v at the workload's shapes",
        "config": p["config"],
        "roofline": p["roofline"],
        "launch_us": p["launch_us"],
        "graph_us_per_launch": p["graph_us_per_launch"],
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a CPU sample")
        line["cpu_baseline"] = cpu_baseline(primary_info)
    else:
        line["cpu_baseline"] = None
    sec = [results[n] for n in names if n != primary]
    if sec:
        line["secondary"] = [{k: r[k] for k in ("workload", "value", "unit", "ms_per_step",
                                                "launch_us", "graph_us_per_launch", "roofline",
                                                "cpu_baseline") if k in r}
                             for r in sec]
    if sweep:
        line["group_sweep"] = {"workload": "decode B16 H64 M4096 D128 bf16, H_kv = 64 / g",
                               "points": sweep}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
