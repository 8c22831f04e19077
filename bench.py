#!/usr/bin/env python3
"""Benchmark of the flexible-mask attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload packed_docs]
                    [--no-cpu-baseline] [--split-tiles S]

A step is one ffa_fwd call (main kernel, plus the split-K combine when the plan
splits) over the whole workload, inputs resident in HBM.  The metric counts
only unmasked FLOPs: 4 * D * Hq * (visible (q, k) pairs per head).  Timing uses
HIP events recorded on the stream the kernels are launched on.

Prints one JSON line.  `roofline` refers to the dominant kernel (ffa_fwd_main,
bound by bf16 MFMA at D >= 64, by the per-score VALU work below); `cpu_baseline`
times the fp64 CPU oracle on a bounded sample of the same workload; `backward`
times ffa_bwd (dq, dk, dv from the forward's out and lse) on the same workload,
outside the forward's step; `also` times the forward of further workloads
(default: the heterogeneous-mask mix, the other configuration the >= 50% target
names, the rectangular causal GQA case and the long-context case) the same way,
outside the step; `combine` times the split-K combine kernel alone on the
long-context case planned with forced chunks of 512 key tiles, against HBM.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
METRIC = "masked-attn fwd TFLOPS (unmasked FLOPs) and % of MI355X bf16 MFMA peak"
WORKLOADS = sorted(list(__import__("workloads").CONFIG_NAMES.values()) + list(__import__("workloads").EXTRA_WORKLOADS))


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-warmup-seconds", type=float, default=0.3,
                    help="keep warming up (untimed) until this much GPU time has passed: the clocks ramp "
                         "over the first tens of milliseconds of sustained load")
    ap.add_argument("--workload", default="packed_docs", choices=WORKLOADS)
    ap.add_argument("--split-tiles", type=int, default=0, help="planner split control (0 auto, <0 never)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward leg")
    ap.add_argument("--also", default="hetero_mask_mix,rect_causal_gqa,long_context",
                    help="comma-separated workloads whose forward is also timed, reported under `also` "
                         "(the bench line's value stays the --workload one); '' for none")
    ap.add_argument("--combine", default="long_context:512",
                    help="workload:split_tiles of the split-K combine leg (forced split, the combine kernel "
                         "timed alone over the partials); '' for none")
    ap.add_argument("--softcap", type=float, default=0.0, help="soft-capping of the scores (0: off)")
    ap.add_argument("--total", action="store_true", help="also time the total-attention pass")
    ap.add_argument("--fp16", action="store_true", help="float16 inputs and outputs instead of bfloat16")
    ap.add_argument("--sinks", type=int, default=0, help="sink logits per head (layout sh; 0: none)")
    ap.add_argument("--rounded-norm", action="store_true",
                    help="forward legs with FFA_EXTRAS_ROUNDED_NORM (out divided by the sum of the rounded weights)")
    ap.add_argument("--backward-only", action="store_true",
                    help="time only the backward (for profiling its kernels)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="time budget of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (for HBM counter calibration)")
    ap.add_argument("--summarize-profiles", metavar="DIR", default=None,
                    help="only write profiles/traffic.json and profiles/clock.json from the rocprofv3 "
                         "counter runs under DIR (no GPU needed)")
    return ap.parse_args()


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CLOCK_FILE = os.path.join(ROOT, "profiles", "clock.json")
HBM_PEAK_TBS = 8.0  # MI355X HBM3E


def alu_peak_tflops(head_dim: int) -> float:
    """Peak of the metric's FLOP count when the per-score VALU work bounds the kernel.

    Per wave64 instruction group of 64 scores the softmax needs about 18 VALU issue
    cycles on a SIMD (v_exp_f32 8, the exponent-argument FMA 4, the row-sum add 4, half
    a bf16 pack 2; measured with probe kernels), so a SIMD turns at most 64 / 18 scores
    into probabilities per cycle: 1024 SIMDs (256 CUs x 4) x 2.4 GHz x 64 / 18 scores/s,
    each worth 4 * D FLOPs of the metric.  Below D = 64 this is lower than the bf16 MFMA
    peak (the MFMA work per score shrinks with D, the softmax work does not)."""
    return 1024 * 2.4e9 * (64.0 / 18.0) * 4.0 * head_dim / 1e12


def roofline_bound(head_dim: int):
    """(bound, peak TFLOP/s) of the forward main kernel at this head dim."""
    alu = alu_peak_tflops(head_dim)
    return ("alu", round(alu, 1)) if alu < PEAK_BF16_TFLOPS else ("mfma", PEAK_BF16_TFLOPS)


def measured_clock(workload: str):
    """Shader clock under the main kernel, derived from a GRBM_GUI_ACTIVE counter pass
    (profiles/clock.json), or None when missing or taken on another kernel source."""
    try:
        with open(CLOCK_FILE) as f:
            c = json.load(f)
    except (OSError, ValueError):
        return None
    if c.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = c.get("workloads", {}).get(workload)
    return None if w is None else {"mhz": w.get("mhz"), "source": "GRBM_GUI_ACTIVE / 8 XCDs / kernel duration "
                                                              "(rocprofv3 counter pass, profiles/clock.json)"}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


KERNEL_SOURCES = [os.path.join(ROOT, "flexible_mask_flash_amd", "csrc", f)
                  for f in ("ffa_fwd.hip", "ffa_device.h", "ffa_internal.h", "ffa_plan.cpp")]


def kernel_source_hash(read=None) -> str:
    """Hash of the forward kernel's sources with comments and blank lines dropped, so that
    an edit of comments alone keeps the counters taken on the code (the sources hold no
    `//` inside string literals and no block comments)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        if read is None:
            with open(f, "r") as fh:
                text = fh.read()
        else:
            text = read(f)
        for line in text.split("\n"):
            code = re.sub(r"//.*$", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch of the main kernel from profiles/traffic.json (FETCH_SIZE + WRITE_SIZE,
    scaled by a plain copy's reading), or None when missing or taken on another kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else w.get("hbm_bytes_per_launch")


TRAFFIC_WORKLOADS = ("packed_docs", "hetero_mask_mix", "rect_causal_gqa", "long_context")
CLOCK_WORKLOADS = ("packed_docs", "hetero_mask_mix", "long_context")
CLOCK_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                  "SQ_INSTS_LDS SQ_WAIT_INST_ANY SQ_INSTS_SALU GRBM_GUI_ACTIVE")


def plan_balance(plan, slots: int) -> dict:
    """Load balance of the forward worklist: each item's cost in key tiles (+3 for its
    prologue and epilogue, +1 for an item with no runs), dispatched longest-first in
    list order onto `slots` resident workgroups; the makespan against the mean."""
    import heapq

    meta = plan.meta_host()
    n = int(plan.info["num_items"])
    recs = meta[16:16 + 16 * n].reshape(n, 16)  # item records after the 16-word header
    costs = [int(t) + (3 if int(r) > 0 else 1) for t, r in zip(recs[:, 6], recs[:, 4])]
    heap = [0] * slots
    for c in costs:
        heapq.heapreplace(heap, heap[0] + c)
    mean = sum(costs) / slots
    return {"slots": slots, "mean_tiles_per_slot": round(mean, 2), "makespan_tiles": max(heap),
            "makespan_over_mean": round(max(heap) / mean, 3) if mean else None}


def algorithmic_bytes(p) -> int:
    """Bytes the forward must move at least: q, k, v read and out written (bf16), lse written (fp32)."""
    d = p.head_dim
    return 2 * d * (2 * p.total_q * p.heads_q + 2 * p.total_k * p.heads_kv) + 4 * p.total_q * p.heads_q


def summarize_profiles(d: str):
    """Write profiles/traffic.json and profiles/clock.json from rocprofv3 counter runs in d:
    d/FETCH_SIZE_<w>, d/WRITE_SIZE_<w> (one counter per run, this file's --workload <w>),
    d/FETCH_SIZE_copy, d/WRITE_SIZE_copy (--copy-calibration) and d/sq_<w> (the counters
    of CLOCK_COUNTERS in one run), each holding rocprofv3's run_counter_collection.csv.
    The last dispatch of the kernel in each run is used; both files carry the hash of
    the kernel sources they were measured on, and bench lines use them only while the
    sources are unchanged."""
    import csv

    def last(tag, counter, kernel):
        with open(os.path.join(d, tag, "run_counter_collection.csv")) as f:
            r = [x for x in csv.DictReader(f) if kernel in x["Kernel_Name"] and x["Counter_Name"] == counter]
        if not r:
            raise SystemExit(f"{tag}: no {counter} for {kernel}")
        return r[-1]

    import workloads as W

    kib_per_gib = (1 << 30) / 1024
    fcopy = float(last("FETCH_SIZE_copy", "FETCH_SIZE", "copyBuffer")["Counter_Value"])
    wcopy = float(last("WRITE_SIZE_copy", "WRITE_SIZE", "copyBuffer")["Counter_Value"])
    fs, ws = round(kib_per_gib / fcopy, 1), round(kib_per_gib / wcopy, 1)
    tr = {"kernel": "ffa_fwd_main", "kernel_source_hash": kernel_source_hash(),
          "method": ("rocprofv3 --pmc FETCH_SIZE and --pmc WRITE_SIZE in separate runs (KiB per dispatch, last "
                     f"dispatch); scaled by a 1 GiB device copy (__amd_rocclr_copyBuffer): FETCH_SIZE read {fcopy} "
                     f"KiB -> x{fs}, WRITE_SIZE read {wcopy} KiB -> x{ws}"),
          "fetch_scale": fs, "write_scale": ws, "workloads": {}}
    for w in TRAFFIC_WORKLOADS:
        f = float(last(f"FETCH_SIZE_{w}", "FETCH_SIZE", "ffa_fwd_main")["Counter_Value"])
        wr = float(last(f"WRITE_SIZE_{w}", "WRITE_SIZE", "ffa_fwd_main")["Counter_Value"])
        p = W.workload(w)
        ab = algorithmic_bytes(p)
        outlse = 2 * p.head_dim * p.total_q * p.heads_q + 4 * p.total_q * p.heads_q
        tr["workloads"][w] = {"fetch_kib": f, "write_kib": wr,
                              "hbm_bytes_per_launch": int(round((f * fs + wr * ws) * 1024)),
                              "algorithmic_bytes": ab, "write_bytes": int(wr * ws * 1024), "out_lse_bytes": outlse}
        print(f"{w:16s} fetch {f * fs / 1024:9.1f} MiB write {wr * ws / 1024:9.1f} MiB  hbm/algo "
              f"{(f * fs + wr * ws) * 1024 / ab:5.2f}  write/(out+lse) {wr * ws * 1024 / outlse:5.3f}")
    ck = {"kernel": "ffa_fwd_main", "kernel_source_hash": kernel_source_hash(),
          "method": (f"rocprofv3 --pmc {CLOCK_COUNTERS} (one run per workload, last dispatch); "
                     "clock = GRBM_GUI_ACTIVE / 8 XCDs / (End - Start timestamp)"), "workloads": {}}
    for w in CLOCK_WORKLOADS:
        c = {}
        with open(os.path.join(d, f"sq_{w}", "run_counter_collection.csv")) as f:
            for x in csv.DictReader(f):
                if "ffa_fwd_main" in x["Kernel_Name"]:
                    c[x["Counter_Name"]] = (float(x["Counter_Value"]), int(x["Start_Timestamp"]),
                                            int(x["End_Timestamp"]))
        dur = (c["GRBM_GUI_ACTIVE"][2] - c["GRBM_GUI_ACTIVE"][1]) * 1e-9
        grbm = c["GRBM_GUI_ACTIVE"][0]
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"][0]
        valu, mfma, lds, salu = (c[k][0] for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_SALU"))
        ck["workloads"][w] = {"mhz": round(grbm / 8 / dur / 1e6, 1), "duration_us": round(dur * 1e6, 1),
                              "grbm_gui_active": grbm, "sq_busy_cycles": c["SQ_BUSY_CYCLES"][0],
                              "mfma_busy_cycles": busy,
                              # the SIMD cycles available: 1024 SIMDs x GRBM cycles per XCD
                              "mfma_busy_frac_of_simd_cycles": round(busy / (1024 * grbm / 8), 4),
                              "valu_per_mfma": round(valu / mfma, 3), "lds_per_mfma": round(lds / mfma, 3),
                              "salu_per_mfma": round(salu / mfma, 3)}
        print(w, ck["workloads"][w])
    for path, obj in ((TRAFFIC_FILE, tr), (CLOCK_FILE, ck)):
        with open(path, "w") as f:
            json.dump(obj, f, indent=1)
            f.write("\n")


def copy_calibration():
    """A plain 1 GiB device copy: the reference kernel for scaling FETCH_SIZE / WRITE_SIZE
    (profile this command), and the HBM rate a streaming kernel reaches on this part
    (timed with HIP events over 20 copies after the first three)."""
    import torch

    n = 1 << 30  # bytes
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copy_ms": round(ms, 4),
                      "copy_read_plus_write_TB_s": round(2 * n / (ms * 1e-3) / 1e12, 3)}), flush=True)


def cpu_baseline(p, q, k, v, budget_s: float):
    """Time the fp64 oracle on whole 256-row blocks of the workload until the budget is spent."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    rng = np.random.default_rng(1234)
    nblk = (p.total_q + 255) // 256
    order = rng.permutation(nblk)
    # q, k, v as float64 once (conversion is not part of the timed oracle work)
    qd, kd, vd = q.double().numpy(), k.double().numpy(), v.double().numpy()
    done_rows, pairs, t_used = 0, 0, 0.0
    for bi in order:
        rows = np.arange(bi * 256, min(p.total_q, bi * 256 + 256))
        t0 = time.perf_counter()
        oracle.attend(qd, kd, vd, p.q_ranges, p.k_ranges, p.mask_types, rows=rows)
        t_used += time.perf_counter() - t0
        m = oracle.mask_rows(rows, p.q_ranges, p.k_ranges, p.mask_types, p.total_k)
        pairs += int(m.sum())
        done_rows += rows.size
        if t_used >= budget_s:
            break
    flops = 4.0 * p.head_dim * p.heads_q * pairs
    return {
        "value": flops / t_used / 1e12,
        "unit": "TFLOPS",
        "cores": int(cores),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{done_rows} of {p.total_q} query rows ({done_rows // 256} seeded random 256-row blocks), "
                  f"all heads, fp64 numpy BLAS; {t_used:.1f} s",
        "seconds": t_used,
    }


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)

    import torch

    import flexible_mask_flash_amd as ffa
    import workloads as W

    ffa.load_library()
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    p = W.workload(args.workload)
    q, k, v = W.make_qkv(p, dtype=torch.float16 if args.fp16 else None)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)

    t0 = time.perf_counter()
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, split_tiles=args.split_tiles)
    plan_ms = (time.perf_counter() - t0) * 1e3
    plan.device_meta(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((p.total_q, p.heads_q), dtype=torch.float32, device=dev)
    strides = {"q": (0, qd.stride(0), qd.stride(1)), "k": (0, kd.stride(0), kd.stride(1)),
               "v": (0, vd.stride(0), vd.stride(1)), "out": (0, out.stride(0), out.stride(1)),
               "lse": (0, lse.stride(0), lse.stride(1))}
    scale = 1.0 / math.sqrt(p.head_dim)
    sink = None
    if args.sinks > 0:
        g = torch.Generator().manual_seed(17)
        sink = torch.randn((args.sinks, p.heads_q), generator=g, dtype=torch.float32).to(dev)
    extras = ffa.make_extras(sink, "sh", args.softcap, total_q=p.total_q, heads_q=p.heads_q, dtype=qd.dtype,
                             rounded_norm=args.rounded_norm)

    def step():
        ffa.run_fwd(plan, qd, kd, vd, out, lse, strides, 1, scale, extras)

    if args.backward_only:
        step()
        torch.cuda.synchronize()
        print(json.dumps({"backward": backward_leg(args, p, qd, kd, vd, out, lse, strides, scale, sink)}),
              flush=True)
        return

    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < args.min_warmup_seconds:
        step()
        warm += 1
        if warm % 5 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the stream ffa_fwd launches on
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]
    total_ms = ev[0].elapsed_time(ev[-1])
    ms_step = total_ms / args.steps
    flops = 4.0 * p.head_dim * p.heads_q * plan.info["visible_pairs"]
    tflops = flops / (ms_step * 1e-3) / 1e12
    med = float(np.median(per))

    props = torch.cuda.get_device_properties(dev)
    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm,
        "warmup_requested": args.warmup,
        "warmup_note": f"untimed warm-up runs until both {args.warmup} steps and "
                       f"{args.min_warmup_seconds} s have passed (the clock ramps under sustained load)",
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if args.fp16 else "bf16",
        "data": "synthetic",
        "config": {
            "workload": p.name,
            **{k_: v_ for k_, v_ in p.describe().items() if k_ != "workload"},
            "visible_pairs_per_head": int(plan.info["visible_pairs"]),
            "flops_per_step": flops,
            "plan": {k_: int(v_) for k_, v_ in plan.info.items()},
            "plan_ms": round(plan_ms, 2),
            "plan_balance": plan_balance(plan, 2 * torch.cuda.get_device_properties(dev).multi_processor_count),
            "split_tiles": args.split_tiles,
            "softcap": args.softcap,
            "sinks": args.sinks,
            "rounded_norm": args.rounded_norm,
        },
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "ms_median": round(med, 4),
        "ms_min": round(min(per), 4),
        "ms_max": round(max(per), 4),
        "wall_s_timed": round(wall, 3),
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "gcn_arch": getattr(props, "gcnArchName", ""), "hip": getattr(torch.version, "hip", None)},
        "roofline": {
            "bound": roofline_bound(p.head_dim)[0],
            "achieved": round(tflops, 2),
            "peak": roofline_bound(p.head_dim)[1],
            "unit": "TFLOP/s",
            "frac": round(tflops / roofline_bound(p.head_dim)[1], 4),
            "traffic": measured_traffic(p.name),
            "kernel": "ffa_fwd_main",
            "algorithmic_flops_per_launch": flops,
            "clock": measured_clock(p.name),
        },
    }
    if not args.no_backward:
        res["backward"] = backward_leg(args, p, qd, kd, vd, out, lse, strides, scale, sink)
    also = [w for w in args.also.split(",") if w and w != p.name]
    if also and not args.backward_only and args.sinks == 0:  # (sink logits are drawn for the main workload only)
        res["also"] = [also_leg(args, w) for w in also]
    if args.combine and not args.backward_only and args.sinks == 0:
        wl, _, st = args.combine.partition(":")
        res["combine"] = combine_leg(args, wl, int(st or 512))
    if args.total:
        res["total_attention"] = total_leg(args, p, qd, kd, lse, scale, sink)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(p, q, k, v, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def also_leg(args, name: str):
    """The forward of another workload, timed like the main step (HIP events on the launch
    stream after at least the same warm-up), with the same options; FLOPs as for the main line."""
    import torch

    import flexible_mask_flash_amd as ffa
    import workloads as W

    if name not in WORKLOADS:
        raise SystemExit(f"--also: unknown workload {name!r}")
    dev = torch.device("cuda", 0)
    p = W.workload(name)
    # drawn on the device (same distribution as the CPU draws; long-context inputs are 2.5 GB)
    qd, kd, vd = W.make_qkv_device(p, dev, dtype=torch.float16 if args.fp16 else None)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, split_tiles=args.split_tiles)
    plan.device_meta(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((p.total_q, p.heads_q), dtype=torch.float32, device=dev)
    strides = {"q": (0, qd.stride(0), qd.stride(1)), "k": (0, kd.stride(0), kd.stride(1)),
               "v": (0, vd.stride(0), vd.stride(1)), "out": (0, out.stride(0), out.stride(1)),
               "lse": (0, lse.stride(0), lse.stride(1))}
    extras = ffa.make_extras(None, "sh", args.softcap, total_q=p.total_q, heads_q=p.heads_q, dtype=qd.dtype,
                             rounded_norm=args.rounded_norm)
    scale = 1.0 / math.sqrt(p.head_dim)

    def step():
        ffa.run_fwd(plan, qd, kd, vd, out, lse, strides, 1, scale, extras)

    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < args.min_warmup_seconds:
        step()
        warm += 1
        if warm % 5 == 0:
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 4.0 * p.head_dim * p.heads_q * plan.info["visible_pairs"]
    tflops = flops / (ms * 1e-3) / 1e12
    bound, peak = roofline_bound(p.head_dim)
    return {"workload": p.name, "value": round(tflops, 2), "unit": "TFLOPS", "ms_per_step": round(ms, 4),
            "steps": args.steps, "warmup": warm, "flops_per_step": flops,
            "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
            "bound": bound, "peak": peak, "frac": round(tflops / peak, 4), "traffic": measured_traffic(p.name),
            "clock": measured_clock(p.name), "data": "synthetic, drawn on the device",
            "num_items": int(plan.info["num_items"]), "num_split_items": int(plan.info["num_split_items"])}


def combine_leg(args, name: str, split_tiles: int):
    """The split-K combine on its own: `name` planned with forced chunks of `split_tiles` key
    tiles, one ffa_fwd call to leave the partials in the workspace, then ffa_combine timed
    with HIP events.  Algorithmic bytes per launch: every split (row, head) reads its
    n_chunks partials (4 D + 4 bytes each) and writes out and lse (2 D + 4 bytes)."""
    import torch

    import flexible_mask_flash_amd as ffa
    import workloads as W

    dev = torch.device("cuda", 0)
    p = W.workload(name)
    qd, kd, vd = W.make_qkv_device(p, dev)
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, split_tiles=split_tiles)
    plan.device_meta(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((p.total_q, p.heads_q), dtype=torch.float32, device=dev)
    strides = {"q": (0, qd.stride(0), qd.stride(1)), "k": (0, kd.stride(0), kd.stride(1)),
               "v": (0, vd.stride(0), vd.stride(1)), "out": (0, out.stride(0), out.stride(1)),
               "lse": (0, lse.stride(0), lse.stride(1))}
    scale = 1.0 / math.sqrt(p.head_dim)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # the forced-split forward (main kernel + combine), a few steps
    ffa.run_fwd(plan, qd, kd, vd, out, lse, strides, 1, scale)
    torch.cuda.synchronize()
    n_fwd = 3
    e0.record(stream)
    for _ in range(n_fwd):
        ffa.run_fwd(plan, qd, kd, vd, out, lse, strides, 1, scale)
    e1.record(stream)
    torch.cuda.synchronize()
    fwd_ms = e0.elapsed_time(e1) / n_fwd
    # the combine alone over the partials the last forward left
    comb = lambda: ffa.run_combine(plan, out, lse, strides, 1)
    warm = 0
    t_w = time.perf_counter()
    while warm < max(3, args.warmup) or time.perf_counter() - t_w < args.min_warmup_seconds:
        comb()
        warm += 1
        if warm % 5 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        comb()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    meta = plan.meta_host()
    ni, nr, nc = plan.info["num_items"], plan.info["num_runs"], plan.info["num_combine"]
    recs = meta[16 + 16 * ni + 8 * nr:16 + 16 * ni + 8 * nr + 8 * nc].reshape(-1, 8).astype(np.int64)
    pairs = recs[:, 1] * plan.info["heads_per_item"]          # (row, head) pairs per entry
    d = p.head_dim
    nbytes = int((pairs * (recs[:, 3] * (4 * d + 4) + 2 * d + 4)).sum())
    tbs = nbytes / (ms * 1e-3) / 1e12
    flops = 4.0 * d * p.heads_q * plan.info["visible_pairs"]
    return {"workload": p.name, "split_tiles": split_tiles, "kernel": "ffa_combine", "bound": "hbm",
            "value": round(tbs, 3), "unit": "TB/s", "achieved": round(tbs, 3), "peak": HBM_PEAK_TBS,
            "frac": round(tbs / HBM_PEAK_TBS, 4), "ms_per_launch": round(ms, 4), "steps": args.steps,
            "algorithmic_bytes_per_launch": nbytes, "num_combine": int(nc),
            "num_split_items": int(plan.info["num_split_items"]),
            "split_forward": {"ms_per_step": round(fwd_ms, 3), "value": round(flops / (fwd_ms * 1e-3) / 1e12, 2),
                              "unit": "TFLOPS", "steps": n_fwd},
            "data": "synthetic, drawn on the device"}


def total_leg(args, p, qd, kd, lse, scale, sink=None):
    """Time ffa_total_attention (key-major pass: scores and probabilities only) on the same
    workload with the forward's lse.  FLOPs counted: 2 * D * Hq * visible pairs (one product)."""
    import torch

    import flexible_mask_flash_amd as ffa

    dev = qd.device
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, backward=True)
    plan.device_meta(dev)
    tot = torch.empty((p.total_k, p.heads_q), dtype=torch.float32, device=dev)
    st = {"q": (0, qd.stride(0), qd.stride(1)), "k": (0, kd.stride(0), kd.stride(1)),
          "lse": (0, lse.stride(0), lse.stride(1)), "total": (0, tot.stride(0), tot.stride(1))}
    extras = ffa.make_extras(sink, "sh", args.softcap, total_q=p.total_q, heads_q=p.heads_q, dtype=qd.dtype)

    def step():
        ffa.run_total(plan, qd, kd, lse, tot, st, 1, scale, extras)

    for _ in range(max(3, args.warmup)):
        step()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 2.0 * p.head_dim * p.heads_q * plan.info["visible_pairs"]
    return {"value": round(flops / (ms * 1e-3) / 1e12, 2), "unit": "TFLOPS", "ms_per_step": round(ms, 4),
            "flops_per_step": flops}


def backward_leg(args, p, qd, kd, vd, out, lse, strides, scale, sink=None):
    """Time ffa_bwd (dQ kernel, dK/dV kernel) on the same workload, with the
    forward's out and lse.  FLOPs counted as 10 * D * Hq * visible pairs: the five products
    of the gradient (dP, dV, dQ, dK and the recomputed scores), none of the recomputation."""
    import torch

    import flexible_mask_flash_amd as ffa
    import workloads as W

    dev = qd.device
    plan = ffa.Plan(p.q_ranges, p.k_ranges, p.mask_types, p.total_q, p.total_k, p.heads_q, p.heads_kv,
                    p.head_dim, backward=True)
    plan.device_meta(dev)
    dout = W.make_dout(p, dtype=qd.dtype).to(dev)
    dq = torch.empty_like(qd)
    dk = torch.empty_like(kd)
    dv = torch.empty_like(vd)
    t = {"q": qd, "k": kd, "v": vd, "out": out, "lse": lse, "dout": dout, "dq": dq, "dk": dk, "dv": dv}
    st = dict(strides)
    for n in ("dout", "dq", "dk", "dv"):
        st[n] = (0, t[n].stride(0), t[n].stride(1))

    dsink = torch.empty_like(sink) if sink is not None else None
    extras = ffa.make_extras(sink, "sh", args.softcap, dsink=dsink, total_q=p.total_q, heads_q=p.heads_q,
                             dtype=qd.dtype)

    def step():
        ffa.run_bwd(plan, t, st, 1, scale, extras)

    warm = 0
    t_w = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t_w < args.min_warmup_seconds:
        step()
        warm += 1
        if warm % 5 == 0:
            torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    flops = 10.0 * p.head_dim * p.heads_q * plan.info["visible_pairs"]
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "masked-attn bwd TFLOPS (10 * D * Hq * unmasked pairs)",
        "value": round(tflops, 2),
        "unit": "TFLOPS",
        "ms_per_step": round(ms, 4),
        "steps": args.steps,
        "warmup": warm,
        "flops_per_step": flops,
        "pct_of_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "plan": {k_: int(v_) for k_, v_ in plan.info.items() if k_ in
                 ("num_dq_items", "num_kv_items", "dq_tiles", "kv_tiles", "bwd_workspace_bytes")},
    }


if __name__ == "__main__":
    main()
