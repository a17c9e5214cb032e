#!/usr/bin/env python3
"""Benchmark of the heterogeneous-adapter LoRA delta on one MI355X.

One step = one pass of the whole decode hot path over one batch: the segment
build and the delta of every projection of the workload (grouped shrink and
grouped expand launches), with inputs resident in HBM.  Prints one JSON line.

Default workload: the 70B full layer (q, k, v, o, gate, up, down at rank 64)
with 128 decode rows, each with its own adapter (128 resident adapters), bf16.
Other seeded workloads: --workload {tiny,q_proj_r16,zipf_paged,prefill_r16,prefill_r64}.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0  # MI355X HBM3E, AMD published
METRIC = "LoRA-delta tokens/s and achieved HBM GB/s (% peak), batch 128 distinct adapters"
DESCRIPTIONS = {
    "tiny": "tiny decode delta: 256->256, rank 8, 4 adapters, 16 rows",
    "q_proj_r16": "70B q_proj decode: 8192->8192, rank 16, 128 rows, 128 distinct adapters",
    "full_layer_r64": "70B full layer decode: q,o 8192->8192; k,v 8192->1024; gate,up 8192->28672; "
                      "down 28672->8192; rank 64 on all 7; 128 rows, 128 distinct adapters",
    "zipf_paged": "Zipf(1.1) decode: 512 paged adapters, ranks {8,16,32,64}, 256 rows, q/k/v/o",
    "prefill_r16": "prefill SGMV: 32 sequences, lengths U[128,2048], rank 16, q/o 8192->8192",
    "prefill_r64": "prefill SGMV: 32 sequences, lengths U[128,2048], rank 64, q/o 8192->8192",
}


def algorithmic(w):
    """Bytes and FLOPs the method must move per step: each distinct adapter
    once at its own rank, each input tensor once, y read and written once;
    split into the shrink side (A, x) and the expand side (B, y)."""
    from adapter_gemv_amd.traffic import step_traffic
    return step_traffic(w.ids, w.num_slots, [(m.name, m.index, m.d_in, m.d_out, m.x_name) for m in w.modules],
                        w.ranks)


def cpu_baseline(w, min_seconds=10.0, max_passes=64):
    """The oracle (single-threaded C, fp64) on the same seeded inputs: whole
    batches, repeated until about min_seconds of CPU work."""
    import numpy as np
    import oracle
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    rows = None
    if w.seq_lens is not None:  # prefill: a bounded sample of rows
        rows = np.arange(0, w.num_rows, max(1, w.num_rows // 256), dtype=np.int32)
    n_rows = w.num_rows if rows is None else rows.size
    t0 = time.perf_counter()
    passes = 0
    while True:
        oracle.build_segments(w.ids, w.num_slots)
        oracle.lora_layer(w, rows=rows)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= max_passes:
            break
    return {"value": passes * n_rows / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} pass(es) of {n_rows} rows through every projection of the workload "
                      f"(segments + fp64 shrink/expand), single-threaded C pinned to one core, {el:.1f} s; "
                      f"host {platform.processor() or platform.machine()}, {os.cpu_count()} logical CPUs"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="full_layer_r64", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--replicas", type=int, default=0,
                    help="independent copies of the adapters to rotate through (0 = enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times), to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the design of sharding is described in DESIGN.md). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "launches": 3}), flush=True)
        return

    from workloads import gen
    from workloads.device import DeviceWorkload

    print(f"[bench] generating {args.workload}", file=sys.stderr, flush=True)
    w = gen.make_workload(args.workload)
    traffic = algorithmic(w)
    adapters_bytes = traffic["adapters"]
    reps = args.replicas or max(1, int(np.ceil(1.0e9 / max(adapters_bytes, 1))))
    reps = min(reps, 64)
    print(f"[bench] uploading {reps} replica(s)", file=sys.stderr, flush=True)
    dws = [DeviceWorkload(w) for _ in range(reps)]
    torch.cuda.synchronize()

    def step(i):
        dws[i % reps].step()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- whole-step throughput
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    value = w.num_rows / (ms * 1e-3)
    gbps = traffic["total"] / (ms * 1e-3) / 1e9

    # ---- per-launch durations of the two grouped kernels (HIP events on the
    # launch stream around each launch)
    import adapter_gemv_amd as lg
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        d = dws[i % reps]
        e = ev[i]
        e[0].record(stream)
        d.build_segments()
        e[1].record(stream)
        lg.layer_shrink(d.ios, w.num_rows, d.table, w.num_slots, d.seg, w.max_rank, d.ws)
        e[2].record(stream)
        lg.layer_expand(d.ios, w.num_rows, d.table, w.num_slots, d.seg, w.max_rank, d.ws)
        e[3].record(stream)
    torch.cuda.synchronize()
    seg_us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1e3
    shr_us = float(np.mean([e[1].elapsed_time(e[2]) for e in ev])) * 1e3
    exp_us = float(np.mean([e[2].elapsed_time(e[3]) for e in ev])) * 1e3
    phases = {"segments": (seg_us, 0), "shrink": (shr_us, traffic["shrink_bytes"]),
              "expand": (exp_us, traffic["expand_bytes"])}
    dom = max(("shrink", "expand"), key=lambda k: phases[k][0])
    dom_us, dom_bytes = phases[dom]
    achieved = dom_bytes / (dom_us * 1e-6) / 1e9
    kernel_name = {"shrink": "decode_shrink_kernel", "expand": "decode_expand_kernel"}[dom]

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded, shapes of the pages' 70B workloads)",
        "config": {"workload": DESCRIPTIONS[args.workload], "name": args.workload, "rows": w.num_rows,
                   "distinct_adapters": int(len(np.unique(w.ids[w.ids >= 0]))),
                   "modules": [m.name for m in w.modules], "max_rank": w.max_rank,
                   "adapter_replicas": reps, "parallelism": "single GPU"},
        "hbm": {"algorithmic_bytes_per_step": traffic["total"], "achieved_gbps": round(gbps, 1),
                "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2), "peak_gbps": PEAK_HBM_GBPS},
        "phases_us": {k: round(v[0], 2) for k, v in phases.items()},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2)},
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
