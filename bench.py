#!/usr/bin/env python3
"""Benchmark of the heterogeneous-adapter LoRA delta on one MI355X.

One step = one pass of the whole decode hot path over one batch: the segment
build and the delta of every projection of the workload (grouped shrink and
grouped expand launches, or the one launch of lora_decode_layer where the
batch fits it), with inputs resident in HBM.  The K timed steps replay from
one captured HIP graph, as a serving loop replays its decode step (--no-graph:
every launch from the host).  Prints one JSON line.

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
    "full_layer_r64_int8": "70B full layer decode as full_layer_r64, adapters int8 with one fp32 scale per row",
    "zipf_formed": "Zipf(1.1) decode over zipf_paged's 512 paged adapters: 256 rows chosen from a 512-request queue "
                   "by the adapter-aware batch former (cap 32 adapters, 4 tail slots, at least 128 rows)",
    "stacked_layer": "70B full layer decode, two adapters per row: one of 4 shared domain adapters (rank 64) and a "
                     "style adapter of its own (rank 16), all 7 projections, 128 rows; one pass per adapter",
    "fused_layer_r64": "70B full layer decode, base projection + delta fused: bf16 W of all 7 projections (1.63 GB) "
                       "and 128 distinct rank-64 adapters, 128 rows; y written once",
    "fused_layer_q4_r64": "70B full layer decode, base projection + delta fused with a 4-bit base: signed 4-bit W "
                          "of all 7 projections with one fp32 scale per 128 inputs (0.43 GB), 120 rows with distinct "
                          "rank-64 adapters and 8 base-only rows; y written once",
}


def formed_workload(gen):
    """The rows the library's batch former picks from the Zipf queue, and a
    report of the former: its choice and its host time per call."""
    import numpy as np
    import adapter_gemv_amd as lg
    q = gen.zipf_queue()
    sel = lg.form_batch(q, **gen.ZIPF_FORMER)
    calls = 200
    t0 = time.perf_counter()
    for _ in range(calls):
        lg.form_batch(q, **gen.ZIPF_FORMER)
    us = (time.perf_counter() - t0) / calls * 1e6
    fifo = q[:gen.ZIPF_FORMER["max_batch"]]
    report = {"queue": int(q.size), **gen.ZIPF_FORMER, "chosen": int(sel.size),
              "distinct_adapters": int(np.unique(q[sel]).size), "fifo_distinct_adapters": int(np.unique(fifo).size),
              "host_us_per_call": round(us, 2)}
    return gen.zipf_paged(ids=q[sel], name="zipf_formed"), report


def algorithmic(w, ids=None):
    """Bytes and FLOPs the method must move per step (per pass with ``ids``):
    each distinct adapter once at its own rank, each input tensor once, y read
    and written once; split into the shrink side (A, x) and the expand side
    (B, y)."""
    from adapter_gemv_amd.traffic import step_traffic
    return step_traffic(w.ids if ids is None else ids, w.num_slots,
                        [(m.name, m.index, m.d_in, m.d_out, m.x_name) for m in w.modules], w.ranks, w.fmt)


def cpu_baseline(w, min_seconds=10.0, max_passes=100000):
    """The oracle (single-threaded C, fp64) on the same seeded inputs: whole
    batches, repeated until about min_seconds of CPU work (max_passes only
    bounds a batch so small that a pass takes microseconds)."""
    import numpy as np
    import oracle
    try:
        os.sched_setaffinity(0, {sorted(os.sched_getaffinity(0))[0]})
    except (AttributeError, OSError):
        pass
    rows = None
    if w.seq_lens is not None:  # prefill: a bounded sample of rows
        rows = np.arange(0, w.num_rows, max(1, w.num_rows // 256), dtype=np.int32)
    if w.W is not None:  # base projection in fp64 on one core: a sample of 8 rows
        rows = np.arange(0, w.num_rows, max(1, w.num_rows // 8), dtype=np.int32)
    n_rows = w.num_rows if rows is None else rows.size
    t0 = time.perf_counter()
    passes = 0
    while True:
        if w.W is not None:
            oracle.build_segments(w.ids, w.num_slots)
            oracle.linear_layer(w, rows=rows)
        elif w.stack is None:
            oracle.build_segments(w.ids, w.num_slots)
            oracle.lora_layer(w, rows=rows)
        else:
            for t in range(w.stack.shape[1]):
                oracle.build_segments(w.stack[:, t], w.num_slots)
            oracle.lora_layer_stacked(w, w.stack, rows=rows)
        passes += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or passes >= max_passes:
            break
    return {"value": passes * n_rows / el, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} pass(es) of {n_rows} rows through every projection of the workload "
                      f"(segments + fp64 shrink/expand), single-threaded C pinned to one core, {el:.1f} s; "
                      f"host {platform.processor() or platform.machine()}, {os.cpu_count()} logical CPUs"}


def fused_comparison(w, d, lg, stream, steps, traffic):
    """The same work unfused, timed like the step: the base product by torch's
    bf16 GEMM into y, then segments and the delta (y read and written); and the
    base product alone."""
    import torch
    xs = {m.name: d.x[m.x_name][:w.num_rows] for m in w.modules}

    def base():
        for m in w.modules:
            torch.mm(xs[m.name], d.W[m.name].t(), out=d.y[m.name])

    def unfused():
        base()
        d.build_segments(stream)
        lg.apply_layer(d.ios, w.num_rows, d.table, w.num_slots, d.seg, w.max_rank, d.ws, stream)

    def timed(fn):
        with torch.cuda.stream(stream):
            for _ in range(3):
                fn()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) / steps

    base_ms, unfused_ms = timed(base), timed(unfused)
    return {"base_weight_bytes": traffic["base_weights"],
            "unfused_ms_per_step": round(unfused_ms, 5), "base_gemm_ms_per_step": round(base_ms, 5),
            "base_gemm_gbps": round(traffic["base_weights"] / (base_ms * 1e-3) / 1e9, 1),
            "unfused": "torch.mm (bf16 GEMM library) into y, then lora_build_segments + lora_apply_layer"}


def copy_ceiling(torch, stream, nbytes=1 << 30, reps=10):
    """A plain device-to-device copy of nbytes on the launch stream: bytes read
    plus bytes written per second (the practical HBM ceiling of this machine)."""
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    with torch.cuda.stream(stream):
        for _ in range(2):
            dst.copy_(src)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        b.record(stream)
        torch.cuda.synchronize()
    s = a.elapsed_time(b) * 1e-3 / reps
    del src, dst
    return 2 * nbytes / s / 1e9


def read_ceiling(torch, stream, nbytes, reps=20, pool_bytes=1 << 30):
    """A kernel that only reads (libread_ceiling.so), over nbytes per launch,
    each launch in the next of enough buffers to span pool_bytes (as the
    adapter replicas do, so the reads come from HBM): bytes read per second,
    reps launches replayed from one HIP graph on the launch stream."""
    import ctypes
    here = os.path.dirname(os.path.abspath(__file__))
    lib = ctypes.CDLL(os.path.join(here, "adapter_gemv_amd", "libread_ceiling.so"))
    lib.read_ceiling_launch.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.read_ceiling_blocks.argtypes = [ctypes.c_uint64]
    nbuf = max(2, -(-pool_bytes // nbytes) + 1)
    bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(nbuf)]
    sink = torch.zeros(lib.read_ceiling_blocks(nbytes), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def launch(i):
        rc = lib.read_ceiling_launch(bufs[i % nbuf].data_ptr(), nbytes, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"read_ceiling_launch: hip error {rc}")

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(reps):
            launch(i)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        a.record(stream)
        g.replay()
        b.record(stream)
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / reps
    del bufs, sink, g
    return nbytes / (us * 1e-6) / 1e9, us


def rank_class(max_rank):
    """Template class of the grouped kernels for a launch's largest rank."""
    return 0 if max_rank <= 8 else 1 if max_rank <= 16 else 2 if max_rank <= 32 else 3


def library_sha256():
    """Hash of the built library: counter figures taken with another build no
    longer describe the kernels (the build is reproducible, and comments do
    not change it)."""
    import hashlib
    with open(os.path.join(ROOT, "adapter_gemv_amd", "liblora_gemv.so"), "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def profile_records():
    """The machine-readable blocks of the counter summaries in profiles/."""
    import re
    out = []
    d = os.path.join(ROOT, "profiles")
    if not os.path.isdir(d):
        return out
    for f in sorted(os.listdir(d)):
        if not f.endswith(".md"):
            continue
        text = open(os.path.join(d, f)).read()
        for block in re.findall(r"```json\n(.*?)\n```", text, re.S):
            try:
                rec = json.loads(block)
            except ValueError:
                continue
            rec["_file"] = f"profiles/{f}"
            out.append(rec)
    return out


def counter_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of
    this workload, or None when there is none or the library has changed
    since the counters were taken."""
    digest = library_sha256()
    for rec in profile_records():
        k = rec.get("kernels", {}).get(kernel)
        if rec.get("workload") == workload and rec.get("library_sha256") == digest and k and \
                k.get("bytes_per_launch") is not None:
            return {"bytes_per_launch": k["bytes_per_launch"], "source": rec["_file"]}
    return None


def _short_kernel_name(name):
    import re
    m = re.search(r"(\w+_kernel)(<\w+>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name.strip('"')[:60]


def summarize_profile(a):
    """Markdown summary of one profiled workload from rocprofv3 CSV output:
    per-kernel durations (kernel trace), FETCH_SIZE / WRITE_SIZE per dispatch
    scaled by a plain copy of known size, and the algorithmic bytes of the
    bench line of the traced run."""
    import csv
    import glob
    from collections import defaultdict

    def csvs(d, pattern):
        return sorted(glob.glob(os.path.join(d, "**", pattern), recursive=True))

    stats = {}
    for f in csvs(a.trace, "*kernel_stats.csv"):
        for r in csv.DictReader(open(f)):
            stats[_short_kernel_name(r["Name"])] = r

    def counter(d, kernel_filter=None):
        agg = defaultdict(list)
        for f in csvs(d, "*counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                agg[_short_kernel_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in agg.items()}, {k: len(v) for k, v in agg.items()}

    fetch, n_fetch = counter(a.fetch)
    write, n_write = counter(a.write)
    cf, _ = counter(a.copy_fetch)
    cw, _ = counter(a.copy_write)
    copy_name = "__amd_rocclr_copyBuffer"
    copy_kib = a.copy_bytes / 1024.0
    f_scale = copy_kib / cf[copy_name]
    w_scale = copy_kib / cw[copy_name]
    bench = json.loads(open(a.bench_json).read().strip().splitlines()[-1])
    alg = bench["hbm"]["algorithmic_bytes_per_launch"]
    lines = [f"# Kernel profile: {bench['config']['name']} ({bench['config']['workload']})", ""]
    lines += ["Commands, run from the repository root on one MI355X (rocprofv3, ROCm 7):", "", "```"]
    lines += open(a.commands).read().strip().splitlines() + ["```", ""]
    lines += ["## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
              "| kernel | calls | avg us | min us | max us | share |", "|---|---:|---:|---:|---:|---:|"]
    for k, r in sorted(stats.items(), key=lambda kv: -float(kv[1]["TotalDurationNs"])):
        lines.append(f"| `{k}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f}% |")
    lines += ["", f"Bench events in the traced run: {json.dumps(bench['phases_us'])} us per launch.", ""]
    lines += ["## HBM bytes (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE; KiB per dispatch)", "",
              f"Scale: a plain device copy of {a.copy_bytes} bytes reads FETCH_SIZE {cf[copy_name]:.1f} KiB and "
              f"WRITE_SIZE {cw[copy_name]:.1f} KiB per dispatch, so FETCH_SIZE x {f_scale:.4f} and "
              f"WRITE_SIZE x {w_scale:.4f} give bytes.", "",
              "| kernel | dispatches | FETCH KiB | WRITE KiB | HBM bytes / launch | algorithmic bytes / launch | "
              "ratio |", "|---|---:|---:|---:|---:|---:|---:|"]
    record = {"workload": bench["config"]["name"], "library_sha256": library_sha256(),
              "fetch_scale": f_scale, "write_scale": w_scale, "kernels": {}}
    for k in sorted(fetch):
        if k not in write or not k.startswith(("lora_", "seg_", "shrink_")):
            continue
        b = (fetch[k] * f_scale + write[k] * w_scale) * 1024.0
        phase = ("shrink" if k.startswith("lora_shrink") else
                 "expand" if k.startswith(("lora_expand", "lora_fused")) else None)
        per_kernel = bench.get("kernels_algorithmic_bytes_per_launch")
        if per_kernel is not None:  # the step's own kernels (a comparison leg's get none)
            alg_b = per_kernel.get(k)
        else:
            alg_b = alg.get(phase) if phase else None
        ratio = f"{b / alg_b:.3f}" if alg_b else "-"
        lines.append(f"| `{k}` | {n_fetch[k]} | {fetch[k]:.1f} | {write[k]:.1f} | {b:.4g} | "
                     f"{alg_b if alg_b else '-'} | {ratio} |")
        st = stats.get(k)
        record["kernels"][k] = {"fetch_kib": round(fetch[k], 1), "write_kib": round(write[k], 1),
                                "bytes_per_launch": round(b), "algorithmic_bytes_per_launch": alg_b,
                                "avg_us": round(float(st["AverageNs"]) / 1e3, 2) if st else None}
    if getattr(a, "mfma", None):
        agg = defaultdict(lambda: defaultdict(list))
        for f in csvs(a.mfma, "*counter_collection.csv"):
            for r in csv.DictReader(open(f)):
                agg[_short_kernel_name(r["Kernel_Name"])][r["Counter_Name"]].append(float(r["Counter_Value"]))
        simds = 1024  # 256 CUs x 4 SIMDs
        lines += ["", "## Matrix cores (rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES "
                  "GRBM_GUI_ACTIVE; per dispatch)", "",
                  "bf16 MFMA flops = MOPS x 512; TFLOP/s = flops / the trace's average duration, against 2,500 "
                  "TFLOP/s dense bf16 (the utilisation figure).  The raw counter ratio MFMA busy cycles / "
                  "(GRBM_GUI_ACTIVE x 1024 SIMDs) is listed too; its denominator as collected here appears to "
                  "span all XCDs, so it reads about 8x below the flops-based figure.", "",
                  "| kernel | MFMA flops / launch | raw busy ratio | TFLOP/s | of peak |", "|---|---:|---:|---:|---:|"]
        for k in sorted(agg):
            c = agg[k]
            if not k.startswith("lora_") or "SQ_INSTS_VALU_MFMA_MOPS_BF16" not in c:
                continue
            mean = {n: sum(v) / len(v) for n, v in c.items()}
            flops = mean["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
            busy = mean.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) / max(mean.get("GRBM_GUI_ACTIVE", 1), 1) / simds
            st = stats.get(k)
            tf = flops / (float(st["AverageNs"]) * 1e-9) / 1e12 if st else 0.0
            lines.append(f"| `{k}` | {flops:.4g} | {100 * busy:.1f}% | {tf:.1f} | {100 * tf / 2500:.2f}% |")
            if k in record["kernels"]:
                record["kernels"][k].update({"mfma_flops": round(flops), "mfma_busy": round(busy, 4),
                                             "mfma_tflops": round(tf, 1)})
    lines += ["", "Machine-readable record (the benchmark reports `traffic` from it while the built library "
              "hashes to `library_sha256`):", "", "```json", json.dumps(record, indent=1), "```", ""]
    print("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="full_layer_r64", choices=sorted(DESCRIPTIONS))
    ap.add_argument("--replicas", type=int, default=0,
                    help="independent copies of the adapters to rotate through (0 = enough to exceed 1 GB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--path", choices=("decode", "phases"), default="decode",
                    help="decode: a step is one lora_decode_layer call (one launch for batches that fit it); "
                         "phases: lora_build_segments + lora_layer_shrink + lora_layer_expand")
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from the host (default: the K steps replay from one captured HIP graph)")
    ap.add_argument("--no-segment-bound", action="store_true",
                    help="give the calls no bound on the segments (max_segments = 0): work items sized for one "
                         "adapter per row")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (3 times), to scale HBM byte counters")
    ap.add_argument("--summarize-profile", action="store_true",
                    help="only print a markdown summary of rocprofv3 CSV output (needs the options below)")
    ap.add_argument("--trace", help="rocprofv3 --kernel-trace --stats output directory")
    ap.add_argument("--fetch", help="rocprofv3 --pmc FETCH_SIZE output directory")
    ap.add_argument("--write", help="rocprofv3 --pmc WRITE_SIZE output directory")
    ap.add_argument("--copy-fetch", help="FETCH_SIZE output directory of the copy calibration")
    ap.add_argument("--copy-write", help="WRITE_SIZE output directory of the copy calibration")
    ap.add_argument("--copy-bytes", type=int, help="bytes of the copy calibration")
    ap.add_argument("--mfma", help="rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES "
                                   "GRBM_GUI_ACTIVE output directory (optional)")
    ap.add_argument("--bench-json", help="the bench line printed by the traced run")
    ap.add_argument("--commands", help="text file with the commands that made the profile")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path. Run with --gpus 1.",
              file=sys.stderr)
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
    former = None
    if args.workload == "zipf_formed":
        w, former = formed_workload(gen)
    else:
        w = gen.make_workload(args.workload)
    q4 = w.W is not None and hasattr(next(iter(w.W.values())), "scales")
    if w.W is not None:  # fused: + the base weights, y written once (not read)
        traffic = algorithmic(w)
        # bf16: 2 bytes per weight; 4-bit: half a byte per weight and 4 bytes per group scale
        w_bytes = sum(m.d_in * m.d_out // 2 + m.d_out * (m.d_in // gen.Q4_GROUP) * 4 if q4 else
                      2 * m.d_in * m.d_out for m in w.modules)
        y_write = traffic["y"] // 2
        b_bytes = traffic["expand_bytes"] - traffic["y"]
        traffic["total"] = w_bytes + traffic["adapters"] + traffic["x"] + y_write
        traffic["expand_bytes"] = w_bytes + b_bytes + traffic["x"] + y_write  # the fused kernel
        traffic["base_weights"] = w_bytes
        passes = [traffic]
    elif w.stack is None:
        traffic = algorithmic(w)
        passes = [traffic]
    else:  # one pass per column: each reads its adapters, x and y again
        passes = [algorithmic(w, w.stack[:, t]) for t in range(w.stack.shape[1])]
        traffic = {k: sum(p[k] for p in passes) for k in passes[0]}
    adapters_bytes = traffic["adapters"]
    reps = args.replicas or max(1, int(np.ceil(1.0e9 / max(adapters_bytes, 1))))
    reps = min(reps, 64)
    print(f"[bench] uploading {reps} replica(s)", file=sys.stderr, flush=True)
    # The host formed the batch, so it passes the batch's distinct adapter count as the segment bound.
    dws = [DeviceWorkload(w, bound_segments=not args.no_segment_bound) for _ in range(reps)]
    torch.cuda.synchronize()

    import adapter_gemv_amd as lg

    # Every launch and every event goes on one stream of default priority.
    stream = torch.cuda.Stream()

    stack = None if w.stack is None else torch.from_numpy(np.ascontiguousarray(w.stack)).cuda()
    # each pass's launch class: the largest rank among its column's adapters (the caller knows it)
    pass_rank = [w.max_rank] if stack is None else [
        max(1, int(w.ranks[w.stack[:, t][(w.stack[:, t] >= 0) & (w.stack[:, t] < w.num_slots)]].max(initial=1)))
        for t in range(w.stack.shape[1])]

    def launch(i):
        d = dws[i % reps]
        if d.W is not None:
            d.build_segments(stream)
            lg.linear_layer(d.lin_ios, w.num_rows, d.ids, d.table, w.num_slots, d.seg, w.max_rank, d.ws, stream,
                            module_mask=d.mask)
            return
        if stack is not None:
            lg.apply_layer_stacked(d.ios, w.num_rows, stack, d.table, w.num_slots, d.seg, w.max_rank, d.ws, stream,
                                   pass_max_rank=pass_rank, module_mask=d.mask)
            return
        if args.path == "decode":
            d.decode_layer(stream)  # segments + delta: one launch when the batch fits it, else three
            return
        d.build_segments(stream)
        lg.layer_shrink(d.ios, w.num_rows, d.table, w.num_slots, d.seg, w.max_rank, d.ws, stream, module_mask=d.mask)
        lg.layer_expand(d.ios, w.num_rows, d.table, w.num_slots, d.seg, w.max_rank, d.ws, stream, module_mask=d.mask)

    for i in range(args.warmup):
        launch(i)
    torch.cuda.synchronize()

    use_graph = not args.no_graph

    def captured(fn, n):
        """fn(0), ..., fn(n-1), captured on the launch stream into one HIP graph
        and replayed once untimed (the replay uploads the graph).  The library
        calls launch kernels only: no allocation, copy or memset is recorded."""
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        return g

    def run_timed(fn, n):
        """ms for fn(0..n-1) between two HIP events on the launch stream: one
        replay of their graph, or n launches from the host"""
        g = captured(fn, n) if use_graph else None
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        if g is not None:
            with torch.cuda.stream(stream):
                g.replay()
        else:
            for i in range(n):
                fn(i)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b)

    # ---- timed region: K steps between two HIP events on the launch stream.
    ms = run_timed(launch, args.steps) / args.steps
    value = w.num_rows / (ms * 1e-3)
    gbps = traffic["total"] / (ms * 1e-3) / 1e9

    # ---- spread: the same K steps again, each between its own pair of HIP
    # events on the launch stream (outside the timed region above)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(args.steps):
        launch(i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)])

    # ---- each kernel's average duration: per phase, K launches back to back
    # (the same replicas in the same order) between two HIP events on the
    # launch stream.  Every replica's segments and partials are already valid
    # from the steps above, so each phase can repeat on its own (the expand
    # then adds its delta more than once, which timing does not care about).
    def phase_us(fn):
        return run_timed(lambda i: fn(dws[i % reps]), args.steps) / args.steps * 1e3

    # A stacked step runs the kernels once per pass (one column of the adapter
    # lists each, in that column's rank class); a kernel's figures sum over
    # its launches in a step.
    cols = [None] if stack is None else [stack[:, t].contiguous() for t in range(stack.shape[1])]
    per_pass = []
    kernels = {}  # name -> [launches, us, algorithmic bytes] per step
    one_launch = args.path == "decode" and w.W is None and stack is None and dws[0].decode_launches() == 1
    if one_launch:  # the step is one kernel: segments, shrink and expand of every projection
        one_us = phase_us(lambda d: d.decode_layer(stream))
        kernels[f"lora_onepass_kernel<{rank_class(w.max_rank)}>"] = [1, one_us, traffic["total"]]
        cols = []
    for t, col in enumerate(cols):
        r = pass_rank[t]
        if col is None:
            seg_us = phase_us(lambda d: d.build_segments(stream))
        else:
            seg_us = phase_us(lambda d: lg.build_segments(col, w.num_slots, d.seg, d.ws, stream))
        if w.W is not None:  # the fused call's two parts: grouped shrink (+ v sums), fused kernel
            shr_us = phase_us(lambda d: lg.linear_shrink(d.lin_ios, w.num_rows, d.ids, d.table, w.num_slots, d.seg,
                                                         r, d.ws, stream, module_mask=d.mask))
            exp_us = phase_us(lambda d: lg.linear_expand(d.lin_ios, w.num_rows, d.ids, d.table, w.num_slots, d.seg,
                                                         r, d.ws, stream, module_mask=d.mask))
        else:
            shr_us = phase_us(lambda d: lg.layer_shrink(d.ios, w.num_rows, d.table, w.num_slots, d.seg, r, d.ws,
                                                        stream, module_mask=d.mask))
            exp_us = phase_us(lambda d: lg.layer_expand(d.ios, w.num_rows, d.table, w.num_slots, d.seg, r, d.ws,
                                                        stream, module_mask=d.mask))
        per_pass.append({"segments": seg_us, "shrink": shr_us, "expand": exp_us})
        for ph, us in (("shrink", shr_us), ("expand", exp_us)):
            name = f"lora_fused_kernel<{'true' if q4 else 'false'}>" if (w.W is not None and ph == "expand") \
                else f"lora_{ph}_kernel<{rank_class(r)}>"
            k = kernels.setdefault(name, [0, 0.0, 0])
            k[0] += 1
            k[1] += us
            k[2] += passes[t][ph + "_bytes"]
    if one_launch:
        phases = {"onepass": (one_us, traffic["total"])}
    else:
        phases = {"segments": (sum(p["segments"] for p in per_pass), 0),
                  "shrink": (sum(p["shrink"] for p in per_pass), traffic["shrink_bytes"]),
                  "expand": (sum(p["expand"] for p in per_pass), traffic["expand_bytes"])}
    ceiling = copy_ceiling(torch, stream)
    read_gbps, read_us = read_ceiling(torch, stream, int(traffic["total"]))
    kernel_name = max(kernels, key=lambda k: kernels[k][1])
    n_launch, tot_us, tot_bytes = kernels[kernel_name]
    achieved = tot_bytes / (tot_us * 1e-6) / 1e9
    dom_us, dom_bytes = tot_us / n_launch, int(round(tot_bytes / n_launch))  # per launch
    counted = counter_traffic(args.workload, kernel_name)

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
        # int8 factors, 4-bit base: integers exact in the bf16/fp32 products
        "dtype": "int4xbf16" if q4 else "int8xbf16" if (w.fmt != 0).any() else "bf16",
        "data": "synthetic (seeded, shapes of the pages' 70B workloads)",
        "config": {"workload": DESCRIPTIONS[args.workload], "name": args.workload, "rows": w.num_rows,
                   "distinct_adapters": int(len(np.unique(w.ids[w.ids >= 0]))),
                   "max_segments": dws[0].seg.max_segments,
                   "modules": [m.name for m in w.modules], "max_rank": w.max_rank,
                   "adapter_replicas": reps, "parallelism": "single GPU"},
        "hbm": {"algorithmic_bytes_per_step": traffic["total"],
                "algorithmic_bytes_per_launch": {"shrink": traffic["shrink_bytes"],
                                                 "expand": traffic["expand_bytes"]},
                "achieved_gbps": round(gbps, 1),
                "pct_of_peak": round(100 * gbps / PEAK_HBM_GBPS, 2), "peak_gbps": PEAK_HBM_GBPS,
                "copy_ceiling_gbps": round(ceiling, 1), "pct_of_copy_ceiling": round(100 * gbps / ceiling, 2),
                "copy_ceiling": "torch copy_ of 1 GiB on the launch stream, read + written bytes / time",
                "read_ceiling_gbps": round(read_gbps, 1), "read_ceiling_us": round(read_us, 2),
                "pct_of_read_ceiling": round(100 * gbps / read_gbps, 2),
                "read_ceiling": "a read-only kernel over the step's algorithmic bytes, from buffers spanning 1 GiB, "
                                "replayed from a HIP graph"},
        "step_ms": {"median": round(float(np.median(per_step)), 5), "p10": round(float(np.percentile(per_step, 10)), 5),
                    "p90": round(float(np.percentile(per_step, 90)), 5), "min": round(float(per_step.min()), 5),
                    "max": round(float(per_step.max()), 5), "steps": int(per_step.size),
                    "how": "each step launched from the host between its own HIP events, in a pass after the "
                           "timed region"},
        "launch": ("the K steps (and each kernel's K launches) replayed from one captured HIP graph, "
                   "after one untimed replay" if use_graph else "every launch from the host"),
        "int8_items": bool(dws[0].int8_items),  # LORA_MASK_INT8_ITEMS passed (every targeted entry int8)
        "path": ("one launch (lora_decode_layer)" if one_launch else
                 "lora_decode_layer (three launches)" if args.path == "decode" and w.W is None and stack is None
                 else "separate launches"),
        "phases_us": {k: round(v[0], 2) for k, v in phases.items()},
        "kernels_algorithmic_bytes_per_launch": {k: int(round(v[2] / v[0])) for k, v in kernels.items()},
        "roofline": {"bound": "hbm", "kernel": kernel_name, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS,
                     "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBPS, 4),
                     "traffic": counted["bytes_per_launch"] if counted else None,
                     "algorithmic_bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_us, 2),
                     "traffic_source": counted["source"] if counted else None},
    }
    if former is not None:
        out["batch_former"] = former
    if w.W is not None and not q4:  # torch has no 4-bit GEMM to compare with
        out["fused"] = fused_comparison(w, dws[0], lg, stream, args.steps, traffic)
    elif q4:
        out["fused"] = {"base_weight_bytes": traffic["base_weights"], "base_format": "4-bit, fp32 scale per 128"}
    if stack is not None:
        out["stacked"] = {"depth": len(per_pass), "pass_max_rank": pass_rank,
                          "passes_us": [{k: round(v, 2) for k, v in p.items()} for p in per_pass],
                          "algorithmic_bytes_per_pass": [p["total"] for p in passes],
                          "distinct_adapters_per_pass": [int(np.unique(w.stack[:, t]).size) for t in
                                                         range(len(per_pass))]}
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
