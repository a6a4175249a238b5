#!/usr/bin/env python3
"""Decode-step benchmark: paged GQA decode attention over an fp8 paged KV cache.

A step is one decode of the whole batch of the bandwidth workload (128
sequences x 8 kv heads x query group 8, head_dim 128, 8192 cached tokens each,
block size 32, 32 partitions of 1 tile group), with inputs already resident in
HBM, through either complete path of the library: tq_decode (partition kernel)
+ tq_decode_reduce (merge), or tq_decode_fused (one launch).  Both are timed;
the faster is the headline step.  Prints ONE JSON line on stdout; details go to
stderr.

  value         algorithmic KV bytes per step / step time (GB/s); KV bytes =
                sum over sequences and kv heads of L * 264 (128 B K codes,
                128 B V codes, 2 fp32 scales)
  roofline      the headline path's first kernel: the same bytes / its average
                duration over K back-to-back launches between two HIP events on
                the launch stream, against MI355X's 8 TB/s (the step time is
                measured the same way over K whole steps; for the one-launch
                fused path the step and the kernel are the same timed region)
  hbm_probe     best read and copy bandwidth of plain streaming kernels, and the
                bandwidth of the decode's own byte pattern with no arithmetic
  cpu_baseline  the fp64 oracle on a bounded sample of the same workload
  kv_writer     tq_kv_write on 16384 new tokens scattered into the same pool
  tq4           the same step over the 4-bit record format (tq4_decode + reduce,
                and tq4_decode_fused): time, GB/s and token-heads/s against fp8
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

HBM_PEAK_GBS = 8000.0
KV_BYTES_PER_TOKEN_HEAD = 2 * 128 + 8
METRIC = "KV-cache GB/s achieved (% of MI355X HBM peak); decode attn µs per step"
KERNEL_SOURCE = os.path.join(ROOT, "paged_gqa_decode_amd", "csrc", "tq_kernels.hip")
KERNEL_NAMES = {"two_kernel": "tq_partition_kernel", "fused": "tq_flat_kernel"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


PROFILES = os.path.join(ROOT, "profiles")


def measured_traffic(workload: str, path_name: str, profiles_dir: str = PROFILES):
    """HBM bytes per launch of the headline kernel from the committed rocprofv3
    counter summary, or None if there is none or the kernel source changed since."""
    path = os.path.join(profiles_dir, f"traffic_{KERNEL_NAMES[path_name]}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_info():
    """CPU model, physical cores and logical CPUs of the host (from /proc/cpuinfo), and the
    CPUs this process may run on."""
    model, phys, logical = None, set(), 0
    try:
        with open("/proc/cpuinfo") as f:
            cur = {}
            for ln in f.read().splitlines() + [""]:
                if not ln.strip():
                    if cur:
                        logical += 1
                        phys.add((cur.get("physical id"), cur.get("core id")))
                        model = model or cur.get("model name")
                    cur = {}
                    continue
                k, _, v = ln.partition(":")
                cur[k.strip()] = v.strip()
    except OSError:
        pass
    return {"cpu_model": model, "physical_cores": len(phys) or None, "logical_cpus": logical or None,
            "cpus_available": len(os.sched_getaffinity(0))}


# The oracle's threads: every CPU this process may use, at most 16 (the CPU share of one GPU
# on an 8-GPU host, whatever the host has in all).
CPU_BASELINE_MAX_THREADS = 16


def cpu_baseline(inp, budget_s: float):
    """Time the fp64 oracle (as it stands) on whole (sequence, kv head) units of the workload:
    with all the threads it may use, and with one thread on a smaller sample."""
    import oracle

    c = inp.to("cpu")
    wl = inp.wl
    info = cpu_info()
    threads = max(1, min(CPU_BASELINE_MAX_THREADS, info["cpus_available"]))
    units = [(s, h) for s in range(wl.num_seqs) for h in range(wl.num_kv_heads)]
    lens = c.seq_lens.numpy()

    def run(n, nthreads):
        sel = units[:n]
        t0 = time.perf_counter()
        oracle.decode(c.q, c.k_cache, c.v_cache, c.kv_scales, c.block_tables, c.seq_lens,
                      inp.softmax_scale, units=sel, nthreads=nthreads)
        return time.perf_counter() - t0, sel

    def sized(nthreads, budget):
        # calibrate on `nthreads` units, then size the sample to about `budget` seconds
        dt, sel = run(nthreads, nthreads)
        n = max(nthreads, min(len(units), int(nthreads * budget / max(dt, 1e-3))))
        n = (n // nthreads) * nthreads or nthreads
        dt, sel = run(n, nthreads)
        kv_bytes = sum(int(lens[s]) for s, _ in sel) * KV_BYTES_PER_TOKEN_HEAD
        return kv_bytes / dt / 1e9, dt, sel

    def token_heads(sel):
        return sum(int(lens[s]) for s, _ in sel)

    gbs, dt, sel = sized(threads, budget_s)
    gbs1, dt1, sel1 = sized(1, budget_s / 3)
    # the whole workload's oracle time at the measured rate (the sample is whole units)
    total_th = sum(int(lens[s]) for s, _ in units)
    step_s = dt * total_th / max(token_heads(sel), 1)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "threads": threads, "cpu_model": info["cpu_model"],
            "physical_cores": info["physical_cores"], "logical_cpus": info["logical_cpus"],
            "cpus_available": info["cpus_available"],
            "token_heads_per_s": round(token_heads(sel) / dt),
            "us_per_step": round(step_s * 1e6),
            "one_thread": {"value": round(gbs1, 4), "unit": "GB/s",
                           "token_heads_per_s": round(token_heads(sel1) / dt1),
                           "sample": f"{len(sel1)} units, {dt1:.1f} s wall"},
            "sample": f"{len(sel)} of {len(units)} (sequence, kv head) units of {wl.name} "
                      f"({int(lens[sel[0][0]])} tokens each, all {wl.query_group_size} query rows), "
                      f"fp64 C oracle on {threads} threads, {dt:.1f} s wall"}


def hbm_probe(dev, read_gib: float = 4.0, copy_gib: float = 1.0, reps: int = 10):
    """Best-of read and copy bandwidth of the streaming probes (GB/s, bytes moved / time)."""
    import torch

    from paged_gqa_decode_amd import probe

    nread = int(read_gib * (1 << 30))
    ncopy = int(copy_gib * (1 << 30))
    src = torch.empty(nread, dtype=torch.uint8, device=dev)
    src.random_(0, 256)
    dst = torch.empty(ncopy, dtype=torch.uint8, device=dev)
    sink = torch.empty(65536, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()

    def best(fn, moved, wgs_list):
        out = (0.0, 0)
        for wgs in wgs_list:
            fn(wgs)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn(wgs)
            e1.record(stream)
            torch.cuda.synchronize()
            out = max(out, (moved * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, wgs))
        return out

    rd = best(lambda w: probe.read(src, sink, w), nread, (2048, 4096, 8192, 16384, 32768))
    cp = best(lambda w: probe.copy(dst, src[:ncopy], w), 2 * ncopy, (2048, 4096, 8192, 16384))
    # The decode's own byte pattern with no arithmetic: 2048 waves x 128 chunks of 4 KiB K,
    # 4 KiB V and 256 B scales = 2.2146 GB, the bandwidth workload's bytes.
    chunks, groups = 128, 256
    kvb = groups * 8 * chunks * 4096
    pk, pv = src[:kvb], src[kvb:2 * kvb]
    ps = src[2 * kvb:2 * kvb + groups * 8 * chunks * 256]
    pat_bytes = 2 * kvb + ps.numel()
    pt = best(lambda w: probe.pattern(pk, pv, ps, chunks, w, sink), pat_bytes, (groups,))
    # The 4-bit format's byte pattern: the same 2048 x 128 chunks of 4 KiB of rows and 192 B of
    # metadata = 1.1241 GB, the bandwidth workload's bytes in that format.
    rows4 = src[:groups * 8 * chunks * 4096]
    meta4 = src[rows4.numel():rows4.numel() + groups * 8 * chunks * 256]
    pat4_bytes = groups * 8 * chunks * (4096 + 192)
    pt4 = best(lambda w: probe.pattern4(rows4, meta4, chunks, w, sink), pat4_bytes, (groups,))
    del src, dst, sink, pk, pv, ps, rows4, meta4
    torch.cuda.empty_cache()
    return {"read_bytes": nread, "copy_bytes": ncopy, "reps": reps,
            "read_gbs": round(rd[0], 1), "read_workgroups": rd[1],
            "pattern_bytes": pat_bytes, "pattern_gbs": round(pt[0], 1),
            "pattern4_bytes": pat4_bytes, "pattern4_gbs": round(pt4[0], 1),
            "copy_gbs": round(cp[0], 1), "copy_workgroups": cp[1]}


PROFILE_KERNELS = ("tq_flat_kernel", "tq_fused_kernel", "tq_partition_kernel", "tq_merge_kernel",
                   "tq_kv_write_kernel", "tq_flat_kernel[tq4]", "tq_partition_kernel[tq4]",
                   "tq_partition_flat_kernel[tq4]", "probe_pattern_kernel", "probe_pattern4_kernel")
PROFILE_CMD = ("rocprofv3 {what} -d <dir>/{sub} -o {sub} --output-format csv -- "
               "python3 bench.py --workload {wl} --steps 20 --warmup 3 --no-cpu-baseline")


def _csv_rows(path):
    import csv

    with open(path) as f:
        return list(csv.DictReader(f))


def _kernel_key(name: str) -> str:
    """Short kernel name from a full one: the function name, with "[tq4]" for the
    4-bit-format instantiation (last template argument true)."""
    import re

    m = re.search(r"\b((?:tq|probe)_\w+)(?:<([^>]*)>)?", name)
    if not m:
        return name
    key = m.group(1)
    if (m.group(2) or "").replace(" ", "").endswith("true"):
        key += "[tq4]"
    return key


def summarize_rocprof(prof_dir: str, workload: str, out_dir: str = PROFILES) -> None:
    """Turn the rocprofv3 output of three profiled bench runs under `prof_dir`
    (trace/: --kernel-trace --stats; fetch/: --pmc FETCH_SIZE; write/: --pmc
    WRITE_SIZE) into the summaries kept under profiles/: per-kernel duration
    statistics, and HBM bytes per launch of each decode kernel, the counters
    scaled by what they read for the copy probe, whose bytes are known."""
    stats = {}
    for r in _csv_rows(os.path.join(prof_dir, "trace", "trace_kernel_stats.csv")):
        k = _kernel_key(r["Name"])
        st = stats.setdefault(k, {"Calls": 0, "TotalNs": 0.0, "MinNs": float("inf"), "MaxNs": 0.0})
        st["Calls"] += int(r["Calls"])
        st["TotalNs"] += float(r["TotalDurationNs"])
        st["MinNs"] = min(st["MinNs"], float(r["MinNs"]))
        st["MaxNs"] = max(st["MaxNs"], float(r["MaxNs"]))
    for st in stats.values():
        st["AverageNs"] = st["TotalNs"] / st["Calls"]

    def per_kernel(sub, counter):
        vals = {}
        for r in _csv_rows(os.path.join(prof_dir, sub, f"{sub}_counter_collection.csv")):
            if r["Counter_Name"] == counter:
                vals.setdefault(_kernel_key(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return {k: sum(v) / len(v) for k, v in vals.items()}

    fetch = per_kernel("fetch", "FETCH_SIZE")
    write = per_kernel("write", "WRITE_SIZE")
    copy_bytes = 1 << 30  # the probe copies 1 GiB: reads 1 GiB, writes 1 GiB
    f_scale = copy_bytes / (fetch["probe_copy_kernel"] * 1024.0)
    w_scale = copy_bytes / (write["probe_copy_kernel"] * 1024.0)
    sha = kernel_sha()
    os.makedirs(out_dir, exist_ok=True)
    lines = [f"# rocprofv3 kernel statistics, {workload} (bench.py, both decode paths)", "",
             "Commands (run from the repository root; <dir> = an output directory):", "",
             "    " + PROFILE_CMD.format(what="--kernel-trace --stats", sub="trace", wl=workload),
             "    " + PROFILE_CMD.format(what="--pmc FETCH_SIZE", sub="fetch", wl=workload),
             "    " + PROFILE_CMD.format(what="--pmc WRITE_SIZE", sub="write", wl=workload),
             f"    python3 bench.py --summarize-rocprof <dir> --workload {workload}", "",
             f"Kernel source sha256: {sha}", "",
             "| kernel | calls | avg us | min us | max us | FETCH_SIZE KiB/launch | WRITE_SIZE KiB/launch |",
             "|---|---|---|---|---|---|---|"]
    for name in PROFILE_KERNELS + ("probe_read_kernel", "probe_copy_kernel"):
        if name not in stats:
            continue
        st = stats[name]
        lines.append(f"| {name} | {st['Calls']} | {float(st['AverageNs']) / 1e3:.1f} | "
                     f"{float(st['MinNs']) / 1e3:.1f} | {float(st['MaxNs']) / 1e3:.1f} | "
                     f"{fetch.get(name, float('nan')):.0f} | {write.get(name, float('nan')):.0f} |")
    lines += ["", f"Counter calibration with the 1 GiB copy probe: bytes = FETCH_SIZE x 1024 x "
              f"{f_scale:.4f}, WRITE_SIZE x 1024 x {w_scale:.4f}.", ""]
    for name in ("tq_flat_kernel", "tq_fused_kernel", "tq_partition_kernel", "tq_flat_kernel[tq4]",
                 "tq_partition_kernel[tq4]", "tq_partition_flat_kernel[tq4]"):
        if name not in fetch or name not in write:
            continue
        fb = fetch[name] * 1024.0 * f_scale
        wb = write[name] * 1024.0 * w_scale
        rec = {"kernel": name, "workload": workload, "kernel_source_sha256": sha,
               "fetch_bytes_per_launch": round(fb), "write_bytes_per_launch": round(wb),
               "hbm_bytes_per_launch": round(fb + wb),
               "avg_duration_us": round(float(stats[name]["AverageNs"]) / 1e3, 2),
               "fetch_scale": round(f_scale, 5), "write_scale": round(w_scale, 5),
               "source": f"profiles/rocprof_{workload}.md"}
        fname = name.replace("[tq4]", "_tq4")
        with open(os.path.join(out_dir, f"traffic_{fname}_{workload}.json"), "w") as f:
            json.dump(rec, f, indent=1)
        lines.append(f"- {name}: {fb / 1e9:.4f} GB fetched + {wb / 1e9:.4f} GB written per launch")
    with open(os.path.join(out_dir, f"rocprof_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


# Two rocprofv3 --pmc passes (each within the per-pass limits of 8 SQ and 2 GRBM
# counters) for the occupancy, issue and stall figures of the decode kernels.
COUNTER_PASSES = (
    ("pmc1", ("SQ_WAVES", "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_INSTS_VALU", "SQ_ACTIVE_INST_VALU",
              "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_LDS", "GRBM_GUI_ACTIVE")),
    ("pmc2", ("SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY",
              "SQ_INSTS_SALU", "SQ_ACTIVE_INST_ANY", "GRBM_GUI_ACTIVE")),
)
COUNTER_KERNELS = ("tq_flat_kernel", "tq_partition_kernel", "tq_merge_kernel", "tq_kv_write_kernel",
                   "tq_flat_kernel[tq4]", "tq_partition_flat_kernel[tq4]", "tq_partition_kernel[tq4]",
                   "probe_pattern_kernel", "probe_pattern4_kernel")
MI355X_XCDS, MI355X_CUS, MI355X_SIMDS = 8, 256, 1024


def summarize_counters(prof_dir: str, workload: str, out_dir: str = PROFILES) -> None:
    """Write profiles/counters_<workload>.md from the COUNTER_PASSES runs under prof_dir:
    per kernel, the average over its dispatches of every counter, and ratios derived from
    them (cycles = GRBM_GUI_ACTIVE / 8 XCDs; quad-cycle counters times 4)."""
    vals = {}
    for sub, _ in COUNTER_PASSES:
        for r in _csv_rows(os.path.join(prof_dir, sub, f"{sub}_counter_collection.csv")):
            k = _kernel_key(r["Kernel_Name"])
            vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    avg = {k: {c: sum(v) / len(v) for c, v in d.items()} for k, d in vals.items()}
    names = [c for _, cs in COUNTER_PASSES for c in cs if c != "GRBM_GUI_ACTIVE"]
    lines = [f"# rocprofv3 SQ counters, {workload} (bench.py, every decode kernel)", "",
             "Commands (run from the repository root; <dir> = an output directory):", ""]
    for sub, cs in COUNTER_PASSES:
        lines.append("    " + PROFILE_CMD.format(what="--pmc " + " ".join(cs), sub=sub, wl=workload))
    lines += [f"    python3 bench.py --summarize-counters <dir> --workload {workload}", "",
              f"Kernel source sha256: {kernel_sha()}", "",
              "Averages per dispatch (counters as rocprofv3 reports them, summed over the device).", "",
              "| kernel | GRBM_GUI_ACTIVE | " + " | ".join(names) + " |",
              "|---|" + "---|" * (len(names) + 1)]
    for k in COUNTER_KERNELS:
        if k not in avg:
            continue
        a = avg[k]
        lines.append(f"| {k} | {a.get('GRBM_GUI_ACTIVE', float('nan')):.4g} | " +
                     " | ".join(f"{a.get(c, float('nan')):.4g}" for c in names) + " |")
    lines += ["", "Derived (cycles = GRBM_GUI_ACTIVE / 8, the kernel's duration in one XCD's clocks; "
              "SQ_WAVE_CYCLES and SQ_ACTIVE_INST_VALU count quad-cycles):", "",
              "| kernel | cycles | waves per SIMD (4 SQ_WAVE_CYCLES / 1024 SIMDs / cycles) | "
              "VALU busy (4 SQ_ACTIVE_INST_VALU / 1024 / cycles) | MFMA busy "
              "(SQ_VALU_MFMA_BUSY_CYCLES / 1024 / cycles) | LDS bank-conflict cycles "
              "(SQ_LDS_BANK_CONFLICT / 256 CUs / cycles) | VALU instructions per wave |",
              "|---|---|---|---|---|---|---|"]
    for k in COUNTER_KERNELS:
        if k not in avg:
            continue
        a = avg[k]
        cyc = a.get("GRBM_GUI_ACTIVE", float("nan")) / MI355X_XCDS
        pct = lambda x: f"{100 * x:.1f} %"  # noqa: E731
        lines.append(
            f"| {k} | {cyc:.4g} | {4 * a.get('SQ_WAVE_CYCLES', float('nan')) / MI355X_SIMDS / cyc:.2f} | "
            f"{pct(4 * a.get('SQ_ACTIVE_INST_VALU', float('nan')) / MI355X_SIMDS / cyc)} | "
            f"{pct(a.get('SQ_VALU_MFMA_BUSY_CYCLES', float('nan')) / MI355X_SIMDS / cyc)} | "
            f"{pct(a.get('SQ_LDS_BANK_CONFLICT', float('nan')) / MI355X_CUS / cyc)} | "
            f"{a.get('SQ_INSTS_VALU', float('nan')) / a.get('SQ_WAVES', float('nan')):.0f} |")
    os.makedirs(out_dir, exist_ok=True)
    with open(os.path.join(out_dir, f"counters_{workload}.md"), "w") as f:
        f.write("\n".join(lines) + "\n")
    print("\n".join(lines))


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="w4_s128_ctx8k")
    ap.add_argument("--kv-layout", default="head", choices=("head", "slot"),
                    help="order of the cache rows in a block: head-major (default) or the page's "
                         "slot-major data region")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-probe", action="store_true", help="skip the HBM read/copy probe")
    ap.add_argument("--summarize-rocprof", metavar="DIR",
                    help="write profiles/ summaries from rocprofv3 output under DIR and exit")
    ap.add_argument("--summarize-counters", metavar="DIR",
                    help="write profiles/counters_<workload>.md from the SQ counter passes under DIR")
    args = ap.parse_args()
    if args.summarize_rocprof:
        summarize_rocprof(args.summarize_rocprof, args.workload)
        return 0
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.workload)
        return 0
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): this library runs "
              "its decode on a single MI355X; sharding across GPUs is not implemented",
              file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    import paged_gqa_decode_amd as tq
    import workloads

    wl = workloads.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    probe_res = None
    if not args.no_probe:
        probe_res = hbm_probe(dev)
        log(f"[bench] HBM probe: read {probe_res['read_gbs']} GB/s, copy {probe_res['copy_gbs']} GB/s, "
            f"decode byte pattern without arithmetic {probe_res['pattern_gbs']} GB/s (4-bit: "
            f"{probe_res['pattern4_gbs']} GB/s)")
    log(f"[bench] generating {wl.name} on {dev}")
    inp = workloads.make_inputs(wl, device=dev, kv_layout=args.kv_layout)
    torch.cuda.synchronize()
    S, Hkv, QG, G = wl.num_seqs, wl.num_kv_heads, wl.query_group_size, wl.tile_groups_per_partition
    P = inp.num_partitions
    maxlen = int(inp.seq_lens.max().item())
    kv_bytes = inp.kv_bytes()
    part = tq.alloc_partials(S, Hkv, P, QG, dev)
    out = torch.empty((S, Hkv * QG, 128), dtype=torch.bfloat16, device=dev)
    workspace = tq.alloc_fused_workspace(S, Hkv, QG, maxlen, dev)
    stream = torch.cuda.current_stream()

    def dec():
        tq.tq_decode(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, inp.seq_lens,
                     part, Hkv, QG, wl.kv_block_size, G, inp.softmax_scale, num_partitions=P,
                     max_seq_len=maxlen, num_blocks=inp.num_blocks, kv_layout=args.kv_layout,
                     stream=stream)

    def red():
        tq.tq_decode_reduce(part, inp.seq_lens, out, Hkv, QG, G, num_partitions=P,
                            max_seq_len=maxlen, stream=stream)

    def fused():
        tq.tq_decode_fused(inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables,
                           inp.seq_lens, out, Hkv, QG, wl.kv_block_size, G, inp.softmax_scale,
                           num_partitions=P, max_seq_len=maxlen, num_blocks=inp.num_blocks,
                           workspace=workspace, kv_layout=args.kv_layout, stream=stream)

    K = args.steps

    def timed(*kernels):
        """Average ms of K back-to-back runs of `kernels` (one step), between two HIP events
        on the launch stream with nothing else enqueued in between."""
        for _ in range(args.warmup):
            for k in kernels:
                k()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(K):
            for k in kernels:
                k()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / K

    # Per-kernel averages: each kernel alone, K launches; then the step itself.
    # The fused step is one launch: its kernel average is the step time itself, from the
    # same timed region as the headline.
    paths = {"two_kernel": {"k1_avg": timed(dec), "k2_avg": timed(red), "ms_per_step": timed(dec, red)}}
    t_fused = timed(fused)
    paths["fused"] = {"k1_avg": t_fused, "k2_avg": 0.0, "ms_per_step": t_fused}
    for name, pth in paths.items():
        log(f"[bench] {wl.name} {name}: step {pth['ms_per_step'] * 1e3:.1f} us "
            f"({kv_bytes / (pth['ms_per_step'] * 1e-3) / 1e9:.0f} GB/s); first kernel "
            f"{pth['k1_avg'] * 1e3:.1f} us, second kernel {pth['k2_avg'] * 1e3:.1f} us")
    # Single steps, each timed alone by two events on the launch stream (the event pair adds a
    # few microseconds to each interval): "cold" with a 1 GiB read before each step (clean
    # evictions of the L2s and the 256 MB last-level cache, nothing left to write back), and
    # "warm" the same way without it.  Reported next to the back-to-back figures; for the
    # 2.2 GB bandwidth workload the two agree.
    from paged_gqa_decode_amd import probe as _probe
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    flush_sink = torch.empty(4096, dtype=torch.int32, device=dev)

    def single(*kernels, evict, reps=20):
        times = []
        for i in range(reps + 2):
            if evict:
                _probe.read(flush, flush_sink, 4096, stream=stream)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for k in kernels:
                k()
            e1.record(stream)
            torch.cuda.synchronize()
            if i >= 2:
                times.append(e0.elapsed_time(e1))
        times.sort()
        n = len(times)
        return {"median": round(times[n // 2] * 1e3, 2), "p10": round(times[n // 10] * 1e3, 2),
                "p90": round(times[(9 * n) // 10] * 1e3, 2)}

    single_us = {"cold": {"two_kernel": single(dec, red, evict=True), "fused": single(fused, evict=True)},
                 "warm": {"two_kernel": single(dec, red, evict=False), "fused": single(fused, evict=False)}}
    del flush, flush_sink
    torch.cuda.empty_cache()
    log(f"[bench] {wl.name} single steps (median of 20): cold (1 GiB read before each) "
        f"two-kernel {single_us['cold']['two_kernel']['median']} us, fused {single_us['cold']['fused']['median']} us; "
        f"warm two-kernel {single_us['warm']['two_kernel']['median']} us, fused {single_us['warm']['fused']['median']} us")
    head = min(paths, key=lambda n: paths[n]["ms_per_step"])
    ms_per_step = paths[head]["ms_per_step"]
    k1_avg = paths[head]["k1_avg"]
    step_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    k1_gbs = kv_bytes / (k1_avg * 1e-3) / 1e9
    log(f"[bench] headline path {head}: step {step_gbs:.0f} GB/s ({100 * step_gbs / HBM_PEAK_GBS:.1f}% "
        f"of peak); {KERNEL_NAMES[head]} {k1_gbs:.0f} GB/s ({100 * k1_gbs / HBM_PEAK_GBS:.1f}% of peak)")

    res = {
        "metric": METRIC,
        "value": round(step_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * step_gbs / HBM_PEAK_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "num_seqs": S, "num_kv_heads": Hkv, "query_group_size": QG,
                   "head_dim": 128, "context_tokens": maxlen, "kv_block_size": wl.kv_block_size,
                   "num_partitions": P, "tile_groups_per_partition": G, "path": head,
                   "kv_layout": args.kv_layout,
                   "kv_format": "e4m3fn codes + fp32 scale per (token, kv head) for K and V",
                   "kv_bytes_per_step": kv_bytes},
        "paths_us": {
            "two_kernel": {"step": round(paths["two_kernel"]["ms_per_step"] * 1e3, 2),
                           "tq_decode": round(paths["two_kernel"]["k1_avg"] * 1e3, 2),
                           "tq_decode_reduce": round(paths["two_kernel"]["k2_avg"] * 1e3, 2)},
            "fused": {"step": round(paths["fused"]["ms_per_step"] * 1e3, 2),
                      "tq_decode_fused": round(paths["fused"]["k1_avg"] * 1e3, 2)},
        },
        "single_step_us": single_us,
        "roofline": {"bound": "hbm", "achieved": round(k1_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(k1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, head), "kernel": KERNEL_NAMES[head],
                     "bytes_per_launch": kv_bytes},
    }
    if probe_res is not None:
        res["hbm_probe"] = probe_res
        res["roofline"]["frac_of_probe_read"] = round(k1_gbs / probe_res["read_gbs"], 4)
        res["roofline"]["frac_of_decode_pattern"] = round(k1_gbs / probe_res["pattern_gbs"], 4)
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on a sample (cpu_baseline)")
        res["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        res["cpu_baseline"] = None

    # The KV-cache writer (the step that fills the cache): a prefill-sized batch of new
    # tokens scattered into random slots of the same pool; bytes per (token, kv head) row =
    # 512 read (bf16 K and V) + 264 written (fp8 codes and two fp32 scales).
    T = 16384
    wkey = workloads.stream_key(wl.seed, "writer")
    new_rows = workloads.random_normal(wkey, 0, 2 * T * Hkv * 128, dev).to(torch.bfloat16)
    k_new, v_new = new_rows.view(2, T, Hkv, 128).unbind(0)
    slots = workloads.random_permutation(wkey, inp.num_blocks * wl.kv_block_size, dev)[:T]
    slots = slots.to(torch.int32)
    write = lambda: tq.tq_kv_write(k_new, v_new, slots, inp.k_cache, inp.v_cache,  # noqa: E731
                                   inp.kv_scales, kv_layout=args.kv_layout, stream=stream)
    w_ms = timed(write)
    w_bytes = T * Hkv * (512 + 264)
    res["kv_writer"] = {"tokens": T, "num_kv_heads": Hkv, "us": round(w_ms * 1e3, 2),
                        "GBps": round(w_bytes / (w_ms * 1e-3) / 1e9, 1), "bytes_per_launch": w_bytes}
    log(f"[bench] kv writer: {T} tokens x {Hkv} heads in {w_ms * 1e3:.1f} us "
        f"({res['kv_writer']['GBps']} GB/s)")

    # The 4-bit record format on the same workload shape (same lengths and tables): its
    # bytes per (token, kv head) are 128 + 6, so the comparison that matters is tokens/s.
    del k_new, v_new, slots, part, workspace
    inp_fp8_tokens = int(inp.seq_lens.to(torch.int64).sum().item()) * Hkv
    del inp
    torch.cuda.empty_cache()
    log(f"[bench] generating {wl.name} in the 4-bit record format")
    t4 = workloads.make_inputs_tq4(wl, device=dev, kv_layout=args.kv_layout)
    part4 = tq.alloc_partials(S, Hkv, P, QG, dev)
    ws4 = tq.alloc_fused_workspace(S, Hkv, QG, maxlen, dev)
    bytes4 = t4.kv_bytes()

    def dec4():
        tq.tq4_decode(t4.q, t4.cache, t4.centroids, t4.block_tables, t4.seq_lens, part4, Hkv, QG,
                      wl.kv_block_size, G, t4.softmax_scale, num_partitions=P, max_seq_len=maxlen,
                      kv_layout=args.kv_layout, stream=stream)

    def fused4():
        tq.tq4_decode_fused(t4.q, t4.cache, t4.centroids, t4.block_tables, t4.seq_lens, out, Hkv,
                            QG, wl.kv_block_size, G, t4.softmax_scale, num_partitions=P,
                            max_seq_len=maxlen, workspace=ws4, kv_layout=args.kv_layout,
                            stream=stream)

    def red4():
        tq.tq_decode_reduce(part4, t4.seq_lens, out, Hkv, QG, G, num_partitions=P,
                            max_seq_len=maxlen, stream=stream)

    t_two4 = timed(dec4, red4)
    t_fused4 = timed(fused4)
    best4 = min(t_two4, t_fused4)
    tok_s = inp_fp8_tokens / (best4 * 1e-3)
    tok_s_fp8 = inp_fp8_tokens / (ms_per_step * 1e-3)
    res["tq4"] = {"format": "4-bit record: 16-centroid K indices + fp16 K norm, 4-bit V + fp16 "
                            "scale and zero point (134 B per token and kv head)",
                  "us_per_step": round(best4 * 1e3, 2),
                  "paths_us": {"two_kernel": round(t_two4 * 1e3, 2), "fused": round(t_fused4 * 1e3, 2)},
                  "GBps": round(bytes4 / (best4 * 1e-3) / 1e9, 1),
                  "pct_of_hbm_peak": round(100 * bytes4 / (best4 * 1e-3) / 1e9 / HBM_PEAK_GBS, 2),
                  "bytes_per_step": bytes4,
                  "token_heads_per_s": round(tok_s, 1),
                  "vs_fp8_token_heads_per_s": round(tok_s / tok_s_fp8, 3)}
    if probe_res:
        res["tq4"]["frac_of_decode_pattern"] = round(
            res["tq4"]["GBps"] / probe_res["pattern4_gbs"], 4)
    log(f"[bench] 4-bit format: step {best4 * 1e3:.1f} us ({res['tq4']['GBps']} GB/s, "
        f"{res['tq4']['pct_of_hbm_peak']}% of peak), {tok_s / 1e9:.1f} G token-heads/s = "
        f"{res['tq4']['vs_fp8_token_heads_per_s']}x the fp8 step")
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
