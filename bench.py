#!/usr/bin/env python3
"""Benchmark of libks, the KS matmul path, on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one pass of the hot path over one batch: plan + launch of the KS
kernel(s) for the workload (ks_matmul for a single factor, ks_chain_matmul
for a chain) on synthetic seeded inputs already resident in HBM. K steps are
timed between two device synchronisations; several copies of the inputs and
outputs rotate so that each step reads data that is not in the 256 MB
Infinity Cache or the L2 (the working set of a step is re-read only after
more than 288 MB of other traffic).

Default workload: the largest configuration, the 65,536-point butterfly
chain -- four factors (16^k, 16, 16, 16^(3-k)), k = 0..3, on 4,096 rows, fp32
(`--dtype bf16`: bf16 X and weights, fp32 accumulation and outputs) -- run
through ks_chain_matmul with fusion where the planner finds it. Other
workloads (`--workload vit_mlp`, `gpt2_mlp`, ...) are available.

Printed: one JSON line with
  value      algorithmic GB/s of a step as run (each launch group reads its
             input and weights and writes its output once) over the wall time
             of the K timed steps;
  roofline   the dominant kernel: the launch group that takes the most time,
             timed on its own with HIP events on the launch stream (back to
             back, rotated inputs), its algorithmic bytes per launch over its
             average launch duration; also the whole step against the bytes
             it moves and against the fully fused minimum |X| + |Y| + weights,
             and a plain device copy's rate as the practical ceiling;
  per_group / per_factor   every launch group, and every factor as a single
             launch, timed the same way;
  cpu_baseline   the fp64 oracle timed on this host's cores on a bounded
             sample of the same workload;
  other_configs  (default run only; --headline-only skips it) the other
             configurations timed the same way and summarised: the ViT
             factor, the GPT-2 chain fused and one launch per factor, the
             butterfly with bf16 inputs, the 65,536-point radix-2 and
             radix-4 butterflies (fused and one launch per factor), and
             the 51-pattern square sweep.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, published
FP32_PEAK_TFLOPS = 157.3         # MI355X fp32 (vector and matrix), published
BF16_PEAK_TFLOPS = 2516.6        # MI355X bf16 dense MFMA, published
CACHE_BYTES = (256 + 32) * 2 ** 20   # Infinity Cache + 8 x 4 MB L2
METRIC = "KS matmul achieved GB/s & TFLOP/s as % of roofline, fp32, 1×MI355X"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


# Kernel sources each counted workload runs, beside the C ABI (ks_api.cpp)
# and the headers: its traffic counters stay valid while these are unchanged.
# Workloads not listed are keyed on every source.
WORKLOAD_SOURCES = {
    "butterfly65536": ("ks_mfma.hip", "ks_slab.hip", "ks_valu.hip"),
    "vit_mlp": ("ks_mfma.hip",),
    "gpt2_mlp": ("ks_fused.hip",),
    "gpt2_mlp:nofuse": ("ks_mfma.hip", "ks_valu.hip"),
    "monarch_n1024": ("ks_monarch.hip",),
    "radix4_n4096": ("ks_resident.hip", "ks_rowchain.hip", "ks_digitchain.hip"),
    "radix2_n1024": ("ks_resident.hip", "ks_rowchain.hip", "ks_digitchain.hip"),
    "radix2_n65536": ("ks_rowchain.hip", "ks_resident.hip"),
    "radix4_n65536": ("ks_rowchain.hip", "ks_resident.hip"),
    "radix2_n16384": ("ks_rowchain.hip", "ks_resident.hip"),
}


# single factors of the square sweep: the kernels the planner picks among
SQUARE_SOURCES = ("ks_mfma.hip", "ks_valu.hip", "ks_col.hip", "ks_generic.hip")


def kernel_source_hash(workload: str = "", no_fuse: bool = False) -> str:
    csrc = os.path.join(ROOT, "kronecker_sparse_structured_amd", "csrc")
    names = sorted(os.listdir(csrc))
    used = WORKLOAD_SOURCES.get(workload + (":nofuse" if no_fuse else ""), WORKLOAD_SOURCES.get(workload))
    if used is None and workload.startswith("square_"):
        used = SQUARE_SOURCES
    if used is not None:
        names = [n for n in names if n.endswith(".h") or n == "ks_api.cpp" or n in used]
    h = hashlib.sha256()
    for name in names:
        if name.endswith((".hip", ".cpp", ".h")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    with open(os.path.join(ROOT, "include", "ks.h"), "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="butterfly65536")
    ap.add_argument("--dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "valu", "mfma", "mfma_lds", "col"])
    ap.add_argument("--no-fuse", action="store_true", help="chains: one launch per factor")
    ap.add_argument("--no-rotate", action="store_true", help="reuse one input/output set (warm caches)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target CPU time of the oracle leg")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle leg")
    ap.add_argument("--no-factors", action="store_true",
                    help="chains: skip timing each factor on its own (profiler runs)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain device copy of known size (for counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every pattern of the square sweep (n = 4096, 16,384 rows) and print "
                         "one line per pattern plus a JSON summary; not the single-line contract run")
    ap.add_argument("--comparator", action="store_true",
                    help="with --sweep (fp32): also time the permute / batched GEMM / permute formulation "
                         "(torch permute copies and torch.bmm) on the same inputs and report the speedup")
    ap.add_argument("--energy", action="store_true",
                    help="GPU energy per call (amdsmi energy counter over ~2 s loops) of the fused kernel and "
                         "of the permute / batched GEMM / permute comparator, fp32; one JSON line")
    ap.add_argument("--backward", action="store_true",
                    help="time the gradients (ks_matmul_dx, ks_matmul_dw) of every factor of the "
                         "workload and print one JSON line; not the contract run")
    ap.add_argument("--families", action="store_true",
                    help="with --sweep: also time every kernel family (and store schedule) that runs each "
                         "pattern and report the fastest (the data the planner's table is fitted on)")
    ap.add_argument("--comparator-only", action="store_true",
                    help="run only the permute / batched GEMM / permute comparator on a single-factor "
                         "workload (for rocprofv3 counters); one JSON line")
    ap.add_argument("--ingest-comparator", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="HBM bytes per call of the comparator from two --comparator-only counter runs "
                         "(same --steps / --warmup)")
    ap.add_argument("--workload-factors", action="store_true",
                    help="with --sweep: also time each factor of the butterfly, ViT and GPT-2 workloads alone, "
                         "at the workload's batch (table rows for the launches those chains make)")
    ap.add_argument("--copy-ceiling", action="store_true",
                    help="time a plain device copy at 64 MiB .. 4 GiB and print one JSON line")
    ap.add_argument("--sweep-text", metavar="PATH",
                    help="with --sweep: also write the per-pattern table as text to PATH; with --from-log: "
                         "write it from a saved --sweep output instead (no GPU)")
    ap.add_argument("--from-log", metavar="LOG", help="a saved --sweep output (see --sweep-text)")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other configurations' summary (other_configs) of the default run; "
                         "profiler runs use it so that only the headline workload's kernels are traced")
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                         "`--calib-copy` run into profiles/traffic_counters.json and exit")
    return ap.parse_args()


CALIB_BYTES = 256 * 2 ** 20      # the --calib-copy device copy reads and writes this many bytes


def ingest_counters(args) -> int:
    """HBM bytes per launch group (and per step) of the workload's KS kernels
    from two counter runs of the same command (`--no-factors --calib-copy`).
    FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are each scaled by what the
    same counter reads for the calibration copy (CALIB_BYTES read and
    written). The KS dispatches come in whole steps, one per launch group in
    group order, so group g's bytes are the mean over the dispatches at
    positions g, g + groups, ..."""
    import csv
    from collections import defaultdict
    from kronecker_sparse_structured_amd import datagen, libks

    wl = datagen.get(args.workload)
    if len(wl.patterns) > 1:
        dt = libks.DTYPE_BF16 if args.dtype == "bf16" else libks.DTYPE_F32
        flags = libks.CHAIN_NO_FUSE if args.no_fuse else libks.CHAIN_AUTO
        per_step = len(libks.ks_chain_groups(wl.patterns, wl.batch, dt, flags))
    else:
        per_step = 1

    def per_dispatch(path, counter):
        vals = defaultdict(float)
        names = {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] != counter:
                    continue
                key = r["Dispatch_Id"]
                vals[key] += float(r["Counter_Value"])
                names[key] = r["Kernel_Name"]
        return vals, names

    out = {}
    per_group = {}
    for path, counter in ((args.ingest_counters[0], "FETCH_SIZE"), (args.ingest_counters[1], "WRITE_SIZE")):
        vals, names = per_dispatch(path, counter)
        ks_ids = sorted((k for k, n in names.items() if "ks::" in n), key=int)
        last_ks = max((int(k) for k in ks_ids), default=-1)
        # the calibration copies run after the timed KS launches (earlier
        # copies are the bench's input replication, of other sizes)
        calib = [vals[k] for k, n in names.items()
                 if ("copyBuffer" in n or "copy_kernel" in n) and int(k) > last_ks]
        if not calib or not ks_ids:
            print("no calibration copy or no KS dispatch in %s" % path, file=sys.stderr)
            return 1
        if len(ks_ids) % per_step != 0:
            print("%d KS dispatches is not a whole number of %d-launch steps" % (len(ks_ids), per_step),
                  file=sys.stderr)
            return 1
        steps = len(ks_ids) // per_step
        factor = CALIB_BYTES / (max(calib) * 1024.0)
        per_group[counter] = [sum(vals[ks_ids[i]] for i in range(g, len(ks_ids), per_step)) / steps * 1024.0 * factor
                              for g in range(per_step)]
        out[counter.lower() + "_factor"] = round(factor, 4)
        out[counter.lower() + "_kib_per_step"] = round(sum(vals[k] for k in ks_ids) / steps, 1)
        out[counter.lower() + "_launches"] = len(ks_ids)
    key = traffic_key(args)
    db = {}
    if os.path.exists(TRAFFIC_FILE):
        db = json.load(open(TRAFFIC_FILE))
    out["group_bytes"] = [int(f + w) for f, w in zip(per_group["FETCH_SIZE"], per_group["WRITE_SIZE"])]
    out["bytes_per_step"] = int(sum(out["group_bytes"]))
    out["launches_per_step"] = per_step
    out["source_hash"] = kernel_source_hash(args.workload, args.no_fuse)
    db[key] = out
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(db, f, indent=1, sort_keys=True)
    print(json.dumps({key: out}))
    return 0


WARM_SECONDS = 0.2


def warm_up(step, min_steps, torch) -> int:
    """Run step(i) at least min_steps times and until about WARM_SECONDS of
    GPU work have passed; returns the number of steps run."""
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(max(min_steps, 1)):
            step(n)
            n += 1
        torch.cuda.synchronize()
        if n >= min_steps and time.perf_counter() - t0 >= WARM_SECONDS:
            return n


def factor_bytes(p, x_bytes, w_bytes, batch):
    a, b, c, d = p
    return x_bytes * batch * a * c * d + 4 * batch * a * b * d + w_bytes * a * b * c * d


def main():
    args = parse()
    if args.ingest_counters:
        return ingest_counters(args)
    if args.ingest_comparator:
        return ingest_comparator_counters(args)
    if args.from_log:
        if not args.sweep_text:
            print("--from-log needs --sweep-text PATH", file=sys.stderr)
            return 2
        with open(args.from_log) as f:
            summary = [json.loads(l) for l in f if l.startswith("{") and '"sweep"' in l][-1]
        write_sweep_text(summary, args.sweep_text)
        return 0
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)
    if args.copy_ceiling:
        return copy_ceilings(args)
    if args.comparator_only:
        return comparator_only(args)
    if args.backward:
        return backward(args)
    if args.energy:
        return energy(args)

    import numpy as np
    import torch
    from kronecker_sparse_structured_amd import datagen, libks

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = datagen.get(args.workload)
    bf16 = args.dtype == "bf16"
    chain = len(wl.patterns) > 1
    X, Ws = datagen.draw(wl)

    def put(a, as_bf16):
        if as_bf16:
            return torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(a).to(dev)

    xb = 2 if bf16 else 4
    wbytes = 2 if bf16 else 4
    batch = wl.batch
    n_out = wl.n_out
    step_bytes = xb * batch * wl.n_in + 4 * batch * n_out
    Wt = [put(W, bf16) for W in Ws]
    ws_bytes = 0
    flags = libks.CHAIN_NO_FUSE if args.no_fuse else libks.CHAIN_AUTO
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    if chain:
        ws_bytes = libks.ks_chain_workspace_size(wl.patterns, batch, dt, flags)
    working = step_bytes + 2 * ws_bytes
    nset = 1 if args.no_rotate else max(2, int(np.ceil(CACHE_BYTES / working)) + 1)
    Xt = [put(X, bf16)]
    for _ in range(nset - 1):
        Xt.append(Xt[0].clone())
    Yt = [torch.empty((batch, n_out), dtype=torch.float32, device=dev) for _ in range(nset)]
    wst = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None for _ in range(nset)]
    del X

    # launch groups of one step (a single factor is one group) and their
    # algorithmic bytes as run: each group reads its input and writes its
    # output once (fp32 between groups) and reads its weights once
    flops = sum(2 * batch * datagen.nnz(p) for p in wl.patterns)
    groups = libks.ks_chain_groups(wl.patterns, batch, dt, flags) if chain else [[0]]
    group_bytes = []
    x_sz = xb
    for grp in groups:
        gb = x_sz * batch * datagen.n_in(wl.patterns[grp[0]]) + 4 * batch * datagen.n_out(wl.patterns[grp[-1]])
        gb += sum(wbytes * datagen.nnz(wl.patterns[k]) for k in grp)
        group_bytes.append(gb)
        x_sz = 4
    bytes_run = sum(group_bytes)
    bytes_min = step_bytes + sum(wbytes * datagen.nnz(p) for p in wl.patterns)

    stream = torch.cuda.current_stream(dev)

    # The timed loop calls the C entry points with arguments marshalled
    # beforehand, so that the host enqueues launches faster than the GPU
    # runs them and the stream never idles between steps.
    lib = libks.load()
    sp = ctypes.c_void_p(int(stream.cuda_stream))
    if chain:
        pats = (libks.ks_pattern_t * len(wl.patterns))(*[libks.ks_pattern_t(*p) for p in wl.patterns])
        wptrs = (ctypes.c_void_p * len(Wt))(*[w.data_ptr() for w in Wt])
        calls = [(lib.ks_chain_matmul,
                  (pats, len(wl.patterns), wptrs, ctypes.c_void_p(Xt[k].data_ptr()),
                   ctypes.c_void_p(Yt[k].data_ptr()), batch, dt,
                   ctypes.c_void_p(wst[k].data_ptr() if wst[k] is not None else None), ws_bytes, flags, sp))
                 for k in range(nset)]
    else:
        opt = libks.ks_options_t()
        opt.kernel = libks.KERNELS[args.kernel]
        pat = libks.ks_pattern_t(*wl.patterns[0])
        calls = [(lib.ks_matmul_ex,
                  (pat, ctypes.c_void_p(Wt[0].data_ptr()), ctypes.c_void_p(Xt[k].data_ptr()),
                   ctypes.c_void_p(Yt[k].data_ptr()), batch, dt, sp, ctypes.byref(opt)))
                 for k in range(nset)]

    def step(i):
        fn, a = calls[i % nset]
        st = fn(*a)
        if st != 0:
            raise libks.KSError(st, "bench step")

    # W warm-up steps, and more until the GPU has been busy for about
    # WARM_SECONDS: clocks ramp up over milliseconds after an idle spell
    warm_steps = warm_up(step, args.warmup, torch)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # average GPU time of one step, from HIP events on the launch stream
    # around the timed launches
    mean_ms = ev0.elapsed_time(ev1) / args.steps

    value = bytes_run * args.steps / wall / 1e9
    peak_flops = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    tflops = flops / (mean_ms * 1e-3) / 1e12

    # Each launch group of a chain timed on its own: back-to-back launches of
    # that group's kernel on inputs of its shape, HIP events on the launch
    # stream. The dominant kernel is the group that takes the most time; the
    # roofline is its algorithmic bytes (or flops) per launch over its
    # average launch duration.
    per_group = None
    if chain and not args.no_factors and not args.calib_copy:
        per_group = time_groups(args, wl, groups, group_bytes, Wt, Xt[0], bf16, flags, lib, sp, stream, torch,
                                np, datagen, libks)
    if per_group:
        dom = max(range(len(per_group)), key=lambda g: per_group[g]["ms"])
        dom_ms, dom_bytes = per_group[dom]["ms"], group_bytes[dom]
        dom_flops = sum(2 * batch * datagen.nnz(wl.patterns[k]) for k in groups[dom])
        dom_label = per_group[dom]["kernel"]
    else:
        dom = 0 if not chain else None
        dom_ms, dom_bytes, dom_flops = mean_ms, bytes_run, flops
        dom_label = (libks.ks_plan_describe(wl.patterns[0], batch, dt) if not chain
                     else "whole step (launch groups not timed on their own)")
    dom_gbs = dom_bytes / (dom_ms * 1e-3) / 1e9
    dom_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    bound = "hbm" if dom_bytes / (HBM_PEAK_GBS * 1e9) >= dom_flops / (peak_flops * 1e12) else "mfma"
    t_roof = max(dom_bytes / (HBM_PEAK_GBS * 1e9), dom_flops / (peak_flops * 1e12))

    traffic = None
    if os.path.exists(TRAFFIC_FILE) and dom is not None:
        try:
            rec = json.load(open(TRAFFIC_FILE)).get(traffic_key(args))
            if (rec and rec.get("source_hash") == kernel_source_hash(args.workload, args.no_fuse)
                    and len(rec.get("group_bytes", [])) > dom):
                traffic = rec["group_bytes"][dom]
        except (ValueError, OSError):
            traffic = None

    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    roofline = {
        "bound": bound,
        "achieved": round(dom_gbs if bound == "hbm" else dom_tflops, 2),
        "peak": HBM_PEAK_GBS if bound == "hbm" else peak_flops,
        "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
        "frac": round((dom_gbs / HBM_PEAK_GBS) if bound == "hbm" else (dom_tflops / peak_flops), 4),
        "traffic": traffic,
        "kernel": dom_label,
        "launch_ms": round(dom_ms, 5),
        "bytes_per_launch": dom_bytes,
        "flops_per_launch": dom_flops,
        "roofline_time_frac": round(t_roof / (dom_ms * 1e-3), 4),
        # the whole step (every launch group) against the bytes it moves as
        # run, and against the fully fused minimum |X| + |Y| + weights
        "step_frac_as_run": round(bytes_run / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "frac_vs_fused_minimum": round(bytes_min / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    if not args.calib_copy and not args.no_factors:
        roofline["copy_ceiling_gbs"] = copy_ceiling(dev, stream, torch)

    # chains: each factor also timed as a single launch (not fused)
    per_factor = None
    if chain and not args.no_factors and not args.calib_copy:
        per_factor = time_factors(wl, Wt, Xt[0], bf16, lib, sp, stream, torch, np, datagen, libks)

    cpu = None
    if not args.no_cpu:
        # same unit as value: the GPU step's as-run bytes per row
        cpu = cpu_baseline(wl, bf16, args.cpu_seconds, row_bytes=(bytes_run - sum(
            wbytes * datagen.nnz(p) for p in wl.patterns)) / batch)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_min_seconds": WARM_SECONDS,
        "ms_per_step": round(wall * 1e3 / args.steps, 5),
        "kernel_ms_mean": round(mean_ms, 5),
        "tflops": round(tflops, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": wl.name,
            "patterns": [list(p) for p in wl.patterns],
            "batch": batch,
            "n_in": wl.n_in,
            "n_out": n_out,
            "bytes_per_step": bytes_run,
            "bytes_min": bytes_min,
            "flops_per_step": flops,
            "chain_fused": bool(chain and not args.no_fuse),
            "launch_groups": [list(g) for g in groups],
            "kernel": args.kernel if not chain else "chain",
            "plan": chain_plan_text(wl.patterns, batch, dt, flags, bf16) if chain else
                    libks.ks_plan_describe(wl.patterns[0], batch, dt),
            "rotating_sets": nset,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if per_group is not None:
        out["per_group"] = per_group
    if per_factor is not None:
        out["per_factor"] = per_factor
    if (args.workload == "butterfly65536" and args.dtype == "f32" and args.kernel == "auto" and not args.no_fuse
            and not args.no_factors and not args.calib_copy and not args.headline_only):
        del Xt, Yt, wst, Wt, calls
        torch.cuda.empty_cache()
        try:
            out["other_configs"] = other_configs(lib, sp, stream, torch, np, datagen, libks)
        except Exception as e:  # noqa: BLE001
            # the headline line is printed whatever happens to this leg
            out["other_configs"] = {"error": "%s: %s" % (type(e).__name__, e)}
    print(json.dumps(out), flush=True)
    return 0


def time_launches(run, nset, stream, torch, reps=20) -> float:
    """Mean milliseconds of run(i) over reps back-to-back calls on rotated
    sets, after the time-based warm-up; HIP events on the launch stream."""
    warm_up(lambda i: run(i % nset), 3, torch)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(reps):
        run(i % nset)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_workload(wl, bf16, flags, lib, sp, stream, torch, np, datagen, libks, reps=20) -> dict:
    """One workload as the contract run does it (ks_matmul for one factor,
    ks_chain_matmul for a chain) on seeded N(0, 1) device inputs with the
    workload's weight scales, rotated so each call reads from HBM. Returns
    the mean call time and the algorithmic bytes as run and fused."""
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    el = torch.bfloat16 if bf16 else torch.float32
    xb = 2 if bf16 else 4
    batch = wl.batch
    Wt = [(torch.randn(datagen.nnz(p), generator=gen, device=dev) * sg).to(el)
          for p, sg in zip(wl.patterns, wl.sigmas)]
    chain = len(wl.patterns) > 1
    groups = libks.ks_chain_groups(wl.patterns, batch, dt, flags) if chain else [[0]]
    bytes_run, x_sz = 0, xb
    for grp in groups:
        bytes_run += x_sz * batch * datagen.n_in(wl.patterns[grp[0]]) + 4 * batch * datagen.n_out(
            wl.patterns[grp[-1]]) + sum(xb * datagen.nnz(wl.patterns[k]) for k in grp)
        x_sz = 4
    wsum = sum(xb * datagen.nnz(p) for p in wl.patterns)
    bytes_min = xb * batch * wl.n_in + 4 * batch * wl.n_out + wsum
    ws_bytes = libks.ks_chain_workspace_size(wl.patterns, batch, dt, flags) if chain else 0
    nset = max(2, int(np.ceil(CACHE_BYTES / (bytes_min + 2 * ws_bytes))) + 1)
    Xt = [torch.randn((batch, wl.n_in), generator=gen, device=dev).to(el)]
    for _ in range(nset - 1):
        Xt.append(Xt[0].clone())
    Yt = [torch.empty((batch, wl.n_out), dtype=torch.float32, device=dev) for _ in range(nset)]
    wst = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None for _ in range(nset)]
    if chain:
        pats = (libks.ks_pattern_t * len(wl.patterns))(*[libks.ks_pattern_t(*p) for p in wl.patterns])
        wptrs = (ctypes.c_void_p * len(Wt))(*[w.data_ptr() for w in Wt])
        calls = [(lib.ks_chain_matmul,
                  (pats, len(wl.patterns), wptrs, ctypes.c_void_p(Xt[k].data_ptr()),
                   ctypes.c_void_p(Yt[k].data_ptr()), batch, dt,
                   ctypes.c_void_p(wst[k].data_ptr() if wst[k] is not None else None), ws_bytes, flags, sp))
                 for k in range(nset)]
    else:
        pat = libks.ks_pattern_t(*wl.patterns[0])
        calls = [(lib.ks_matmul, (pat, ctypes.c_void_p(Wt[0].data_ptr()), ctypes.c_void_p(Xt[k].data_ptr()),
                                  ctypes.c_void_p(Yt[k].data_ptr()), batch, dt, sp)) for k in range(nset)]

    def run(i):
        fn, a = calls[i]
        st = fn(*a)
        if st != 0:
            raise libks.KSError(st, "bench %s" % wl.name)

    ms = time_launches(run, nset, stream, torch, reps)
    flops = sum(2 * batch * datagen.nnz(p) for p in wl.patterns)
    del Xt, Yt, wst, Wt, calls
    return {"ms": ms, "bytes_run": bytes_run, "bytes_min": bytes_min, "flops": flops,
            "launches": len(groups)}


def other_configs(lib, sp, stream, torch, np, datagen, libks) -> dict:
    """The other configurations of the KS workloads, each timed like the
    headline (rotated inputs, back-to-back calls, HIP events), summarised:
    the ViT factor, the GPT-2 chain fused and one launch per factor, the
    65,536-point butterfly with bf16 inputs and weights, the 65,536-point
    radix-2 and radix-4 butterflies fused and one launch per factor, and the 51-pattern
    square sweep (roofline fraction of each pattern: bytes over 8 TB/s or
    flops over the fp32 matrix peak, whichever takes longer)."""
    out = {}

    def frac(b, ms):
        return round(b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    r = time_workload(datagen.get("vit_mlp"), False, libks.CHAIN_AUTO, lib, sp, stream, torch, np, datagen,
                      libks)
    out["vit_mlp"] = {"dtype": "f32", "ms": round(r["ms"], 5), "GB/s": round(r["bytes_run"] / r["ms"] / 1e6, 1),
                      "TFLOP/s": round(r["flops"] / r["ms"] / 1e9, 2), "frac": frac(r["bytes_run"], r["ms"]),
                      "plan": libks.ks_plan_describe((4, 64, 16, 6), 25216, libks.DTYPE_F32)}
    g = {}
    for name, flags in (("fused", libks.CHAIN_AUTO), ("one_launch_per_factor", libks.CHAIN_NO_FUSE)):
        r = time_workload(datagen.get("gpt2_mlp"), False, flags, lib, sp, stream, torch, np, datagen, libks)
        g[name] = {"ms": round(r["ms"], 5), "launches": r["launches"],
                   "frac_as_run": frac(r["bytes_run"], r["ms"]),
                   "frac_vs_fused_minimum": frac(r["bytes_min"], r["ms"])}
    out["gpt2_mlp"] = {"dtype": "f32", **g}
    r = time_workload(datagen.get("butterfly65536"), True, libks.CHAIN_AUTO, lib, sp, stream, torch, np, datagen,
                      libks, reps=10)
    out["butterfly65536_bf16"] = {"dtype": "bf16", "ms": round(r["ms"], 5), "launches": r["launches"],
                                  "GB/s": round(r["bytes_run"] / r["ms"] / 1e6, 1),
                                  "frac_as_run": frac(r["bytes_run"], r["ms"]),
                                  "frac_vs_fused_minimum": frac(r["bytes_min"], r["ms"])}
    # butterflies on rows wider than LDS: closure tiles and register-resident slabs
    for name in ("radix2_n65536", "radix4_n65536"):
        w = {}
        for key, flags in (("fused", libks.CHAIN_AUTO), ("one_launch_per_factor", libks.CHAIN_NO_FUSE)):
            r = time_workload(datagen.get(name), False, flags, lib, sp, stream, torch, np, datagen, libks,
                              reps=10)
            w[key] = {"ms": round(r["ms"], 5), "launches": r["launches"],
                      "frac_as_run": frac(r["bytes_run"], r["ms"]),
                      "frac_vs_fused_minimum": frac(r["bytes_min"], r["ms"])}
        out[name] = {"dtype": "f32", **w}
    fr, small, big = [], [], []
    for p in datagen.square_sweep_patterns():
        wl = datagen.get("square_%d_%d_%d_%d" % p)
        r = time_workload(wl, False, libks.CHAIN_AUTO, lib, sp, stream, torch, np, datagen, libks, reps=30)
        t_roof = max(r["bytes_run"] / (HBM_PEAK_GBS * 1e9), r["flops"] / (FP32_PEAK_TFLOPS * 1e12))
        f = t_roof / (r["ms"] * 1e-3)
        fr.append(f)
        (small if p[1] <= 32 else big).append(f)
        if p[1] == 128:
            out.setdefault("_b128", []).append(round(f, 3))
    out["square_sweep"] = {
        "dtype": "f32", "patterns": len(fr), "rows": 16384,
        "roofline_frac_median": round(float(np.median(fr)), 4),
        "roofline_frac_min": round(float(np.min(fr)), 4),
        "roofline_frac_max": round(float(np.max(fr)), 4),
        "b_le_32_patterns": len(small),
        "b_le_32_hbm_frac_median": round(float(np.median(small)), 4),
        "b_le_32_at_or_above_0.70": int(sum(f >= 0.70 for f in small)),
        "b_128_mfma_fracs": out.pop("_b128"),
    }
    torch.cuda.empty_cache()
    return out


def traffic_key(args) -> str:
    return args.workload + ":" + args.dtype + (":nofuse" if args.no_fuse else "")


def time_groups(args, wl, groups, group_bytes, Wt, X0, bf16, flags, lib, sp, stream, torch, np, datagen, libks):
    """Each launch group of the chain on its own, as the chain runs it: the
    first group on the workload's X, later ones on fp32 inputs of their
    shape (with bf16 weights in a bf16 chain); a single factor through
    ks_matmul_ex with the planner's choice, a fused group through
    ks_chain_matmul on its factors (one launch, no workspace)."""
    dev = X0.device
    batch = wl.batch
    out = []
    for g, grp in enumerate(groups):
        k0, k1 = grp[0], grp[-1]
        pats = wl.patterns[k0:k1 + 1]
        if k0 == 0:
            gdt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
        else:
            gdt = libks.DTYPE_BF16W if bf16 else libks.DTYPE_F32
        sets = max(2, int(np.ceil(CACHE_BYTES / group_bytes[g])) + 1)
        xs = [X0 if k0 == 0 else torch.randn((batch, datagen.n_in(pats[0])), device=dev)]
        for _ in range(sets - 1):
            xs.append(xs[0].clone())
        ys = [torch.empty((batch, datagen.n_out(pats[-1])), dtype=torch.float32, device=dev) for _ in range(sets)]
        if len(grp) == 1:
            opt = libks.ks_options_t()
            pat = libks.ks_pattern_t(*pats[0])
            fn = lib.ks_matmul_ex
            gcalls = [(pat, ctypes.c_void_p(Wt[k0].data_ptr()), ctypes.c_void_p(xs[j].data_ptr()),
                       ctypes.c_void_p(ys[j].data_ptr()), batch, gdt, sp, ctypes.byref(opt)) for j in range(sets)]
            plan = libks.ks_plan_describe(pats[0], batch, gdt)
        else:
            if libks.ks_chain_groups(pats, batch, gdt, flags) != [list(range(len(pats)))]:
                raise RuntimeError("launch group %s does not run as one launch on its own" % (grp,))
            # a pair that could meet unaligned pointers keeps a spare buffer
            # in its workspace; with these aligned tensors it is not touched
            wsb = libks.ks_chain_workspace_size(pats, batch, gdt, flags)
            gws = torch.empty(wsb, dtype=torch.uint8, device=dev) if wsb else None
            parr = (libks.ks_pattern_t * len(pats))(*[libks.ks_pattern_t(*p) for p in pats])
            warr = (ctypes.c_void_p * len(pats))(*[Wt[k].data_ptr() for k in grp])
            fn = lib.ks_chain_matmul
            gcalls = [(parr, len(pats), warr, ctypes.c_void_p(xs[j].data_ptr()), ctypes.c_void_p(ys[j].data_ptr()),
                       batch, gdt, ctypes.c_void_p(gws.data_ptr() if gws is not None else None), wsb, flags, sp)
                      for j in range(sets)]
            plan = chain_plan_text(pats, batch, gdt, flags, bf16 and k0 == 0)

        def run(j):
            st = fn(*gcalls[j % sets])
            if st != 0:
                raise libks.KSError(st, "bench group %s" % (grp,))

        warm_up(run, 3, torch)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        reps = 20
        e0.record(stream)
        for j in range(reps):
            run(j)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        gbs = group_bytes[g] / (ms * 1e-3) / 1e9
        out.append({"factors": list(grp), "ms": round(ms, 5), "bytes": group_bytes[g], "GB/s": round(gbs, 1),
                    "frac": round(gbs / HBM_PEAK_GBS, 4), "kernel": plan})
        del xs, ys
    return out


def time_factors(wl, Wt, X0, bf16, lib, sp, stream, torch, np, datagen, libks):
    """Every factor of a chain as a single launch (ks_matmul_ex, the
    planner's choice) on inputs of its shape, back to back with HIP events."""
    dev = X0.device
    batch = wl.batch
    xb = 2 if bf16 else 4
    wbytes = 2 if bf16 else 4
    out = []
    for k, p in enumerate(wl.patterns):
        dtk = (libks.DTYPE_BF16 if k == 0 else libks.DTYPE_BF16W) if bf16 else libks.DTYPE_F32
        xbk = xb if k == 0 else 4
        fbytes = factor_bytes(p, xbk, wbytes, batch)
        ksets = max(1, int(np.ceil(CACHE_BYTES / fbytes)) + 1)
        xs = [X0 if k == 0 else torch.randn((batch, datagen.n_in(p)), device=dev)]
        for _ in range(ksets - 1):
            xs.append(xs[0].clone())
        ys = [torch.empty((batch, datagen.n_out(p)), dtype=torch.float32, device=dev) for _ in range(ksets)]
        opt = libks.ks_options_t()
        pat = libks.ks_pattern_t(*p)
        fcalls = [(pat, ctypes.c_void_p(Wt[k].data_ptr()), ctypes.c_void_p(xs[j].data_ptr()),
                   ctypes.c_void_p(ys[j].data_ptr()), batch, dtk, sp, ctypes.byref(opt)) for j in range(ksets)]
        reps = 20
        warm_up(lambda j: lib.ks_matmul_ex(*fcalls[j % ksets]), 3, torch)
        f0 = torch.cuda.Event(enable_timing=True)
        f1 = torch.cuda.Event(enable_timing=True)
        f0.record(stream)
        for j in range(reps):
            st = lib.ks_matmul_ex(*fcalls[j % ksets])
            if st != 0:
                raise libks.KSError(st, "bench factor")
        f1.record(stream)
        torch.cuda.synchronize()
        fms = f0.elapsed_time(f1) / reps
        out.append({"pattern": list(p), "ms": round(fms, 5),
                    "GB/s": round(fbytes / (fms * 1e-3) / 1e9, 1),
                    "frac": round(fbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                    "plan": libks.ks_plan_describe(p, batch, dtk)})
        del xs, ys
    return out


COPY_BYTES = 2 ** 30     # the device copy of copy_ceiling reads and writes this many bytes


def copy_ceiling(dev, stream, torch, nbytes=COPY_BYTES) -> float:
    """A plain device-to-device copy of nbytes (torch's copy kernel; 1 GiB
    by default), timed with HIP events over back-to-back calls after
    warm-up: GB/s counting the bytes read plus the bytes written. A practical
    streaming ceiling of this GPU, reported beside the published 8 TB/s
    peak."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    warm_up(lambda i: dst.copy_(src), 3, torch)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del src, dst
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def copy_ceilings(args) -> int:
    """The copy ceiling at several sizes (the sweep's per-launch traffic is
    about 256 MiB each way; the butterfly factors move 1 GiB each way); one
    JSON line."""
    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)
    rows = []
    for mib in (64, 256, 1024, 4096):
        gbs = copy_ceiling(dev, stream, torch, mib * 2 ** 20)
        rows.append({"bytes_each_way": mib * 2 ** 20, "GB/s": gbs, "frac_of_8TBs": round(gbs / HBM_PEAK_GBS, 4)})
    print(json.dumps({"copy_ceiling": "torch device copy, read + write bytes", "rows": rows}), flush=True)
    return 0


def backward(args) -> int:
    """Gradients of each factor of the workload on synthetic dY (fp32) and
    inputs: dX = dY W (the transposing launch plus the forward product of the
    transposed pattern) and dK, each timed back to back over rotated buffers
    after warm-up. Bytes as run: dX reads dY and W (twice: transpose, then
    the product) and writes dX and the transposed W; dK reads dY and X,
    writes the partial sums and reads them back, and writes dK."""
    import numpy as np
    import torch
    from kronecker_sparse_structured_amd import datagen, libks

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    wl = datagen.get(args.workload)
    bf16 = args.dtype == "bf16"
    batch = wl.batch
    sx = 2 if bf16 else 4
    stream = torch.cuda.current_stream(dev)
    rng = np.random.default_rng(11)
    rows = []
    for k, p in enumerate(wl.patterns):
        a, b, c, d = p
        n_in, n_out, nnz = a * c * d, a * b * d, a * b * c * d
        # inputs of factor k > 0 are fp32 intermediates in a chain
        xdt = torch.bfloat16 if (bf16 and k == 0) else torch.float32
        W = torch.from_numpy(rng.standard_normal((a, d, b, c), dtype=np.float32)).to(dev)
        if bf16:
            W = W.to(torch.bfloat16)
        nset = 2
        Xs = [torch.randn((batch, n_in), device=dev).to(xdt) for _ in range(nset)]
        dYs = [torch.randn((batch, n_out), device=dev) for _ in range(nset)]
        dXs = [torch.empty((batch, n_in), device=dev) for _ in range(nset)]
        dWs = [torch.empty((a, d, b, c), device=dev) for _ in range(nset)]
        dt_x = libks.DTYPE_BF16W if bf16 else libks.DTYPE_F32
        dt_w = libks.DTYPE_BF16 if xdt == torch.bfloat16 else libks.DTYPE_F32
        wsx_b = libks.ks_matmul_dx_workspace_size(p, dt_x)
        wsw_b = libks.ks_matmul_dw_workspace_size(p, batch, dt_w)
        wsx = torch.empty(max(wsx_b, 1), dtype=torch.uint8, device=dev)
        wsw = torch.empty(max(wsw_b, 1), dtype=torch.uint8, device=dev)
        run_dx = lambda i: libks.ks_matmul_dx(p, W, dYs[i % nset], dXs[i % nset], batch, dt_x, wsx, wsx_b, stream)
        run_dw = lambda i: libks.ks_matmul_dw(p, dYs[i % nset], Xs[i % nset], dWs[i % nset], batch, dt_w,
                                              wsw if wsw_b else None, wsw_b, stream)

        def timed(fn):
            t0 = time.time()
            while time.time() - t0 < 0.2:
                fn(0)
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            reps = 20
            for i in range(reps):
                fn(i)
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps * 1e-3

        sw = 2 if bf16 else 4
        t_dx, t_dw = timed(run_dx), timed(run_dw)
        by_dx = 4 * batch * n_out + 4 * batch * n_in + 3 * sw * nnz
        by_dw = 4 * batch * n_out + (sx if xdt == torch.bfloat16 else 4) * batch * n_in + 4 * nnz + 2 * wsw_b
        flops = 2 * batch * nnz
        fr = lambda by, s: max(by / 8.0e12, flops / 157.3e12) / s
        rows.append({"pattern": list(p),
                     "dx_ms": round(t_dx * 1e3, 5), "dx_GB/s": round(by_dx / t_dx / 1e9, 1),
                     "dx_roofline_frac": round(fr(by_dx, t_dx), 4),
                     "dx_plan": libks.ks_plan_describe((a, c, b, d), batch, dt_x),
                     "dw_ms": round(t_dw * 1e3, 5), "dw_GB/s": round(by_dw / t_dw / 1e9, 1),
                     "dw_roofline_frac": round(fr(by_dw, t_dw), 4), "dw_workspace_bytes": wsw_b})
    print(json.dumps({"metric": "KS matmul gradients (dX, dK) per factor, % of roofline, 1xMI355X",
                      "workload": wl.name, "batch": batch, "dtype": args.dtype, "data": "synthetic",
                      "factors": rows}), flush=True)
    return 0


def chain_plan_text(patterns, batch, dt, flags, bf16) -> str:
    """One entry per launch of the chain (the library's own description of
    each launch group), "; "-separated, without the factor ranges."""
    from kronecker_sparse_structured_amd import libks
    del bf16  # the dtype code already says which factors read bf16
    parts = libks.ks_chain_describe(patterns, batch, dt, flags).split("; ")
    return "; ".join(p.split("] ", 1)[1] if p.startswith("[") else p for p in parts)


def sweep(args) -> int:
    """The square sweep: every (a, b, b, d) with b in {4 .. 128} and
    a * b * d = 4096 on 16,384 rows, fp32 (or bf16), each on its own seeded
    inputs, timed like the contract run (rotated input sets, back-to-back
    launches, HIP events around the timed launches on the launch stream)."""
    import numpy as np
    import torch
    from kronecker_sparse_structured_amd import datagen, libks

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    bf16 = args.dtype == "bf16"
    dt = libks.DTYPE_BF16 if bf16 else libks.DTYPE_F32
    xb = 2 if bf16 else 4
    lib = libks.load()
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(int(stream.cuda_stream))
    peak_flops = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    rows = []
    items = [(p, datagen.get("square_%d_%d_%d_%d" % p), "square") for p in datagen.square_sweep_patterns()]
    if args.workload_factors:
        # each factor of these workloads alone, at the workload's batch (the
        # launches a chain makes for factors it does not fuse)
        seen = set(tuple(p) for p, _, _ in items)
        for name in WORKLOAD_FACTOR_SETS:
            src = datagen.get(name)
            for k, p in enumerate(src.patterns):
                if tuple(p) in seen:
                    continue
                seen.add(tuple(p))
                items.append((tuple(p), datagen.Workload(name, [tuple(p)], src.batch, [src.sigmas[k]],
                                                         src.seed + 100 + k), name))
    for p, wl, set_name in items:
        X, Ws = datagen.draw(wl)
        put = ((lambda a: torch.from_numpy(datagen.bf16_bits(a).view(np.int16)).to(dev).view(torch.bfloat16))
               if bf16 else (lambda a: torch.from_numpy(a).to(dev)))
        batch = wl.batch
        nbytes = factor_bytes(p, xb, xb, batch)
        flops = 2 * batch * datagen.nnz(p)
        nset = max(2, int(np.ceil(CACHE_BYTES / nbytes)) + 1)
        Xt = [put(X)]
        for _ in range(nset - 1):
            Xt.append(Xt[0].clone())
        Wt = put(Ws[0])
        Yt = [torch.empty((batch, datagen.n_out(p)), dtype=torch.float32, device=dev) for _ in range(nset)]
        opt = libks.ks_options_t()
        pat = libks.ks_pattern_t(*p)
        calls = [(pat, ctypes.c_void_p(Wt.data_ptr()), ctypes.c_void_p(Xt[k].data_ptr()),
                  ctypes.c_void_p(Yt[k].data_ptr()), batch, dt, sp, ctypes.byref(opt)) for k in range(nset)]
        warm_up(lambda i: lib.ks_matmul_ex(*calls[i % nset]), 5, torch)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        steps = 30
        e0.record(stream)
        for i in range(steps):
            st = lib.ks_matmul_ex(*calls[i % nset])
            if st != 0:
                raise libks.KSError(st, "sweep %s" % (p,))
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        t_roof = max(nbytes / (HBM_PEAK_GBS * 1e9), flops / (peak_flops * 1e12))
        bound = "hbm" if nbytes / (HBM_PEAK_GBS * 1e9) >= flops / (peak_flops * 1e12) else "mfma"
        row = {"pattern": list(p), "set": set_name, "batch": batch, "ms": round(ms, 5),
               "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
               "bound": bound,
               "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / peak_flops, 4),
               "roofline_frac": round(t_roof / (ms * 1e-3), 4),
               "plan": libks.ks_plan_describe(p, batch, dt)}
        if args.comparator and not bf16:
            row.update(comparator(p, batch, Xt, Wt, Yt, nset, ms, stream, torch))
        if args.families:
            row["families"] = time_families(p, batch, Wt, Xt, Yt, nset, dt, lib, sp, stream, torch, libks)
            best = min(row["families"], key=lambda f: f["ms"])
            row["best"] = {"kernel": best["kernel"], "store_waves": best["store_waves"],
                           "mfma_tile": best["mfma_tile"], "mfma_loaders": best["mfma_loaders"]}
        rows.append(row)
        print("%-18s %9.1f us %8.1f GB/s %7.2f TFLOP/s  %s  roofline %.3f   %s" % (
            str(tuple(p)), ms * 1e3, row["GB/s"], row["TFLOP/s"], bound, row["roofline_frac"],
            ("permute-bmm %.1f us, x%.2f  " % (row["comparator_ms"] * 1e3, row["speedup"])
             if "speedup" in row else "") + row["plan"][:60]), flush=True)
        del Xt, Yt, Wt, X, Ws
    fr = [r["roofline_frac"] for r in rows if r["set"] == "square"]
    extra = {}
    sp_all = [r["speedup"] for r in rows if "speedup" in r]
    if sp_all:
        extra = {"speedup_vs_permute_bmm_median": round(float(np.median(sp_all)), 3),
                 "speedup_min": round(float(np.min(sp_all)), 3), "speedup_max": round(float(np.max(sp_all)), 3),
                 "faster_than_permute_bmm": int(sum(s > 1.0 for s in sp_all))}
    summary = {"sweep": "square n=4096, 16384 rows", "dtype": args.dtype, "patterns": len(rows), **extra,
               "roofline_frac_median": round(float(np.median(fr)), 4),
               "roofline_frac_min": round(float(np.min(fr)), 4),
               "roofline_frac_max": round(float(np.max(fr)), 4), "rows": rows}
    print(json.dumps(summary), flush=True)
    if args.sweep_text:
        write_sweep_text(summary, args.sweep_text)
    return 0


# workloads whose factors --workload-factors adds to the sweep
WORKLOAD_FACTOR_SETS = ("butterfly65536", "vit_mlp", "gpt2_mlp")


def write_sweep_text(summary, path):
    """The sweep as a text table (one line per pattern, then the fractions by
    block size): the form kept under profiles/."""
    import numpy as np
    rows = summary["rows"]
    dt = summary["dtype"]
    peak = BF16_PEAK_TFLOPS if dt == "bf16" else FP32_PEAK_TFLOPS
    out = ["# Square pattern sweep: every (a, b, b, d) with b in {4, 8, 16, 32, 64, 128}, a * b * d = 4096, "
           "16,384 rows, %s" % ("bf16 X and weights" if dt == "bf16" else "fp32"),
           "",
           "command ($REPO = repository root):  python3 $REPO/bench.py --sweep%s --sweep-text <this file>"
           % (" --dtype bf16" if dt == "bf16" else ""),
           "(each pattern on its own seeded inputs; two rotated input/output sets of ~537 MB each, so every "
           "launch reads",
           " from HBM; 0.2 s of warm-up launches, then 30 back-to-back launches timed with HIP events on the "
           "launch stream)",
           "",
           "roofline = max(bytes / 8 TB/s, flops / %.1f TFLOP/s) / measured time; bound = the larger term" % peak,
           "",
           "pattern               time us       GB/s    TFLOP/s  bound  roofline  plan"]
    for r in rows:
        out.append("%-20s %9.1f %10.1f %10.2f %7s %9.3f  %s%s" % (
            str(tuple(r["pattern"])), r["ms"] * 1e3, r["GB/s"], r["TFLOP/s"], r["bound"], r["roofline_frac"],
            "" if r.get("set", "square") == "square" else "[%s, %d rows] " % (r["set"], r["batch"]), r["plan"]))
    square = [r for r in rows if r.get("set", "square") == "square"]
    fr = [r["roofline_frac"] for r in square]
    small = [r["roofline_frac"] for r in square if r["pattern"][1] <= 32]
    b128 = [r["roofline_frac"] for r in square if r["pattern"][1] == 128]
    out += ["",
            "roofline fraction over the %d square patterns: median %.3f, min %.3f, max %.3f"
            % (len(fr), np.median(fr), min(fr), max(fr))]
    if small:
        out.append("b = c <= 32 (%d patterns, HBM-bound): median %.3f, min %.3f, max %.3f of 8 TB/s"
                   % (len(small), np.median(small), min(small), max(small)))
    if b128:
        out.append("b = c = 128 (%d patterns, MFMA-bound): %s of %.1f TFLOP/s"
                   % (len(b128), ", ".join("%.2f" % v for v in b128), peak))
    with open(path, "w") as f:
        f.write("\n".join(out) + "\n")


# Kernel families (and the matrix-core family's store schedules, tile
# candidates and loader waves) timed per pattern by --sweep --families:
# (name, ks_kernel_t, ks_store_waves_t, mfma tile, mfma loaders; 0 = the
# kernel's own choice).
FAMILY_VARIANTS = ([("mfma/compute", 3, 1, 0, 0), ("mfma/dedicated", 3, 2, 0, 0)] +
                   [("mfma/t%d/%s" % (t, sn), 3, sw, t, 0) for t in range(1, 8)
                    for sn, sw in (("compute", 1), ("dedicated", 2))] +
                   [("mfma/2l/compute", 3, 1, 0, 2), ("mfma/2l/dedicated", 3, 2, 0, 2)] +
                   [("valu", 2, 0, 0, 0), ("col", 5, 0, 0, 0)])


def time_families(p, batch, Wt, Xt, Yt, nset, dt, lib, sp, stream, torch, libks):
    """Every family that runs pattern p, each timed like the sweep's
    automatic choice (back-to-back launches over the rotated sets after
    warm-up, HIP events); families that refuse the pattern are skipped."""
    out = []
    pat = libks.ks_pattern_t(*p)
    for name, kernel, store, tile, loaders in FAMILY_VARIANTS:
        opt = libks.ks_options_t()
        opt.kernel = kernel
        opt.store_waves = store
        opt.mfma_tile = tile
        opt.mfma_loaders = loaders
        calls = [(pat, ctypes.c_void_p(Wt.data_ptr()), ctypes.c_void_p(Xt[k].data_ptr()),
                  ctypes.c_void_p(Yt[k].data_ptr()), batch, dt, sp, ctypes.byref(opt)) for k in range(nset)]
        st = lib.ks_matmul_ex(*calls[0])
        if st == libks.KS_ERR_UNSUPPORTED:
            continue
        if st != 0:
            raise libks.KSError(st, "sweep family %s %s" % (name, p))
        warm_up(lambda i: lib.ks_matmul_ex(*calls[i % nset]), 5, torch)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(30):
            lib.ks_matmul_ex(*calls[i % nset])
        e1.record(stream)
        torch.cuda.synchronize()
        out.append({"name": name, "kernel": kernel, "store_waves": store, "mfma_tile": tile,
                    "mfma_loaders": loaders, "ms": round(e0.elapsed_time(e1) / 30, 5)})
    return out


def comparator_only(args) -> int:
    """The permute / batched GEMM / permute comparator alone on a
    single-factor workload (W + K steps over rotated sets, then, with
    --calib-copy, the calibration copies), for counting its HBM traffic
    under rocprofv3 --pmc; prints one JSON line with its time per call."""
    import numpy as np
    import torch
    from kronecker_sparse_structured_amd import datagen

    dev = torch.device("cuda:0")
    wl = datagen.get(args.workload)
    p = wl.patterns[0]
    X, Ws = datagen.draw(wl)
    batch = wl.batch
    nbytes = factor_bytes(p, 4, 4, batch)
    nset = max(2, int(np.ceil(CACHE_BYTES / nbytes)) + 1)
    Xt = [torch.from_numpy(X).to(dev)]
    for _ in range(nset - 1):
        Xt.append(Xt[0].clone())
    Wt = torch.from_numpy(Ws[0]).to(dev)
    Yt = [torch.empty((batch, datagen.n_out(p)), dtype=torch.float32, device=dev) for _ in range(nset)]
    run = comparator_fn(p, batch, Xt, Wt, Yt, torch)
    stream = torch.cuda.current_stream(dev)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        run(i % nset)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        run(i % nset)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    if args.calib_copy:
        src = torch.empty(CALIB_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps({"comparator": "permute / torch.bmm / permute", "workload": wl.name, "pattern": list(p),
                      "calls": args.warmup + args.steps, "ms": round(ms, 5),
                      "bytes_fused_algorithmic": nbytes}), flush=True)
    return 0


def ingest_comparator_counters(args) -> int:
    """HBM bytes per call of the comparator from the two counter runs of
    --comparator-only: every dispatch except device copies (the input
    replication and the calibration copies) and fills, each counter scaled
    by its reading on the calibration copy, divided by the calls."""
    import csv
    from collections import defaultdict
    from kronecker_sparse_structured_amd import datagen

    wl = datagen.get(args.workload)
    p = wl.patterns[0]
    calls = args.warmup + args.steps
    res = {}
    for path, counter in ((args.ingest_comparator[0], "FETCH_SIZE"), (args.ingest_comparator[1], "WRITE_SIZE")):
        vals, names = defaultdict(float), {}
        with open(path) as f:
            for r in csv.DictReader(f):
                if r["Counter_Name"] == counter:
                    vals[r["Dispatch_Id"]] += float(r["Counter_Value"])
                    names[r["Dispatch_Id"]] = r["Kernel_Name"]
        copies = sorted((k for k, n in names.items() if "copyBuffer" in n), key=int)
        calib = [vals[k] for k in copies[-3:]]
        work = [vals[k] for k, n in names.items() if "copyBuffer" not in n and "FillFunctor" not in n]
        factor = CALIB_BYTES / (max(calib) * 1024.0)
        res[counter] = sum(work) * 1024.0 * factor / calls
        res[counter.lower() + "_factor"] = round(factor, 4)
        res[counter.lower() + "_dispatches_per_call"] = round(len(work) / calls, 2)
    xy = 4 * wl.batch * (datagen.n_in(p) + datagen.n_out(p))
    out = {"workload": wl.name, "pattern": list(p), "comparator_bytes_per_call": int(res["FETCH_SIZE"] + res["WRITE_SIZE"]),
           "X_plus_Y_bytes": xy, "ratio_to_X_plus_Y": round((res["FETCH_SIZE"] + res["WRITE_SIZE"]) / xy, 4),
           **{k: v for k, v in res.items() if k not in ("FETCH_SIZE", "WRITE_SIZE")}}
    print(json.dumps(out))
    return 0


def comparator_fn(p, batch, Xt, Wt, Yt, torch):
    """run(k): Y[k] from X[k] by permute / torch.bmm / permute (see comparator)."""
    a, b, c, d = p
    Kt = Wt.view(a * d, b, c).transpose(1, 2).contiguous()        # (a*d, c, b)

    def run(k):
        Xp = Xt[k].view(batch, a, c, d).permute(1, 3, 0, 2).contiguous().view(a * d, batch, c)
        Z = torch.bmm(Xp, Kt)                                        # (a*d, batch, b)
        Yt[k].view(batch, a, b, d).copy_(Z.view(a, d, batch, b).permute(2, 0, 3, 1))

    return run


def energy(args) -> int:
    """Energy per call from the device's energy accumulator (amdsmi, counter
    x its resolution), read around ~2 s of back-to-back calls after warm-up,
    for the fused kernel and the comparator on the same inputs; fp32. The
    average power over the loop is reported too. Context only: the counter
    covers the whole device (idle draw included)."""
    import numpy as np
    import torch
    from kronecker_sparse_structured_amd import datagen, libks
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handle = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception as exc:                       # no energy counter on this machine
        print(json.dumps({"metric": "energy", "error": str(exc)}), flush=True)
        return 1

    def joules():
        e = amdsmi.amdsmi_get_energy_count(handle)
        return e["energy_accumulator"] * e["counter_resolution"] * 1e-6

    dev = torch.device("cuda:0")
    rows = []
    for name in ["vit_mlp", "square_16_16_16_16", "square_32_128_128_1"]:
        wl = datagen.get(name)
        p = wl.patterns[0]
        X, Ws = datagen.draw(wl)
        nset = 2
        Xt = [torch.from_numpy(X).to(dev) for _ in range(nset)]
        Wt = torch.from_numpy(Ws[0]).to(dev)
        Yt = [torch.empty((wl.batch, wl.n_out), device=dev) for _ in range(nset)]
        fused = lambda k: libks.ks_matmul(p, Wt, Xt[k], Yt[k], wl.batch, libks.DTYPE_F32)
        comp = comparator_fn(p, wl.batch, Xt, Wt, Yt, torch)
        row = {"workload": name, "pattern": list(p)}
        for label, fn in (("fused", fused), ("permute_bmm", comp)):
            warm_up(lambda i: fn(i % nset), 5, torch)
            j0, t0, n = joules(), time.perf_counter(), 0
            while time.perf_counter() - t0 < 2.0:
                for _ in range(10):
                    fn(n % nset)
                    n += 1
                torch.cuda.synchronize()
            j1, t1 = joules(), time.perf_counter()
            row[label] = {"calls": n, "mJ_per_call": round((j1 - j0) / n * 1e3, 4),
                          "avg_W": round((j1 - j0) / (t1 - t0), 1), "us_per_call": round((t1 - t0) / n * 1e6, 2)}
        row["energy_ratio"] = round(row["permute_bmm"]["mJ_per_call"] / max(row["fused"]["mJ_per_call"], 1e-12), 3)
        rows.append(row)
        del Xt, Yt, Wt
    print(json.dumps({"metric": "GPU energy per call (amdsmi energy accumulator), fused vs permute/bmm/permute",
                      "dtype": "f32", "data": "synthetic", "rows": rows}), flush=True)
    return 0


def comparator(p, batch, Xt, Wt, Yt, nset, ms_ours, stream, torch):
    """The formulation the KS abstract page (first paragraph) ascribes to
    existing kernels: permute X so that each (alpha, delta) block's rows are
    contiguous, one batched GEMM over the a*d blocks (torch.bmm, i.e. the
    vendor BLAS), permute the result back into Y's layout. Weights are
    rearranged once, outside the timed region. Returns its time per call,
    the speedup of the fused kernel over it, and the largest relative
    difference between the two outputs on one input set."""
    ref = Yt[0].clone()
    run = comparator_fn(p, batch, Xt, Wt, Yt, torch)

    warm_up(lambda i: run(i % nset), 3, torch)
    run(0)
    torch.cuda.synchronize()
    diff = float((Yt[0] - ref).abs().max() / ref.abs().max().clamp_min(1e-30))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    steps = 10
    e0.record(stream)
    for i in range(steps):
        run(i % nset)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"comparator_ms": round(ms, 5), "speedup": round(ms / ms_ours, 3), "comparator_max_rel_diff": diff}


def cpu_baseline(wl, bf16, target_s, row_bytes=None):
    """The fp64 oracle as it stands, timed on this host on a bounded number
    of rows of the same workload; reported in the same unit (GB/s of the
    workload's algorithmic bytes per row)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from kronecker_sparse_structured_amd import datagen

    lib = oracle.load()
    xw = "bf16" if bf16 else "f32"
    # at most 4,096 rows, and at most 8 M input elements (wide chains), drawn
    # the same way as the workload; the timed runs repeat over them
    small = datagen.scaled(wl, max(1, min(wl.batch, 4096, (8 << 20) // wl.n_in)))
    X, Ws = datagen.draw(small)
    Wd = [oracle.widen(datagen.bf16_bits(W), "bf16") if bf16 else oracle.widen(W) for W in Ws]
    Xd_all = oracle.widen(datagen.bf16_bits(X), "bf16") if bf16 else oracle.widen(X)

    def run(rows):
        t0 = time.perf_counter()
        if len(wl.patterns) == 1:
            oracle.ks_matmul(wl.patterns[0], Wd[0], Xd_all[:rows], lib=lib)
        else:
            oracle.ks_chain_matmul(wl.patterns, Wd, Xd_all[:rows], lib=lib)
        return time.perf_counter() - t0

    rows = min(16, small.batch)
    t = run(rows)
    while t < 0.2 and rows < small.batch:
        rows = min(small.batch, rows * 4)
        t = run(rows)
    per_row = t / rows
    want = int(max(1, min(small.batch, target_s / per_row)))
    reps = max(1, int(target_s / (per_row * want)))
    total_t = 0.0
    for _ in range(reps):
        total_t += run(want)
    rows_done = want * reps
    if row_bytes is None:
        row_bytes = (2 if bf16 else 4) * wl.n_in + 4 * wl.n_out
    gbs = row_bytes * rows_done / total_t / 1e9
    cores = oracle.num_threads(lib)

    # the same oracle on one thread (OpenMP's runtime setter), fewer rows
    one = None
    try:
        import ctypes
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(1)
        rows1 = max(1, min(small.batch, int(target_s / 8 / (per_row * cores))))
        t1 = run(rows1)
        gomp.omp_set_num_threads(cores)
        one = round(row_bytes * rows1 / t1 / 1e9, 4)
    except OSError:
        rows1 = 0
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(gbs, 4),
        "unit": "GB/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d rows of %s (%d of %d rows, %d repeat(s)), %.1f s on %d threads; %s" % (
            rows_done, wl.name, want, wl.batch, reps, total_t, cores, model or "cpu model unknown"),
        "value_one_thread": one,
    }


if __name__ == "__main__":
    sys.exit(main())
