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

Default workload: the ViT-S/16 MLP up-projection as one KS factor, pattern
(4, 64, 16, 6) mapping 384 -> 1536, 25,216 rows (128 images x 197 tokens),
fp32.

Printed: one JSON line with the throughput (algorithmic GB/s), TFLOP/s, the
roofline of the dominant kernel (its average launch duration from HIP events
on the launch stream around the timed launches) and the fp64 oracle timed on
this host's cores on a bounded sample of the same workload.
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


# Kernel sources that the counted workloads (the ViT factor, the GPT-2 pair,
# the butterfly chain) never run: the gradient kernels and the row-resident
# chain kernel. Editing them does not invalidate those workloads' traffic
# counters.
_NOT_COUNTED = ("ks_backward.hip", "ks_rowchain.hip")


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kronecker_sparse_structured_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")) and name not in _NOT_COUNTED:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode())
                h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="vit_mlp")
    ap.add_argument("--dtype", default="f32", choices=["f32", "bf16"])
    ap.add_argument("--kernel", default="auto", choices=["auto", "generic", "valu", "mfma", "mfma_lds"])
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
    ap.add_argument("--ingest-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of a "
                         "`--calib-copy` run into profiles/traffic_counters.json and exit")
    return ap.parse_args()


CALIB_BYTES = 256 * 2 ** 20      # the --calib-copy device copy reads and writes this many bytes


def ingest_counters(args) -> int:
    """HBM bytes per step of the workload's KS kernel(s) from two counter
    runs of the same command. FETCH_SIZE and WRITE_SIZE (KiB per dispatch)
    are each scaled by what the same counter reads for the calibration copy
    (CALIB_BYTES read and written) and summed over the KS dispatches, then
    divided by the number of steps (one dispatch per step for a single
    factor, one per launch group for a chain)."""
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
    scaled = {}
    for path, counter in ((args.ingest_counters[0], "FETCH_SIZE"), (args.ingest_counters[1], "WRITE_SIZE")):
        vals, names = per_dispatch(path, counter)
        ks_ids = [k for k, n in names.items() if "ks::" in n]
        last_ks = max((int(k) for k in ks_ids), default=-1)
        # the calibration copies run after the timed KS launches (earlier
        # copies are the bench's input replication, of other sizes)
        calib = [vals[k] for k, n in names.items()
                 if ("copyBuffer" in n or "copy_kernel" in n) and int(k) > last_ks]
        ks = [vals[k] for k in ks_ids]
        if not calib or not ks:
            print("no calibration copy or no KS dispatch in %s" % path, file=sys.stderr)
            return 1
        if len(ks) % per_step != 0:
            print("%d KS dispatches is not a whole number of %d-launch steps" % (len(ks), per_step),
                  file=sys.stderr)
            return 1
        steps = len(ks) // per_step
        factor = CALIB_BYTES / (max(calib) * 1024.0)
        scaled[counter] = (sum(ks) / steps) * 1024.0 * factor
        out[counter.lower() + "_factor"] = round(factor, 4)
        out[counter.lower() + "_kib_per_step"] = round(sum(ks) / steps, 1)
        out[counter.lower() + "_launches"] = len(ks)
    key = args.workload + ":" + args.dtype + (":nofuse" if args.no_fuse else "")
    db = {}
    if os.path.exists(TRAFFIC_FILE):
        db = json.load(open(TRAFFIC_FILE))
    out["bytes_per_step"] = int(scaled["FETCH_SIZE"] + scaled["WRITE_SIZE"])
    out["launches_per_step"] = per_step
    out["source_hash"] = kernel_source_hash()
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
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(rows would shard across GPUs with no exchange); run with --gpus 1.",
              file=sys.stderr)
        return 2
    if args.sweep:
        return sweep(args)
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

    # algorithmic bytes and flops of one step, as run
    flops = sum(2 * batch * datagen.nnz(p) for p in wl.patterns)
    if chain:
        # as run: each launch group reads its input and writes its output
        # once (fp32 between groups) and reads its weights once.
        bytes_run = 0
        x_sz = xb
        for grp in libks.ks_chain_groups(wl.patterns, batch, dt, flags):
            bytes_run += x_sz * batch * datagen.n_in(wl.patterns[grp[0]])
            bytes_run += 4 * batch * datagen.n_out(wl.patterns[grp[-1]])
            bytes_run += sum(wbytes * datagen.nnz(wl.patterns[k]) for k in grp)
            x_sz = 4
        bytes_min = step_bytes + sum(wbytes * datagen.nnz(p) for p in wl.patterns)
    else:
        bytes_run = factor_bytes(wl.patterns[0], xb, wbytes, batch)
        bytes_min = bytes_run

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
    # average GPU time of one step (one launch for a single factor), from
    # HIP events on the launch stream around the timed launches
    mean_ms = ev0.elapsed_time(ev1) / args.steps

    value = bytes_run * args.steps / wall / 1e9
    achieved = bytes_run / (mean_ms * 1e-3) / 1e9
    peak_flops = BF16_PEAK_TFLOPS if bf16 else FP32_PEAK_TFLOPS
    tflops = flops / (mean_ms * 1e-3) / 1e12
    t_roof = max(bytes_run / (HBM_PEAK_GBS * 1e9), flops / (peak_flops * 1e12))
    bound = "hbm" if bytes_run / (HBM_PEAK_GBS * 1e9) >= flops / (peak_flops * 1e12) else "mfma"

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        try:
            rec = json.load(open(TRAFFIC_FILE)).get(args.workload + ":" + args.dtype +
                                                     (":nofuse" if args.no_fuse else ""))
            if rec and rec.get("source_hash") == kernel_source_hash():
                traffic = rec.get("bytes_per_step")
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
        "achieved": round(achieved if bound == "hbm" else tflops, 2),
        "peak": HBM_PEAK_GBS if bound == "hbm" else peak_flops,
        "unit": "GB/s" if bound == "hbm" else "TFLOP/s",
        "frac": round((achieved / HBM_PEAK_GBS) if bound == "hbm" else (tflops / peak_flops), 4),
        "traffic": traffic,
        "roofline_time_frac": round(t_roof / (mean_ms * 1e-3), 4),
    }

    # chains: each factor timed on its own (back-to-back launches of its
    # kernel on inputs of its shape), and the chain's fraction also against
    # the fully fused minimum |X| + |Y| + weights
    per_factor = None
    if chain and not args.no_factors and not args.calib_copy:
        per_factor = []
        for k, p in enumerate(wl.patterns):
            dtk = dt if k == 0 else (libks.DTYPE_BF16W if bf16 else libks.DTYPE_F32)
            xbk = xb if k == 0 else 4
            fbytes = factor_bytes(p, xbk, wbytes, batch)
            ksets = max(1, int(np.ceil(CACHE_BYTES / fbytes)) + 1)
            xs = [Xt[0] if k == 0 else torch.randn((batch, datagen.n_in(p)), device=dev)]
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
            per_factor.append({"pattern": list(p), "ms": round(fms, 5),
                               "GB/s": round(fbytes / (fms * 1e-3) / 1e9, 1),
                               "frac": round(fbytes / (fms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                               "plan": libks.ks_plan_describe(p, batch, dtk)})
            del xs, ys
        roofline["frac_vs_fused_minimum"] = round(bytes_min / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, bf16, args.cpu_seconds)

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": warm_steps,
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
            "kernel": args.kernel if not chain else "chain",
            "plan": chain_plan_text(wl.patterns, batch, dt, flags, bf16) if chain else
                    libks.ks_plan_describe(wl.patterns[0], batch, dt),
            "rotating_sets": nset,
            "parallelism": "single GPU",
        },
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    if per_factor is not None:
        out["per_factor"] = per_factor
    print(json.dumps(out), flush=True)
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
    """One entry per launch of the chain: the kernel plan of a single factor,
    or the pair that runs as one launch."""
    from kronecker_sparse_structured_amd import libks
    parts = []
    for grp in libks.ks_chain_groups(patterns, batch, dt, flags):
        if len(grp) == 2:
            parts.append("fused pair %s -> %s (one launch, intermediate in LDS)"
                         % (tuple(patterns[grp[0]]), tuple(patterns[grp[1]])))
        elif len(grp) > 2:
            parts.append("fused run of factors %d..%d (one launch, rows resident in LDS)" % (grp[0], grp[-1]))
        else:
            k = grp[0]
            fdt = libks.DTYPE_F32 if not bf16 else (libks.DTYPE_BF16 if k == 0 else libks.DTYPE_BF16W)
            parts.append(libks.ks_plan_describe(patterns[k], batch, fdt))
    return "; ".join(parts)


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
    for p in datagen.square_sweep_patterns():
        wl = datagen.get("square_%d_%d_%d_%d" % p)
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
        row = {"pattern": list(p), "ms": round(ms, 5),
               "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
               "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
               "bound": bound,
               "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "mfma_frac": round(flops / (ms * 1e-3) / 1e12 / peak_flops, 4),
               "roofline_frac": round(t_roof / (ms * 1e-3), 4),
               "plan": libks.ks_plan_describe(p, batch, dt)}
        if args.comparator and not bf16:
            row.update(comparator(p, batch, Xt, Wt, Yt, nset, ms, stream, torch))
        rows.append(row)
        print("%-18s %9.1f us %8.1f GB/s %7.2f TFLOP/s  %s  roofline %.3f   %s" % (
            str(tuple(p)), ms * 1e3, row["GB/s"], row["TFLOP/s"], bound, row["roofline_frac"],
            ("permute-bmm %.1f us, x%.2f  " % (row["comparator_ms"] * 1e3, row["speedup"])
             if "speedup" in row else "") + row["plan"][:60]), flush=True)
        del Xt, Yt, Wt, X, Ws
    fr = [r["roofline_frac"] for r in rows]
    extra = {}
    sp_all = [r["speedup"] for r in rows if "speedup" in r]
    if sp_all:
        extra = {"speedup_vs_permute_bmm_median": round(float(np.median(sp_all)), 3),
                 "speedup_min": round(float(np.min(sp_all)), 3), "speedup_max": round(float(np.max(sp_all)), 3),
                 "faster_than_permute_bmm": int(sum(s > 1.0 for s in sp_all))}
    print(json.dumps({"sweep": "square n=4096, 16384 rows", "dtype": args.dtype, "patterns": len(rows), **extra,
                      "roofline_frac_median": round(float(np.median(fr)), 4),
                      "roofline_frac_min": round(float(np.min(fr)), 4),
                      "roofline_frac_max": round(float(np.max(fr)), 4), "rows": rows}), flush=True)
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


def cpu_baseline(wl, bf16, target_s):
    """The fp64 oracle as it stands, timed on this host on a bounded number
    of rows of the same workload; reported in the same unit (GB/s of the
    workload's algorithmic bytes per row)."""
    import numpy as np
    sys.path.insert(0, ROOT)
    import oracle
    from kronecker_sparse_structured_amd import datagen

    lib = oracle.load()
    xw = "bf16" if bf16 else "f32"
    small = datagen.scaled(wl, min(wl.batch, 4096))
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
    xb = 2 if bf16 else 4
    row_bytes = xb * wl.n_in + 4 * wl.n_out
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
