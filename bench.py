#!/usr/bin/env python3
"""Benchmark: forward + backward of the 2D Gaussian splatting layer on one GPU.

One step = forward (per-Gaussian preprocessing, tile binning, forward raster)
plus backward (gradient raster reusing the forward's binning, finalisation)
over one batch: 384 frames of 128x128x3 with 4096 Gaussians each (32 x 12
frames, scales log-uniform in [0.5, 8] px, anisotropy up to 4:1, amplitudes
N(0, 0.5), 3-sigma truncation), seeded synthetic inputs resident in HBM.

Prints one JSON line.  ``value`` is Gaussian-pixel evaluations per second for
forward + backward: the number of (Gaussian, pixel) pairs inside the
truncation -- counted on the GPU by the library's support count, which walks
the forward raster's lists in the same fp32 arithmetic, outside the timed
region -- divided by the step time.  The CPU leg reports the fp64 oracle's
count of the same pairs beside it.
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

FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector: 256 CU x 2.4 GHz x 256 flop/clk
HBM_PEAK_GBS = 8000.0


def flops_per_pair(C):
    """Algorithmic flops per support pair (add/mul = 1, fma = 2, exp = 1,
    compare/select = 0): forward d(2) z(6) q(3) exp(1) accumulate(2C);
    backward recompute(12) h(2C-1) v(1) A(2C) five sums(10)."""
    return 12 + 2 * C, 24 + 4 * C


def kernel_bytes(B, N, H, W, C, pairs_tiles, T):
    """Algorithmic HBM bytes per launch of each kernel (each tensor moved once)."""
    BN, img = B * N, B * H * W * C * 4
    nT = ((H + T - 1) // T) * ((W + T - 1) // T)
    P = 5 + C
    return {
        "preprocess": BN * P * 4 + BN * 40,
        "bin_count": BN * 8 + B * nT * 4,
        "scan": None,   # the group totals: a few KB whose count depends on the binning plan
        "bin_write": BN * 8 + B * nT * 4 + pairs_tiles * 4,
        "forward_raster": pairs_tiles * 4 + BN * (32 + C * 4) + img,
        "zero_verify": BN * P * 4,
        "backward_raster": pairs_tiles * 4 + BN * (32 + C * 4) + img + 2 * BN * P * 4,
        "finalize": 2 * BN * P * 4 + BN * P * 4,
    }


def loss_flops_bytes(B, H, W, C):
    """Algorithmic work of the L1 + SSIM loss per launch pair, per value:
    forward 3 products + 2 x (5 quantities x 11 taps x 2) window flops + 20
    for SSIM and its three partials; gradient 2 x (3 x 11 x 2) + 8.  HBM:
    forward reads I, T and writes three partial maps (20 B), gradient reads
    the maps, I, T and writes dL/dI (24 B)."""
    M = B * H * W * C
    return {"loss_fwd": (M * (3 + 220 + 20), M * 20), "loss_bwd": (M * (132 + 8), M * 24)}


def adapter_leg(args, _lib, torch, B, N, H, W, C, params, image, grad_image, target, ws, ws_bytes,
                st, step):
    """Grid initialisation, activation and its gradient on a square grid of N
    Gaussians per frame, and the concat-fused step ([target | render] with
    Cp = C) against the plain step; HIP-event timing of every launch."""
    g = int(round(N ** 0.5))
    if g * g != N:
        return None
    P = 5 + C
    dev = params.device
    raw = torch.empty_like(params)
    act = torch.empty_like(params)
    graw = torch.empty_like(params)
    out = torch.empty((B, H, W, 2 * C), dtype=torch.float32, device=dev)
    gout = torch.cat([grad_image, grad_image], dim=-1).contiguous()
    gparams = torch.empty_like(params)
    gpix = torch.empty_like(image)

    def ops():
        _lib.pdr_grid_init(raw.data_ptr(), B, g, g, H, W, C, 0.5, target.data_ptr(), st)
        _lib.pdr_params_activate(raw.data_ptr(), act.data_ptr(), B, g, g, H, W, C, st)
        # (the activated values stand in for dL/dparams)
        _lib.pdr_params_activate_backward(raw.data_ptr(), act.data_ptr(), graw.data_ptr(), B, g, g,
                                          H, W, C, st)

    def concat_step():
        _lib.pdr_splat_forward_concat(params.data_ptr(), target.data_ptr(), C, out.data_ptr(), B,
                                      N, H, W, C, args.radius, ws.data_ptr(), ws_bytes, st)
        _lib.pdr_splat_backward_concat(params.data_ptr(), gout.data_ptr(), C, gparams.data_ptr(),
                                       gpix.data_ptr(), B, N, H, W, C, args.radius, ws.data_ptr(),
                                       ws_bytes, 1, st)

    for _ in range(args.warmup):
        ops()
        concat_step()
    _lib.pdr_splat_timing(True)
    _lib.pdr_splat_timing_read(reset=True)
    for _ in range(args.steps):
        ops()
    torch.cuda.synchronize()
    t = _lib.pdr_splat_timing_read(reset=True)
    _lib.pdr_splat_timing(False)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {"grid": "%dx%d" % (g, g), "kernels": {}}
    per = B * N * P * 4
    nbytes = {"grid_init": per + B * N * C * 4, "activate": 2 * per,
              "activate_bwd": 2 * per + B * N * 4 * 4}
    for name in ("grid_init", "activate", "activate_bwd"):
        tot, cnt = t[name]
        avg = tot / cnt
        res["kernels"][name] = {"avg_ms": round(avg, 5),
                                "alg_GBps": round(nbytes[name] / (avg * 1e-3) / 1e9, 1),
                                "hbm_frac": round(nbytes[name] / (avg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    for name, fn in (("plain_step_ms", step), ("concat_step_ms", concat_step)):
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = round(e0.elapsed_time(e1) / args.steps, 5)
    res["concat_extra_bytes"] = 4 * B * H * W * C * 4   # pixel read + write, gradient read + write
    return res


def backward_algo_leg(args, _lib, torch, B, N, H, W, C, params, grad_image, grad_params, ws,
                      ws_bytes, st):
    """The backward alone (reusing the forward's binning) with each algorithm:
    the tile raster and the tile-free span walk (C <= 16)."""
    out = {}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for name, algo in (("tile", _lib.PDR_BWD_TILE), ("span", _lib.PDR_BWD_SPAN)):
        if algo == _lib.PDR_BWD_SPAN and C > 16:
            continue

        def run():
            _lib.pdr_splat_backward_algo(params.data_ptr(), grad_image.data_ptr(), 0,
                                         grad_params.data_ptr(), B, N, H, W, C, args.radius,
                                         ws.data_ptr(), ws_bytes, 1, algo, st)
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        out[name + "_backward_ms"] = round(e0.elapsed_time(e1) / args.steps, 5)
    return out


# Kernel classes of the per-kernel timing, by kernel name prefix (rocprofv3
# names kernels "pdr::k_...(args)").
KERNEL_CLASSES = (("k_preprocess", "preprocess"), ("k_rows<", "bin_count"),
                  ("k_rowscan", "bin_count"), ("k_rowstart", "bin_count"),
                  ("k_bin<false", "bin_count"), ("k_count_scan", "scan"),
                  ("k_bin<true", "bin_write"), ("k_forward<", "forward_raster"),
                  ("k_zero_verify", "zero_verify"), ("k_backward<", "backward_raster"),
                  ("k_finalize", "finalize"))
CSRC = "differentiable_gaussian_splatting_pdr_amd/csrc"


def kernel_sources():
    """Every file the library is built from: a summary of counters or
    durations is only valid for the build it was taken on."""
    files = sorted(os.path.join(CSRC, f) for f in os.listdir(os.path.join(ROOT, CSRC))
                   if f.endswith((".hip", ".hpp")))
    return files + ["include/pdr_splat.h", "differentiable_gaussian_splatting_pdr_amd/build.py"]


def short_kernel_name(name):
    import re
    m = re.search(r"\b(k_\w+(<[^(]*>)?)", name)
    return m.group(1) if m else name.split("(")[0][:60]


def kernel_class(short):
    for prefix, cls in KERNEL_CLASSES:
        if short.startswith(prefix):
            return cls
    return None


def sizes_tag(wl):
    return "%dx%dx%dx%d_n%d" % (wl.B, wl.H, wl.W, wl.C, wl.N)


def workload_text(wl, radius):
    return "%d frames of %dx%dx%d, N=%d Gaussians/frame, %g-sigma truncation" % (
        wl.B, wl.H, wl.W, wl.C, wl.N, radius)


def _find_csv(d, suffix):
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return hits


def summarize(args):
    """Summaries of rocprofv3 output for profiles/ (host only)."""
    import csv
    import statistics
    from differentiable_gaussian_splatting_pdr_amd import workloads
    wl = workloads.WORKLOADS[args.workload]
    tag = sizes_tag(wl)
    srcs = kernel_sources()
    if args.summarize_trace:
        rows = []
        for f in _find_csv(args.summarize_trace, "kernel_trace.csv"):
            rows += list(csv.DictReader(open(f)))
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        per = {}
        for r in rows:
            k = short_kernel_name(r["Kernel_Name"])
            per.setdefault(k, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
        last = args.profile_loop
        kernels, classes = {}, {}
        for k, v in per.items():
            tail = v[-last:] if last else v
            kernels[k] = {"calls": len(v), "avg_us_all": round(statistics.mean(v), 2),
                          "min_us": round(min(v), 2), "max_us": round(max(v), 2),
                          "avg_us_last": round(statistics.mean(tail), 2), "last": len(tail),
                          "class": kernel_class(k)}
            if kernel_class(k) and len(v) >= last:
                c = kernel_class(k)
                classes[c] = round(classes.get(c, 0.0) + statistics.mean(tail), 2)
        stats = []
        for f in _find_csv(args.summarize_trace, "kernel_stats.csv"):
            stats += list(csv.DictReader(open(f)))
        out = {"workload": workload_text(wl, args.radius), "command": args.command,
               "warmup_steps": args.warmup, "profiled_steps": last, "sources": srcs,
               "source_digest": source_digest(srcs), "kernels": kernels,
               "class_avg_us_last": classes,
               "note": "avg_us_last: mean over each kernel's last profiled_steps dispatches "
                       "(steady clocks); avg_us_all: over every dispatch of the run, the "
                       "figure of rocprofv3 --stats"}
        jpath = os.path.join(ROOT, "profiles", "kernel_trace_%s.json" % tag)
        with open(jpath, "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")
        md = ["# Kernel trace: %s, MI355X" % workload_text(wl, args.radius), "",
              "Command (from /tmp with TMPDIR=/tmp; `<repo>` is the repository root):", "",
              "    " + args.command, "",
              "Summarised by `python3 bench.py --summarize-trace <dir> --warmup %d "
              "--profile-loop %d --workload %d`.  The program runs one checked step, %d "
              "warm-up steps and %d profiled steps (forward + backward reusing the binning)."
              % (args.warmup, last, args.workload, args.warmup, last), "",
              "rocprofv3 `--stats` (every dispatch of the run):", "",
              "| kernel | calls | avg us | min us | max us | % GPU time |", "|---|---|---|---|---|---|"]
        for r in sorted(stats, key=lambda r: -float(r["TotalDurationNs"])):
            md.append("| `%s` | %s | %.1f | %.1f | %.1f | %.1f |" % (
                short_kernel_name(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, float(r["Percentage"])))
        md += ["", "Steady state, mean over each kernel's last %d dispatches of the trace:" % last,
               "", "| kernel | class | avg us (last %d) | avg us (all) |" % last, "|---|---|---|---|"]
        for k, v in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_us_last"]):
            if v["calls"] >= last:
                md.append("| `%s` | %s | %.1f | %.1f |" % (k, v["class"], v["avg_us_last"],
                                                            v["avg_us_all"]))
        md += ["", "bench.py reads the `class_avg_us_last` figures from `kernel_trace_%s.json` "
               "(when its source digest matches the build) and reports the roofline of the "
               "dominant kernel from both its live HIP-event timing and this trace." % tag, ""]
        with open(os.path.join(ROOT, "profiles", "kernel_trace_%s.md" % tag), "w") as fh:
            fh.write("\n".join(md))
        print(json.dumps({"written": [os.path.relpath(jpath, ROOT)], "classes": classes}))
    if args.summarize_pmc:
        vals = {}
        for d, counter in zip(args.summarize_pmc, ("FETCH_SIZE", "WRITE_SIZE")):
            for f in _find_csv(d, "counter_collection.csv"):
                for r in csv.DictReader(open(f)):
                    if r["Counter_Name"] != counter:
                        continue
                    k = short_kernel_name(r["Kernel_Name"])
                    vals.setdefault((counter, k), []).append(float(r["Counter_Value"]))
        if not args.calib_copy_mb:
            raise SystemExit("--summarize-pmc needs --calib-copy-mb (the reference copy's size)")
        true_kib = args.calib_copy_mb * 1024.0
        out = {"kernel": args.kernel, "workload": workload_text(wl, args.radius),
               "sources": srcs, "source_digest": source_digest(srcs),
               "commands": args.command.split(" && ") if args.command else []}
        total = 0.0
        for counter, key in (("FETCH_SIZE", "fetch"), ("WRITE_SIZE", "write")):
            copies = [max(v) for (c, k), v in vals.items() if c == counter and "copyBuffer" in k]
            if not copies:
                raise SystemExit("no reference copy in the %s run" % counter)
            scale = true_kib / max(copies)
            ks = [(k, v) for (c, k), v in vals.items()
                  if c == counter and kernel_class(k) == args.kernel]
            if len(ks) != 1:
                raise SystemExit("kernel class %s: %d kernels in the %s run" % (
                    args.kernel, len(ks), counter))
            k, v = ks[0]
            b = statistics.median(v) * 1024.0 * scale
            out[key + "_bytes"] = b
            out[key + "_scale"] = scale
            out["kernel_name"] = k
            total += b
        out["bytes_per_launch"] = total
        out["scaling_rule"] = ("median KiB per dispatch x 1024, times the ratio of a %d MiB "
                               "copy's true bytes to what the same counter reads for it"
                               % args.calib_copy_mb)
        path = os.path.join(ROOT, "profiles", "traffic_%s_%s.json" % (args.kernel, tag))
        with open(path, "w") as fh:
            json.dump(out, fh, indent=1)
            fh.write("\n")
        print(json.dumps({"written": os.path.relpath(path, ROOT),
                          "bytes_per_launch": total}))


def source_digest(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def cpu_baseline_leg(params, grad, wl, radius, budget_s, want_count=True):
    """The oracle (fp64 CPU) timed on this host's cores on a bounded sample of
    the workload's frames; also counts the support pairs of the full batch
    (a cross-check of the GPU's count)."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    threads = oracle.default_threads()
    total_pairs = None
    if want_count:
        total_pairs = int(oracle.count_support(params, wl.H, wl.W, radius, nthreads=threads).sum())
    # size the sample from a 4-frame probe so the timed run is ~budget_s
    probe = min(4, wl.B)
    t0 = time.perf_counter()
    oracle.render(params[:probe], wl.H, wl.W, radius, extras=False, nthreads=threads)
    oracle.grad(params[:probe], grad[:probe], wl.H, wl.W, radius, extras=False, nthreads=threads)
    per_frame = (time.perf_counter() - t0) / probe * min(probe, threads)
    frames = int(max(1, min(wl.B, budget_s * threads / max(per_frame, 1e-6))))
    frames = max(1, (frames // threads) * threads) if frames >= threads else frames
    sp, sg = params[:frames], grad[:frames]
    t0 = time.perf_counter()
    _, _, _, pairs = oracle.render(sp, wl.H, wl.W, radius, extras=False, nthreads=threads)
    oracle.grad(sp, sg, wl.H, wl.W, radius, extras=False, nthreads=threads)
    dt = time.perf_counter() - t0
    # one frame on one thread
    t1 = time.perf_counter()
    _, _, _, p1 = oracle.render(params[:1], wl.H, wl.W, radius, extras=False, nthreads=1)
    oracle.grad(params[:1], grad[:1], wl.H, wl.W, radius, extras=False, nthreads=1)
    dt1 = time.perf_counter() - t1
    return {
        "value": float(pairs.sum()) / dt,
        "unit": "evals/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "%d of %d frames, forward+backward, fp64 C, %.2f s wall" % (frames, wl.B, dt),
        "frames_per_s": frames / dt,
        "one_thread_evals_per_s": float(p1.sum()) / dt1,
    }, total_pairs


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first: the rasters' launch durations settle over about "
                         "the first 40 launches of a run while the clocks ramp")
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--radius", type=float, default=3.0)
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="target wall seconds of the oracle baseline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile-loop", type=int, default=0,
                    help="only run --warmup and then this many steps (for rocprofv3), print "
                         "nothing else")
    ap.add_argument("--with-loss", action="store_true",
                    help="with --profile-loop: also run the L1 + SSIM loss each step")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="with --profile-loop: also run one device-to-device copy of this many "
                         "MiB, the reference kernel for scaling HBM byte counters")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="no GPU: write profiles/kernel_trace_<sizes>.{json,md} from the "
                         "rocprofv3 --kernel-trace --stats output in DIR of a --profile-loop run "
                         "(pass the same --workload, --warmup and --profile-loop)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU: write profiles/traffic_<kernel>_<sizes>.json from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of a --profile-loop run "
                         "with --calib-copy-mb (pass the same --calib-copy-mb)")
    ap.add_argument("--kernel", default="backward_raster",
                    help="with --summarize-pmc: the kernel class to summarise")
    ap.add_argument("--command", default="",
                    help="with --summarize-*: the rocprofv3 command(s) that made the input, "
                         "recorded in the summary ('<repo>' for the repository root)")
    args = ap.parse_args()
    if args.summarize_trace or args.summarize_pmc:
        summarize(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(frames are independent; see the design notes on sharding)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from differentiable_gaussian_splatting_pdr_amd import _lib, workloads

    wl, params_np, grad_np = workloads.make_inputs(args.workload)
    B, N, H, W, C = wl.B, wl.N, wl.H, wl.W, wl.C
    dev = torch.device("cuda:0")
    params = torch.from_numpy(params_np).to(dev)
    grad_image = torch.from_numpy(grad_np).to(dev)
    image = torch.empty((B, H, W, C), dtype=torch.float32, device=dev)
    grad_params = torch.empty_like(params)
    st = torch.cuda.current_stream(dev).cuda_stream

    # exact list capacity from one binning pass
    ws_fixed = _lib.pdr_splat_workspace_bytes(B, N, H, W, C, 0)
    T = _lib.pdr_splat_tile_size()
    nT = ((H + T - 1) // T) * ((W + T - 1) // T)
    probe = torch.empty(ws_fixed, dtype=torch.uint8, device=dev)
    off = torch.empty(B * nT + 1, dtype=torch.int32, device=dev)
    lst = torch.empty(1, dtype=torch.int32, device=dev)
    _lib.pdr_splat_bin(params.data_ptr(), B, N, H, W, C, args.radius, off.data_ptr(),
                       lst.data_ptr(), 0, probe.data_ptr(), ws_fixed, st)
    _, tile_pairs = _lib.pdr_splat_check(probe.data_ptr(), st)
    del probe, off, lst
    ws_bytes = _lib.pdr_splat_workspace_bytes(B, N, H, W, C, tile_pairs)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    # the work count: (Gaussian, pixel) pairs inside the truncation, on the GPU
    count = torch.zeros(1, dtype=torch.int64, device=dev)
    _lib.pdr_splat_count_support(params.data_ptr(), B, N, H, W, C, args.radius,
                                 count.data_ptr(), ws.data_ptr(), ws_bytes, st)
    rc, _ = _lib.pdr_splat_check(ws.data_ptr(), st)
    if rc != 0:
        raise SystemExit("support count failed: %s" % _lib.status_string(rc))
    support_pairs = int(count.item())

    def step():
        _lib.pdr_splat_forward(params.data_ptr(), image.data_ptr(), B, N, H, W, C, args.radius,
                               ws.data_ptr(), ws_bytes, st)
        _lib.pdr_splat_backward(params.data_ptr(), grad_image.data_ptr(), grad_params.data_ptr(),
                                B, N, H, W, C, args.radius, ws.data_ptr(), ws_bytes, 1, st)

    step()
    rc, _ = _lib.pdr_splat_check(ws.data_ptr(), st)
    if rc != 0:
        raise SystemExit("first step failed: %s" % _lib.status_string(rc))

    # training loss on the rendered frames against a seeded synthetic target
    _, target_np = workloads.make_loss_inputs(B, H, W, C, seed=1000 + args.workload)
    target = torch.from_numpy(target_np).to(dev)
    del target_np
    loss_ws_bytes = _lib.pdr_loss_workspace_bytes(B, H, W, C)
    loss_ws = torch.empty(loss_ws_bytes, dtype=torch.uint8, device=dev)
    loss_val = torch.empty((), dtype=torch.float64, device=dev)
    loss_grad = torch.empty_like(image)

    def loss_step():
        _lib.pdr_loss_l1_ssim(image.data_ptr(), target.data_ptr(), B, H, W, C, 0.2, 1e-4, 9e-4,
                              loss_grad.data_ptr(), loss_val.data_ptr(), loss_ws.data_ptr(),
                              loss_ws_bytes, st)

    if args.profile_loop:
        # warm-up steps first (the clocks ramp over the first launches), then
        # the profiled steps; summaries use the last profile_loop dispatches
        for _ in range(args.warmup + args.profile_loop):
            step()
            if args.with_loss:
                loss_step()
        if args.calib_copy_mb:
            n = args.calib_copy_mb << 20
            src = torch.ones(n // 4, dtype=torch.float32, device=dev)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
        torch.cuda.synchronize()
        print("profile loop done: %d steps" % args.profile_loop, flush=True)
        return

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: K steps, events on the launch stream and a host clock
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    host_ms = (time.perf_counter() - h0) * 1e3 / args.steps
    ms = e0.elapsed_time(e1) / args.steps

    # per-kernel durations: the same K steps with HIP events around every launch
    _lib.pdr_splat_timing(True)
    _lib.pdr_splat_timing_read(reset=True)
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms_events = e0.elapsed_time(e1) / args.steps
    per_kernel = _lib.pdr_splat_timing_read(reset=True)
    _lib.pdr_splat_timing(False)
    rc, _ = _lib.pdr_splat_check(ws.data_ptr(), st)
    if rc != 0:
        raise SystemExit("timed steps failed: %s" % _lib.status_string(rc))

    # the loss: same K, HIP events around every launch
    for _ in range(args.warmup):
        loss_step()
    _lib.pdr_splat_timing(True)
    _lib.pdr_splat_timing_read(reset=True)
    e0.record()
    for _ in range(args.steps):
        loss_step()
    e1.record()
    torch.cuda.synchronize()
    loss_ms = e0.elapsed_time(e1) / args.steps
    loss_kernels = _lib.pdr_splat_timing_read(reset=True)
    _lib.pdr_splat_timing(False)
    lfb = loss_flops_bytes(B, H, W, C)
    loss_out = {"ms": round(loss_ms, 5), "values_per_s": B * H * W * C / (loss_ms * 1e-3),
                "lambda": 0.2, "kernels": {}}
    for name in ("loss_fwd", "loss_bwd", "loss_reduce"):
        tot, cnt = loss_kernels[name]
        if not cnt:
            continue
        avg = tot / cnt
        row = {"avg_ms": round(avg, 5)}
        if name in lfb:
            fl, by = lfb[name]
            row["alg_TFLOPs"] = round(fl / (avg * 1e-3) / 1e12, 3)
            row["alg_GBps"] = round(by / (avg * 1e-3) / 1e9, 1)
        loss_out["kernels"][name] = row
    ldom = max(lfb, key=lambda k: loss_out["kernels"][k]["avg_ms"])
    lach = loss_out["kernels"][ldom]["alg_TFLOPs"]
    loss_out["roofline"] = {"bound": "alu", "kernel": ldom, "achieved": lach,
                            "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(lach / FP32_PEAK_TFLOPS, 4),
                            "hbm_frac": round(loss_out["kernels"][ldom]["alg_GBps"] / HBM_PEAK_GBS, 4)}

    adapter_out = adapter_leg(args, _lib, torch, B, N, H, W, C, params, image, grad_image, target,
                              ws, ws_bytes, st, step)
    algo_out = backward_algo_leg(args, _lib, torch, B, N, H, W, C, params, grad_image, grad_params,
                                 ws, ws_bytes, st)

    cpu = None
    if not args.no_cpu_baseline:
        cpu, oracle_pairs = cpu_baseline_leg(params_np, grad_np, wl, args.radius, args.cpu_budget)
        # cross-check of the work count: the fp64 count differs only by pairs
        # whose q is within rounding of the truncation boundary
        cpu["support_pairs_oracle"] = oracle_pairs
        cpu["support_pairs_rel_diff"] = abs(oracle_pairs - support_pairs) / max(oracle_pairs, 1)

    f_fwd, f_bwd = flops_per_pair(C)
    kernels = {}
    kb = kernel_bytes(B, N, H, W, C, tile_pairs, T)
    for name, (tot_ms, cnt) in per_kernel.items():
        if cnt == 0:
            continue
        avg = tot_ms / cnt
        row = {"avg_ms": round(avg, 5), "launches_per_step": cnt // args.steps}
        if kb.get(name) is not None:
            row["alg_GBps"] = round(kb[name] / (avg * 1e-3) / 1e9, 1)
        if support_pairs is not None and name in ("forward_raster", "backward_raster"):
            fl = support_pairs * (f_fwd if name == "forward_raster" else f_bwd)
            row["alg_TFLOPs"] = round(fl / (avg * 1e-3) / 1e12, 3)
        kernels[name] = row
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    roofline = None
    if support_pairs is not None:
        fl = support_pairs * (f_fwd if dom == "forward_raster" else f_bwd)
        avg = kernels[dom]["avg_ms"] * 1e-3
        ach = fl / avg / 1e12
        tag = sizes_tag(wl)

        def committed(name):
            # a profiles/ summary, if it was taken on the sources built here
            path = os.path.join(ROOT, "profiles", name)
            if not os.path.exists(path):
                return None, path
            with open(path) as fh:
                t = json.load(fh)
            ok = t.get("sources") == kernel_sources() and \
                t.get("source_digest") == source_digest(t.get("sources", []))
            return (t if ok else None), path

        t, tpath = committed("traffic_%s_%s.json" % (dom, tag))
        traffic = t.get("bytes_per_launch") if t else None
        t, kpath = committed("kernel_trace_%s.json" % tag)
        traced = None
        if t and dom in t.get("class_avg_us_last", {}):
            tus = t["class_avg_us_last"][dom]
            tach = fl / (tus * 1e-6) / 1e12
            traced = {"avg_launch_ms": round(tus * 1e-3, 5), "achieved": round(tach, 3),
                      "frac": round(tach / FP32_PEAK_TFLOPS, 4),
                      "profile": os.path.relpath(kpath, ROOT)}
        roofline = {"bound": "alu", "achieved": round(ach, 3), "peak": FP32_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(ach / FP32_PEAK_TFLOPS, 4),
                    "traffic": traffic, "kernel": dom,
                    "flops_per_launch": fl, "avg_launch_ms": kernels[dom]["avg_ms"],
                    "alg_bytes_per_launch": kb[dom],
                    "traffic_profile": os.path.relpath(tpath, ROOT) if traffic else None,
                    "traced": traced}
    value = support_pairs / (ms * 1e-3) if support_pairs is not None else None
    out = {
        "metric": "fwd+bwd Gaussian-pixel evals/s and frames/s at 128x128x3, N=4096; % FP32 peak",
        "value": value,
        "unit": "evals/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%d frames of %dx%dx%d, N=%d Gaussians/frame, 3-sigma truncation"
                   % (B, H, W, C, N), "frames": B, "H": H, "W": W, "C": C,
                   "gaussians_per_frame": N, "radius": args.radius},
        "frames_per_s": B / (ms * 1e-3),
        "support_pairs": support_pairs,
        "tile_pairs": int(tile_pairs),
        # every listed (tile, Gaussian) entry spans T*T pixel lanes; the
        # support pairs among them show the lane waste before unit culling
        "tile_lane_pairs": int(tile_pairs) * T * T,
        "tile_lane_efficiency": (round(support_pairs / (int(tile_pairs) * T * T), 4)
                                 if support_pairs and tile_pairs else None),
        "fp32_peak_frac_fwd_bwd": (round(support_pairs * (f_fwd + f_bwd) / (ms * 1e-3) / 1e12
                                         / FP32_PEAK_TFLOPS, 4) if support_pairs else None),
        "ms_per_step_host": round(host_ms, 5),
        "ms_per_step_with_kernel_events": round(ms_events, 5),
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "loss": loss_out,
        "adapter": adapter_out,
        "backward_algorithms": algo_out,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
