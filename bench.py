#!/usr/bin/env python3
"""Benchmark: InstanceNorm2d fp32 on x[112,64,512,512] (7168 slices x 262144), one MI355X.

A step is one inorm_forward call over the whole tensor (statistics + normalize, inputs already
in HBM). The metric is effective bandwidth = minimum algorithmic bytes / time, with
min bytes = 4*N*C*H*W read + 4*N*C*H*W written = 15,032,385,536 B, against the 8 TB/s HBM peak.

Prints ONE JSON line on stdout (progress goes to stderr):
  value / ms_per_step  from HIP events around the K timed steps on the launch stream;
  roofline             the dominant kernel's achieved GB/s = algorithmic bytes per launch /
                       its average launch duration (events around each launch), vs 8000 GB/s;
                       traffic = HBM bytes per launch from the committed rocprofv3 counter
                       summary when it was taken on the current kernel source, else null;
  cpu_baseline         the fp64 oracle timed on a bounded sample of the same slices on the
                       host cores (rank 0, one GPU), with the sample's max |gpu - oracle|;
  copy_ceiling_GBps    the fastest streaming copy of the same bytes (the library's persistent
                       copy), and pct_of_copy_ceiling = roofline.achieved against it;
  config.input_sha256  SHA-256 of x's bytes (the other inputs' hashes are in extra);
  extra                the one-shot copy (the counters' calibration kernel) and the other
                       workloads' times (skipped with --no-extra).
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

HBM_PEAK_GBPS = 8000.0
N, C, H, W = 112, 64, 512, 512
S = H * W
MIN_BYTES = 2 * 4 * N * C * S
METRIC = "InstanceNorm2d fp32 effective GB/s (min bytes/time) and % of HBM peak, 1 GPU"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "inorm_pipelined_112x64x512x512_traffic.json")
KERNEL_SOURCES = ["normalization_reductions_amd/csrc/resident_norm.hip",
                  "normalization_reductions_amd/csrc/resident.hpp",
                  "normalization_reductions_amd/csrc/common.hpp"]


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def committed_traffic():
    """HBM bytes per launch from the committed counter summary, if it matches this source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None, "no committed counter summary"
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None, "kernel source changed since the counters were taken"
    return t.get("hbm_bytes_per_launch"), "from %s" % os.path.relpath(TRAFFIC_FILE, ROOT)


HEADLINE_KERNEL = "norm_pipelined_kernel<256, 16, false, false>"
COPY_KERNEL = "copy_vec_kernel"


def _counter_rows(path, counter, needle, before=None):
    """Counter values of the dispatches of kernel `needle`, in dispatch order; with `before`,
    only those dispatched before the first dispatch of kernel `before`."""
    import csv

    with open(path, newline="") as f:
        rows = [r for r in csv.DictReader(f) if r["Counter_Name"] == counter]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    if before is not None:
        first = next((int(r["Dispatch_Id"]) for r in rows if before in r["Kernel_Name"]), None)
        if first is not None:
            rows = [r for r in rows if int(r["Dispatch_Id"]) < first]
    return [float(r["Counter_Value"]) for r in rows if needle in r["Kernel_Name"]]


def traffic_summary(fetch_csv, write_csv):
    """Host-only: turn two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE;
    csv output) into the per-launch HBM byte count of the headline kernel. Each counter is
    calibrated by what it reads for the plain copy kernel of the same run, which moves exactly
    MIN_BYTES / 2 each way. Only the headline launches count: those before the copy kernel's
    first launch (the smaller workloads timed afterwards launch the same kernel)."""
    kf = _counter_rows(fetch_csv, "FETCH_SIZE", HEADLINE_KERNEL, before=COPY_KERNEL)
    kw = _counter_rows(write_csv, "WRITE_SIZE", HEADLINE_KERNEL, before=COPY_KERNEL)
    cf = _counter_rows(fetch_csv, "FETCH_SIZE", COPY_KERNEL)
    cw = _counter_rows(write_csv, "WRITE_SIZE", COPY_KERNEL)
    if not (kf and kw and cf and cw):
        raise SystemExit("counter files lack the headline or the copy kernel")
    # the same copy kernel also makes the smaller workloads' cold copies: calibrate on the
    # dispatches of the headline's bytes (the largest) alone
    cf = [v for v in cf if v > 0.5 * max(cf)]
    cw = [v for v in cw if v > 0.5 * max(cw)]
    mean = lambda v: sum(v) / len(v)
    each_way = MIN_BYTES // 2
    fs = each_way / (mean(cf) * 1024)
    ws = each_way / (mean(cw) * 1024)
    rd = mean(kf) * 1024 * fs
    wr = mean(kw) * 1024 * ws
    t = {
        "kernel": HEADLINE_KERNEL,
        "workload": "InstanceNorm2d x[112,64,512,512] fp32",
        "fetch_size_kib_per_launch": kf, "write_size_kib_per_launch": kw,
        "copy_kernel_fetch_kib": cf, "copy_kernel_write_kib": cw,
        "copy_bytes_each_way": each_way,
        "fetch_scale": round(fs, 6), "write_scale": round(ws, 6),
        "hbm_read_bytes_per_launch": int(rd), "hbm_write_bytes_per_launch": int(wr),
        "hbm_bytes_per_launch": int(rd + wr), "algorithmic_bytes_per_launch": MIN_BYTES,
        "traffic_over_algorithmic": round((rd + wr) / MIN_BYTES, 5),
        "kernel_source_files": KERNEL_SOURCES, "kernel_source_sha256": kernel_source_hash(),
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(t, f, indent=1)
        f.write("\n")
    print(json.dumps(t, indent=1))
    return 0


def time_calls(fn, steps, warmup, torch, flush=None):
    """Returns (total ms for `steps` calls, mean and median ms per call measured around each
    call). `flush`, if given, runs before each call outside the per-call events."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    t0.record()
    for k in range(steps):
        if flush is not None:
            flush()
        starts[k].record()
        fn()
        ends[k].record()
    t1.record()
    torch.cuda.synchronize()
    total = t0.elapsed_time(t1)
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    time_calls.last = sorted(per)  # per-call durations of the latest timing, ascending
    return total, sum(per) / len(per), sorted(per)[len(per) // 2]


def host_description():
    """CPU model, logical CPUs and NUMA nodes of the host running the oracle."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        nodes = len([d for d in os.listdir("/sys/devices/system/node")
                     if d.startswith("node") and d[4:].isdigit()])
    except OSError:
        nodes = None
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "numa_nodes": nodes}


def cpu_baseline(x, y, budget_s, torch):
    """fp64 oracle on the first M slices, M sized to ~budget_s of CPU time."""
    import numpy as np

    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)
    xv = x.view(N * C, S)
    yv = y.view(N * C, S)
    m0 = 16
    xs = xv[:m0].cpu().numpy()
    t = time.perf_counter()
    oracle.instance_norm_slices(xs, nthreads=threads)
    t_cal = max(time.perf_counter() - t, 1e-3)
    m = int(min(N * C, max(m0, m0 * budget_s / t_cal)))
    m = max(threads, m // threads * threads)
    xs = xv[:m].cpu().numpy()
    t = time.perf_counter()
    ref = oracle.instance_norm_slices(xs, nthreads=threads)
    dt = time.perf_counter() - t
    ys = yv[:m].cpu().numpy()
    err = float(np.max(np.abs(ys.astype(np.float64) - ref)))
    gbps = (2 * 4 * m * S) / dt / 1e9
    log("cpu oracle: %d slices in %.2f s on %d threads -> %.3f GB/s; sample max_abs_err %.3e"
        % (m, dt, threads, gbps, err))
    return ({"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
             "sample": "first %d of %d slices (%d x 262144 fp32), fp64 oracle, %.1f s wall"
                       % (m, N * C, m, dt),
             "wall_s": round(dt, 3), "host": host_description()},
            {"slices": m, "max_abs_err": err})


def sha256_device(t, torch, chunk_bytes=256 << 20):
    """SHA-256 of a device tensor's bytes (row-major), copied to the host in chunks."""
    h = hashlib.sha256()
    flat = t.reshape(-1).view(torch.uint8)
    for lo in range(0, flat.numel(), chunk_bytes):
        h.update(flat[lo:lo + chunk_bytes].cpu().numpy().tobytes())
    return h.hexdigest()


def sha256_host(a):
    import numpy as np

    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def copy_ceiling(torch, nra, x, y, steps, warmup):
    """The fastest streaming copy of the same bytes (the library's persistent copy: one
    workgroup per CU taking 64 KiB units from a counter): the practical HBM ceiling."""
    cws = torch.zeros(256, dtype=torch.uint8, device=x.device)
    tot, per, med = time_calls(lambda: nra.stream_copy(x, y, workspace=cws), steps, warmup, torch)
    gbps = MIN_BYTES / (per / 1e3) / 1e9
    log("persistent copy of the same bytes (the ceiling): %.3f ms -> %.1f GB/s" % (per, gbps))
    return gbps


CONFIGS = {
    1: "InstanceNorm2d fp32, affine=False, eps=1e-5: x[2,4,32,32] ~ N(0,1)*s+o, per slice "
       "s~U(0.5,2), o~U(-3,3)",
    2: "InstanceNorm2d fp32, affine=False, eps=1e-5: x[16,64,256,256], per slice o~U(-100,100), "
       "s~U(0.1,10) on N(0,1)",
    3: "InstanceNorm2d fp32, affine=False, eps=1e-5: x[112,64,512,512] ~ N(0,1)",
    4: "Conv2d(8->64,k=3,valid,bias) on x[128,8,64,64]~N(0,1); training-mode BatchNorm2d, "
       "eps=1e-5; x2.0",
    5: "Conv3d(3->16,k=3,valid,bias) on x[128,3,16,32,32]~N(0,1); x multiplier; InstanceNorm3d; "
       "clamp[-1,1]; x multiplier; max over C",
}


def config_results(torch, nra, head, x3_sha, steps, warmup, out_dir):
    """Part of the CPU-baseline leg: one JSON file per workload in out_dir, with its GPU time
    (HIP events around each call; workloads 1, 2, 4, 5 after a 512 MB read that empties the
    caches), the fp64 oracle's time on the host cores over the same inputs, and the maximum
    |gpu - oracle| over every output element. Workload 3 reuses the headline's measurements."""
    import numpy as np

    import oracle
    import synth

    os.makedirs(out_dir, exist_ok=True)
    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush = lambda: scrub.sum()
    threads = int(os.environ.get("OMP_NUM_THREADS") or os.cpu_count() or 1)

    def record(cfg, rec):
        rec = dict({"config": cfg, "workload": CONFIGS[cfg], "tolerance_max_abs": 1e-4,
                    "oracle": "fp64 CPU oracle (oracle/oracle.c), %d threads" % threads}, **rec)
        with open(os.path.join(out_dir, "config%d.json" % cfg), "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        log("config %d: %s" % (cfg, json.dumps({k: rec[k] for k in ("gpu_ms_median", "max_abs_err_vs_oracle")})))

    def gpu_time(fn):
        tot, mean, med = time_calls(fn, steps, warmup, torch, flush)
        return {"gpu_ms_median": round(med, 5), "gpu_ms_mean": round(mean, 5),
                "gpu_ms_min": round(time_calls.last[0], 5)}

    for cfg in (1, 2):
        inp = synth.host_inputs(cfg)
        x = T(inp["x"])
        y = torch.empty_like(x)
        rec = gpu_time(lambda: nra.inorm_forward(x, y, eps=inp["eps"]))
        torch.cuda.synchronize()
        t = time.perf_counter()
        ref = oracle.instance_norm(inp["x"], eps=inp["eps"], nthreads=threads)
        dt = time.perf_counter() - t
        nbytes = 2 * 4 * x.numel()
        rec.update({"shape": list(inp["x"].shape), "input_sha256": {"x": sha256_host(inp["x"])},
                    "min_bytes": nbytes, "GBps": round(nbytes / (rec["gpu_ms_median"] / 1e3) / 1e9, 1),
                    "oracle_s": round(dt, 3),
                    "max_abs_err_vs_oracle": float(np.max(np.abs(y.cpu().numpy().astype(np.float64) - ref))),
                    "elements_compared": int(x.numel())})
        record(cfg, rec)
        del x, y
    record(3, {"shape": [N, C, H, W], "input_sha256": {"x": x3_sha}, "min_bytes": MIN_BYTES,
               "gpu_ms_median": head["median"], "gpu_ms_mean": head["mean"], "gpu_ms_min": head["min"],
               "GBps": round(MIN_BYTES / (head["median"] / 1e3) / 1e9, 1),
               "timing": "HIP events around each call, inputs resident, no cache emptying (15 GB)",
               "oracle_s": head["oracle_s"], "max_abs_err_vs_oracle": head["max_abs_err"],
               "elements_compared": head["elements"]})
    conv_gflop = {4: 2 * 128 * 64 * 62 * 62 * 72 / 1e9, 5: 2 * 128 * 16 * 12600 * 81 / 1e9}
    for cfg in (4, 5):
        inp = synth.host_inputs(cfg)
        a = (T(inp["x"]), T(inp["w"]), T(inp["b"]))
        if cfg == 4:
            out = torch.empty((128, 64, 62, 62), device=dev)
            g, be = T(inp["gamma"]), T(inp["beta"])
            fn = lambda: nra.conv_norm_epilogue_forward(*a, out=out, norm=nra.NR_NORM_BATCH_TRAIN,
                                                        eps=inp["eps"], gamma=g, beta=be,
                                                        out_scale=inp["scale"])
            orc = lambda: oracle.conv_norm_epilogue(inp["x"], inp["w"], inp["b"], batch=True,
                                                    gamma=inp["gamma"], beta=inp["beta"],
                                                    out_scale=inp["scale"], nthreads=threads)
            keys = ("x", "w", "b", "gamma", "beta")
        else:
            out = torch.empty((128, 14, 30, 30), device=dev)
            m = T(inp["mult"])
            fn = lambda: nra.conv_norm_epilogue_forward(*a, out=out, norm=nra.NR_NORM_INSTANCE,
                                                        eps=inp["eps"], pre_mul=m, clamp=inp["clamp"],
                                                        post_mul=m, reduce_max_c=True)
            orc = lambda: oracle.conv_norm_epilogue(inp["x"], inp["w"], inp["b"], batch=False,
                                                    pre_mul=inp["mult"], clamp=inp["clamp"],
                                                    post_mul=inp["mult"], reduce_max_c=True,
                                                    nthreads=threads)
            keys = ("x", "w", "b", "mult")
        rec = gpu_time(fn)
        fn()
        torch.cuda.synchronize()
        t = time.perf_counter()
        ref = orc()
        dt = time.perf_counter() - t
        rec.update({"shape": list(inp["x"].shape), "input_sha256": {k: sha256_host(inp[k]) for k in keys},
                    "conv_gflop": round(conv_gflop[cfg], 3),
                    "conv_TFLOPs_over_chain_time": round(conv_gflop[cfg] / rec["gpu_ms_median"], 2),
                    "oracle_s": round(dt, 3),
                    "max_abs_err_vs_oracle": float(np.max(np.abs(out.cpu().numpy().astype(np.float64) - ref))),
                    "elements_compared": int(out.numel())})
        record(cfg, rec)
        del a, out


def extras(torch, nra, x, y, steps, warmup):
    import numpy as np

    import synth

    out = {}
    # the one-shot streaming copy of the same bytes (4 KiB per workgroup; also the kernel that
    # calibrates the byte counters)
    tot, per, med = time_calls(lambda: nra.stream_copy(x, y), steps, warmup, torch)
    out["oneshot_copy_GBps"] = round(MIN_BYTES / (per / 1e3) / 1e9, 1)
    log("one-shot stream copy of the same bytes: %.3f ms -> %.1f GB/s" % (per, out["oneshot_copy_GBps"]))
    # the runtime's own device-to-device copy of the same bytes (torch's copy_), for comparison
    tot, per, med = time_calls(lambda: y.copy_(x), steps, warmup, torch)
    out["runtime_copy_GBps"] = round(MIN_BYTES / (per / 1e3) / 1e9, 1)
    log("runtime device copy of the same bytes: %.3f ms -> %.1f GB/s" % (per, out["runtime_copy_GBps"]))
    # the same workload through the two-pass streaming variant
    tot, per, med = time_calls(lambda: nra.inorm_forward(x, y, variant=nra.NR_VARIANT_SPLIT),
                               steps, warmup, torch)
    out["split_variant_GBps"] = round(MIN_BYTES / (per / 1e3) / 1e9, 1)
    log("split (2R+1W) variant: %.3f ms -> %.1f GB/s effective" % (per, out["split_variant_GBps"]))

    dev = x.device
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    # the smaller workloads fit in the 256 MB last-level cache: before each timed call, read a
    # 512 MB buffer so that the call's inputs come from HBM (a read leaves no dirty lines for the
    # timed call to write back, as writing the buffer would)
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    flush = lambda: scrub.sum()
    i2 = synth.host_inputs(2)
    out["input_sha256"] = {"workload2_x": sha256_host(i2["x"])}
    x2 = T(i2["x"])
    y2 = torch.empty_like(x2)
    tot, per, med = time_calls(lambda: nra.inorm_forward(x2, y2), steps, warmup, torch, flush)
    b2 = 2 * 4 * x2.numel()
    # the same bytes copied cold (the one-shot copy, the fastest measured at these sizes): what
    # a pass that reads x once and writes y once can reach with the caches emptied first
    tc, cper, cmed = time_calls(lambda: nra.stream_copy(x2, y2), steps, warmup, torch, flush)
    out["inorm_16x64x256x256"] = {"ms": round(per, 4), "GBps": round(b2 / (per / 1e3) / 1e9, 1),
                                  "cold_copy_ms": round(cper, 4),
                                  "pct_of_cold_copy": round(100 * cper / per, 1)}
    log("inorm x[16,64,256,256]: %.4f ms -> %.1f GB/s (cold copy of the same bytes %.4f ms)"
        % (per, b2 / (per / 1e3) / 1e9, cper))
    del x2, y2

    # standalone training batch norm on the batch-norm model's conv output shape (126 MB)
    xb = torch.randn((128, 64, 62, 62), device=dev, generator=torch.Generator(device=dev).manual_seed(11))
    out["input_sha256"]["bn_train_x"] = sha256_device(xb, torch)
    yb = torch.empty_like(xb)
    tot, per, med = time_calls(lambda: nra.bn_train_forward(xb, yb), steps, warmup, torch, flush)
    bb = 2 * 4 * xb.numel()
    tc, cper, cmed = time_calls(lambda: nra.stream_copy(xb, yb), steps, warmup, torch, flush)
    out["bn_train_128x64x62x62"] = {"ms": round(per, 4), "GBps": round(bb / (per / 1e3) / 1e9, 1),
                                    "cold_copy_ms": round(cper, 4),
                                    "pct_of_cold_copy": round(100 * cper / per, 1)}
    log("bn_train x[128,64,62,62]: %.4f ms -> %.1f GB/s (cold copy of the same bytes %.4f ms)"
        % (per, bb / (per / 1e3) / 1e9, cper))
    del xb, yb

    i4 = synth.host_inputs(4)
    out["input_sha256"].update({"workload4_" + k: sha256_host(i4[k]) for k in ("x", "w", "b", "gamma", "beta")})
    a4 = (T(i4["x"]), T(i4["w"]), T(i4["b"]))
    g4, be4 = T(i4["gamma"]), T(i4["beta"])
    o4 = torch.empty((128, 64, 62, 62), device=dev)
    f4 = lambda: nra.conv_norm_epilogue_forward(*a4, out=o4, norm=nra.NR_NORM_BATCH_TRAIN,
                                                gamma=g4, beta=be4, out_scale=2.0)
    tot, per, med = time_calls(f4, steps, warmup, torch, flush)
    out["conv2d_bn_train_x2_128x8x64x64"] = {"ms": round(per, 4),
                                             "conv_TFLOPs_over_chain_time": round(2 * 128 * 64 * 62 * 62 * 72 / (per / 1e3) / 1e12, 2)}
    log("conv2d+bn_train+x2: %.4f ms" % per)

    i5 = synth.host_inputs(5)
    out["input_sha256"].update({"workload5_" + k: sha256_host(i5[k]) for k in ("x", "w", "b", "mult")})
    a5 = (T(i5["x"]), T(i5["w"]), T(i5["b"]))
    m5 = T(i5["mult"])
    o5 = torch.empty((128, 14, 30, 30), device=dev)
    f5 = lambda: nra.conv_norm_epilogue_forward(*a5, out=o5, norm=nra.NR_NORM_INSTANCE,
                                                pre_mul=m5, clamp=(-1.0, 1.0), post_mul=m5,
                                                reduce_max_c=True)
    tot, per, med = time_calls(f5, steps, warmup, torch, flush)
    out["conv3d_in3d_clamp_maxc_128x3x16x32x32"] = {
        "ms": round(per, 4), "conv_TFLOPs_over_chain_time": round(2 * 128 * 16 * 12600 * 81 / (per / 1e3) / 1e12, 2)}
    log("conv3d+IN3d+clamp+max_c: %.4f ms" % per)

    # both chains captured once in a HIP graph (their workspaces allocated beforehand) and
    # replayed: the same kernels without per-call host launch overhead
    gs = torch.cuda.Stream(device=dev)
    w4 = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)  # holds either chain's plan
    w5 = torch.zeros(256 << 20, dtype=torch.uint8, device=dev)
    g4f = lambda: nra.conv_norm_epilogue_forward(*a4, out=o4, norm=nra.NR_NORM_BATCH_TRAIN,
                                                 gamma=g4, beta=be4, out_scale=2.0,
                                                 workspace=w4, stream=gs)
    g5f = lambda: nra.conv_norm_epilogue_forward(*a5, out=o5, norm=nra.NR_NORM_INSTANCE,
                                                 pre_mul=m5, clamp=(-1.0, 1.0), post_mul=m5,
                                                 reduce_max_c=True, workspace=w5, stream=gs)
    for name, fn in (("conv2d_bn_train_x2_graph_replay", g4f), ("conv3d_in3d_clamp_maxc_graph_replay", g5f)):
        gs.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(gs):
            fn()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=gs):
            fn()
        torch.cuda.synchronize()
        tot, per, med = time_calls(graph.replay, steps, warmup, torch, flush)
        out[name] = {"ms": round(per, 4)}
        log("%s: %.4f ms" % (name, per))
        del graph

    # the same IN3d chain with channels-last input and conv output
    x5cl = a5[0].permute(0, 2, 3, 4, 1).contiguous()
    f5cl = lambda: nra.conv_norm_epilogue_forward(x5cl, a5[1], a5[2], out=o5,
                                                  norm=nra.NR_NORM_INSTANCE, pre_mul=m5,
                                                  clamp=(-1.0, 1.0), post_mul=m5,
                                                  reduce_max_c=True, channels_last=True)
    tot, per, med = time_calls(f5cl, steps, warmup, torch, flush)
    out["conv3d_in3d_clamp_maxc_channels_last_128x16x32x32x3"] = {
        "ms": round(per, 4), "conv_TFLOPs_over_chain_time": round(2 * 128 * 16 * 12600 * 81 / (per / 1e3) / 1e12, 2)}
    log("conv3d+IN3d+clamp+max_c, channels last: %.4f ms" % per)

    # eval-mode batch norm folded into the conv (running statistics of the training chain)
    rm4 = torch.empty(64, device=dev).uniform_(-0.5, 0.5)
    rv4 = torch.empty(64, device=dev).uniform_(0.5, 2.0)
    fe = lambda: nra.conv_bn_eval_forward(*a4, rm4, rv4, out=o4, gamma=g4, beta=be4, out_scale=2.0)
    tot, per, med = time_calls(fe, steps, warmup, torch, flush)
    out["conv2d_bn_eval_x2_128x8x64x64"] = {
        "ms": round(per, 4), "conv_TFLOPs": round(2 * 128 * 64 * 62 * 62 * 72 / (per / 1e3) / 1e12, 2)}
    log("conv2d+bn_eval(folded)+x2: %.4f ms" % per)
    out["timing_note"] = ("workloads 2, 4, 5, the standalone batch norm and the eval conv: mean of "
                          "HIP events around each call, a 512 MB buffer read before each call")
    return out


def conv_producers(steps, warmup):
    """The conv producers alone on the two model shapes (the eval entry point with running mean
    0, running variance 1, eps 0: W and b pass unchanged), each producer selected by the
    library's NORMRED_CONV override: the vector-ALU direct kernel, the fp32 matrix-instruction
    producers and the default bf16-split ones. Prints one JSON line of median ms per call (HIP
    events, a 512 MB read before each)."""
    import numpy as np
    import torch

    import normalization_reductions_amd as nra
    import synth

    dev = torch.device("cuda:0")
    T = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    scrub = torch.ones(128 << 20, dtype=torch.float32, device=dev)
    res = {"metric": "conv producer time, ms (median per call)", "shapes": {}}
    for wl, name, cout, oshape in ((4, "conv2d 8->64 x[128,8,64,64]", 64, (128, 64, 62, 62)),
                                   (5, "conv3d 3->16 x[128,3,16,32,32]", 16, (128, 16, 14, 30, 30))):
        inp = synth.host_inputs(wl)
        a = (T(inp["x"]), T(inp["w"]), T(inp["b"]))
        rm = torch.zeros(cout, device=dev)
        rv = torch.ones(cout, device=dev)
        out = torch.empty(oshape, device=dev)
        f = lambda: nra.conv_bn_eval_forward(*a, rm, rv, out=out, eps=0.0)
        times = {}
        for mode in ("valu", "fp32", "default"):
            if mode == "default":
                os.environ.pop("NORMRED_CONV", None)
            else:
                os.environ["NORMRED_CONV"] = mode
            time_calls(f, steps, warmup, torch, lambda: scrub.sum())
            times[mode] = round(time_calls.last[len(time_calls.last) // 2], 4)
            log("%s, producer %s: %.4f ms" % (name, mode, times[mode]))
        os.environ.pop("NORMRED_CONV", None)
        res["shapes"][name] = times
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--variant", choices=["auto", "resident", "split"], default="auto")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--results-dir", default=None,
                    help="with the CPU baseline: also write one JSON per workload (1-5) into this "
                         "directory (GPU time, oracle time, max |gpu - oracle| over every output)")
    ap.add_argument("--conv-producers", action="store_true",
                    help="time the conv producers alone (vector ALU against matrix cores) on the "
                         "two model shapes, print one JSON line and exit")
    ap.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="host only: write the committed HBM traffic summary from two rocprofv3 "
                         "--pmc counter_collection.csv files of this script, then exit")
    args = ap.parse_args()
    if args.traffic_summary:
        return traffic_summary(*args.traffic_summary)
    if args.conv_producers:
        return conv_producers(args.steps, args.warmup)
    if args.gpus != 1:
        print("bench.py measures one GPU only: instance norm shards over the batch with no "
              "communication, and no multi-GPU path is built (--gpus %d refused)" % args.gpus,
              file=sys.stderr)
        return 2
    if args.steps < 1:
        print("--steps must be >= 1", file=sys.stderr)
        return 2

    import torch

    import normalization_reductions_amd as nra
    import synth

    dev = torch.device("cuda:0")
    variant = {"auto": nra.NR_VARIANT_AUTO, "resident": nra.NR_VARIANT_RESIDENT,
               "split": nra.NR_VARIANT_SPLIT}[args.variant]
    log("%s; drawing x[%d,%d,%d,%d] on the device" % (nra.version(), N, C, H, W))
    x = synth.device_inputs_cfg3(dev)["x"]
    y = torch.empty_like(x)
    ws = torch.zeros(nra.inorm_workspace_size(N, C, S), dtype=torch.uint8, device=dev)

    step = lambda: nra.inorm_forward(x, y, eps=1e-5, workspace=ws, variant=variant)
    total_ms, launch_ms, launch_med = time_calls(step, args.steps, args.warmup, torch)
    launch_min = time_calls.last[0]
    flags = nra.workspace_check(ws)
    if flags:
        log("workspace flags %#x: an exchange wait gave up; results invalid" % flags)
        return 1
    ms = total_ms / args.steps
    value = MIN_BYTES / (ms / 1e3) / 1e9
    achieved = MIN_BYTES / (launch_ms / 1e3) / 1e9
    log("%d steps: %.4f ms/step -> %.1f GB/s (%.1f%% of %.0f GB/s); per launch %.4f ms (median %.4f)"
        % (args.steps, ms, value, 100 * value / HBM_PEAK_GBPS, HBM_PEAK_GBPS, launch_ms, launch_med))
    traffic, tnote = committed_traffic()
    log("traffic: %s (%s)" % (traffic, tnote))
    ceiling = copy_ceiling(torch, nra, x, y, args.steps, min(args.warmup, 3))
    step()  # the copy overwrote y: y again holds the instance norm of x
    torch.cuda.synchronize()
    x_sha = sha256_device(x, torch)
    log("input x sha256 %s" % x_sha)

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic: x ~ N(0,1) drawn on the device by torch's generator seeded with "
                "0x5EED0003",
        "config": {"workload": "InstanceNorm2d x[112,64,512,512] fp32, eps=1e-5, affine=False",
                   "N": N, "C": C, "H": H, "W": W, "min_bytes_per_step": MIN_BYTES,
                   "variant": args.variant, "input_sha256": x_sha},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "copy_ceiling_GBps": round(ceiling, 1),
        "pct_of_copy_ceiling": round(100 * achieved / ceiling, 2),
        "launch_ms": {"mean": round(launch_ms, 5), "median": round(launch_med, 5),
                      "min": round(launch_min, 5)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "norm_pipelined_kernel<256,16> (read-once, 16 parts of 64 KiB "
                               "per slice)" if args.variant != "split"
                               else "split partial/merge/apply"},
        "cpu_baseline": None,
    }
    if not args.no_extra:
        res["extra"] = extras(torch, nra, x, y, args.steps, min(args.warmup, 3))
        step()  # y again holds the instance norm of x for the baseline comparison
        torch.cuda.synchronize()
    if not args.no_cpu_baseline:
        cb, par = cpu_baseline(x, y, args.cpu_seconds, torch)
        res["cpu_baseline"] = cb
        res["parity_sample"] = par
        if args.results_dir:
            head = {"median": round(launch_med, 5), "mean": round(launch_ms, 5),
                    "min": round(launch_min, 5), "max_abs_err": par["max_abs_err"],
                    "elements": par["slices"] * S, "oracle_s": cb["wall_s"]}
            config_results(torch, nra, head, x_sha, args.steps, min(args.warmup, 3), args.results_dir)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
