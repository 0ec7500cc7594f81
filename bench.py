"""Benchmark: fp16 GEMM TFLOP/s on one MI355X and the fraction of the dense
FP16 MFMA peak, on seeded synthetic inputs.

One step is one call of the whole hot path, C = A . B, on the 8192 x 8192 x
8192 workload (A ~ N(0, 1) activations, B ~ N(0, 1/sqrt(K)) weights, seed 4)
with the inputs already resident in GPU memory.  Prints one JSON line.

The roofline entry reports the GEMM kernel's achieved TFLOP/s (2 M N K per
launch over the average launch duration: the timed region, K calls back to
back between two events on the launch stream, divided by K) against MI355X's
dense FP16 MFMA peak; median, minimum and 90th percentile come from a second
pass of K calls, each between its own events; ``traffic`` is the HBM bytes
per launch measured by rocprofv3 counters for this exact kernel source (null
when the source has changed since they were taken).  The CPU baseline times
the plain oracle on a bounded block of the same product.
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

PEAK_FLOPS_PER_CLOCK = 256 * 4096                   # 256 CUs x 4096 flop/clk/CU (dense FP16 MFMA)
PEAK_TFLOPS = PEAK_FLOPS_PER_CLOCK * 2.4e9 / 1e12  # at the 2.4 GHz peak clock
METRIC = "fp16 GEMM TFLOP/s at 1 MI355X and % of dense FP16 MFMA peak"
SPARSE_METRIC = ("2:4-sparse fp16 GEMM TFLOP/s at 1 MI355X (2 flop per product of a kept value: "
                 "M N K per call) and % of dense FP16 MFMA peak")
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "tiled_dense_gemm_fp16_amd", "csrc")
KERNEL_SOURCES = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                        if f.endswith((".hip", ".h", ".cpp")) and not f.startswith("mfma_probe"))


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def traffic_file(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.json")


def measured_counters(workload: str, config_name: str):
    """The committed counter summary of this workload, if it was taken on the
    current kernel source and this configuration; else None."""
    try:
        with open(traffic_file(workload)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if (t.get("kernel_sha256") != kernel_source_hash() or t.get("workload") != workload
            or t.get("kernel_config") != config_name):
        return None
    return t


def measured_traffic(workload: str, config_name: str):
    """HBM bytes per launch from the committed counter summary (see measured_counters)."""
    t = measured_counters(workload, config_name)
    if t is None:
        return None
    return float(t["fetch_bytes_per_launch"]) + float(t["write_bytes_per_launch"])


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform

    return platform.processor() or "unknown"


def cpu_baseline(a, b, w, budget_s: float, sparse=None):
    """Time the oracle on a seeded block of the same product (rows x columns
    of C, full K), sized to take roughly ``budget_s`` seconds."""
    import numpy as np
    import torch

    import oracle
    import workloads

    A = a.view(torch.int16).numpy().view(np.uint16)
    B = b.view(torch.int16).numpy().view(np.uint16)
    rows_all, cols_all = workloads.sample_indices(w)
    cols = cols_all.numpy()
    if sparse is None:
        run = lambda rows: oracle.gemm_sampled(A, B, rows, cols)          # noqa: E731
        per_element = 2.0 * w.K
    else:
        vals, meta = sparse
        run = lambda rows: oracle.gemm_sp_sampled(vals, meta, B, rows, cols)   # noqa: E731
        per_element = 1.0 * w.K                                           # products of kept values
    # calibrate on a small block, then size the timed block
    n_cal = 128
    run(rows_all[:16].numpy())                                            # warm the pages
    t0 = time.perf_counter()
    run(rows_all[:n_cal].numpy())
    t_cal = max(time.perf_counter() - t0, 1e-3)
    n_rows = int(min(len(rows_all), max(n_cal, n_cal * budget_s / t_cal)))
    rows = rows_all[:n_rows].numpy()
    t0 = time.perf_counter()
    run(rows)
    dt = time.perf_counter() - t0
    flops = per_element * len(rows) * len(cols)
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.cpu_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{len(rows)} seeded rows x {len(cols)} seeded columns of C at full K={w.K} "
                  f"({flops / 1e9:.1f} GFLOP, fp64 accumulation) in {dt:.1f} s",
    }


COPY_BYTES = 256 * 1024 * 1024


def copy_calibration() -> int:
    """A plain device-to-device copy of COPY_BYTES, three times: the reference
    kernel whose FETCH_SIZE / WRITE_SIZE readings calibrate the counters."""
    import torch

    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES}), flush=True)
    return 0


def _counter_per_dispatch(csv_path: str, counter: str, kernel_substr: str):
    import csv
    import collections

    per = collections.defaultdict(float)
    with open(csv_path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter and kernel_substr in r["Kernel_Name"]:
                per[int(r["Dispatch_Id"])] += float(r["Counter_Value"])
    return sorted(per.values())


def traffic_from(directory: str, workload: str, config_name: str) -> int:
    """Turn rocprofv3 --pmc CSVs into HBM bytes per GEMM launch, calibrated by
    the copy kernel, and record them with the kernel source hash (the sparse
    product runs the same kernel template, so the same kernel name matches)."""
    import glob
    import statistics

    def one(sub, counter, kernel):
        paths = glob.glob(os.path.join(directory, sub, "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            raise SystemExit(f"no counter CSV under {directory}/{sub}")
        vals = _counter_per_dispatch(paths[0], counter, kernel)
        if not vals:
            raise SystemExit(f"no {counter} rows for {kernel!r} in {paths[0]}")
        return statistics.median(vals)

    def busy_fraction(kernel):
        """Medians over dispatches of the matrix cores' busy share and of the
        GPU's active cycles per XCD (GRBM_GUI_ACTIVE reads the sum over the 8
        XCDs), if the SQ pass is there."""
        import csv
        import collections

        paths = glob.glob(os.path.join(directory, "sq", "**", "*counter_collection.csv"), recursive=True)
        if not paths:
            return None, None
        per = collections.defaultdict(lambda: collections.defaultdict(float))
        with open(paths[0]) as f:
            for r in csv.DictReader(f):
                if kernel in r["Kernel_Name"]:
                    per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
        fr = [d["SQ_VALU_MFMA_BUSY_CYCLES"] / (4.0 * d["SQ_BUSY_CU_CYCLES"]) for d in per.values()
              if d.get("SQ_BUSY_CU_CYCLES")]
        cyc = [d["GRBM_GUI_ACTIVE"] / 8.0 for d in per.values() if d.get("GRBM_GUI_ACTIVE")]
        return (statistics.median(fr) if fr else None), (statistics.median(cyc) if cyc else None)

    copy_fetch = one("copy_fetch", "FETCH_SIZE", "copyBuffer")
    copy_write = one("copy_write", "WRITE_SIZE", "copyBuffer")
    f_fetch = COPY_BYTES / (copy_fetch * 1024.0)
    f_write = COPY_BYTES / (copy_write * 1024.0)
    fetch = one("fetch", "FETCH_SIZE", "gemm_f16_kernel") * 1024.0 * f_fetch
    write = one("write", "WRITE_SIZE", "gemm_f16_kernel") * 1024.0 * f_write
    rec = {"workload": workload, "kernel_config": config_name, "kernel_sha256": kernel_source_hash(),
           "fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
           "fetch_calibration": f_fetch, "write_calibration": f_write,
           "copy_fetch_kib": copy_fetch, "copy_write_kib": copy_write}
    busy, cycles = busy_fraction("gemm_f16_kernel")
    if busy is not None:
        rec["mfma_busy_frac"] = busy
    if cycles is not None:
        rec["gpu_cycles_per_launch"] = cycles
    with open(traffic_file(workload), "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed calls first (about 0.3 s at 8192^3, so the clocks settle)")
    ap.add_argument("--workload", default="gemm_8192")
    ap.add_argument("--config", type=int, default=-1, help="kernel configuration (-1: automatic)")
    ap.add_argument("--sparse", action="store_true",
                    help="time the 2:4-sparse product instead: A pruned to 2:4 and compressed once "
                         "on the GPU before timing")
    ap.add_argument("--layout", default="nn", choices=["nn", "nt", "tn", "tt"],
                    help="dense only: A and/or B given transposed (t: A stored K x M, B stored N x K), "
                         "the same product C = A . B")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the MFMA-only ceiling probe")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the copy kernel used to calibrate FETCH_SIZE / WRITE_SIZE")
    ap.add_argument("--traffic-from", metavar="DIR",
                    help="only convert rocprofv3 counter CSVs under DIR/{fetch,write,copy_fetch,copy_write}")
    args = ap.parse_args()

    if args.copy_calibration:
        return copy_calibration()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the GEMM shards over GPUs without communication; see the design notes)",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tiled_dense_gemm_fp16_amd as g
    import workloads

    if not os.path.exists(g.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()

    w = workloads.WORKLOADS[args.workload]
    if args.sparse and args.layout != "nn":
        print("--layout applies to the dense product only", file=sys.stderr)
        return 2
    ta, tb = args.layout[0] == "t", args.layout[1] == "t"
    workload_name = w.name + ("" if args.layout == "nn" else "_" + args.layout) + ("_sparse_2of4" if args.sparse else "")
    if args.traffic_from:
        if args.sparse:
            p = g.plan_sp(w.M, w.N, w.K, 1 << 20, 1 << 20, 1 << 20, 1 << 20, config=args.config)
            name = g.sp_config_name(p["config"])
        else:
            p = g.plan(w.M, w.N, w.K, 1 << 20, 1 << 20, 1 << 20, config=args.config, trans_a=ta, trans_b=tb)
            name = g.config_name(p["config"])
        return traffic_from(args.traffic_from, workload_name, name)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a, b = workloads.make_inputs(w)
    ad, bd = a.to(dev), b.to(dev)
    cd = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    epi = "relu" if w.relu else "none"
    stream = torch.cuda.current_stream(dev)
    if args.sparse:
        vals, meta = g.sp_compress(ad, stream=stream)
        torch.cuda.synchronize()
        del ad
        plan = g.plan_sp(w.M, w.N, w.K, vals.data_ptr(), meta.data_ptr(), bd.data_ptr(), cd.data_ptr(),
                         config=args.config)

        def call():
            g.gemm_sp(vals, meta, bd, epilogue=epi, out=cd, config=args.config, stream=stream)
    else:
        if ta:
            ad = ad.t().contiguous()
        if tb:
            bd = bd.t().contiguous()
        plan = g.plan(w.M, w.N, w.K, ad.data_ptr(), bd.data_ptr(), cd.data_ptr(), config=args.config,
                      trans_a=ta, trans_b=tb)
        # the arguments are checked once; each call enters the C library
        # (which validates, plans and launches) with the bound tensors
        call = g.prepare(ad, bd, epilogue=epi, out=cd, config=args.config, stream=stream, trans_a=ta, trans_b=tb)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()

    # the timed region: K calls back to back, bracketed by two events on the
    # launch stream (an event between calls would idle the GPU ~10 us each)
    region0 = torch.cuda.Event(enable_timing=True)
    region1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    region0.record(stream)
    for _ in range(args.steps):
        call()
    region1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = region0.elapsed_time(region1)

    # the distribution of single launches: the same K calls again, each
    # bracketed by its own events
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        call()
        ends[i].record(stream)
    torch.cuda.synchronize()
    launch_ms = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)])
    kernel_ms = region_ms / args.steps          # average launch duration over the timed region
    ms_per_step = wall * 1e3 / args.steps
    flops = float(plan["flops"])          # 2 M N K; sparse: M N K (products of kept values)
    value = flops * args.steps / wall / 1e12
    achieved = flops / (kernel_ms * 1e-3) / 1e12

    # a spot check of the timed output against the oracle (a 64 x 64 seeded block)
    import oracle
    rows, cols = workloads.sample_indices(w, 64)
    got = cd[rows.to(dev)][:, cols.to(dev)].cpu().view(torch.int16).numpy().view(np.uint16)
    A_host = a.view(torch.int16).numpy().view(np.uint16)
    B_host = b.view(torch.int16).numpy().view(np.uint16)
    host_sparse = oracle.sp_compress(A_host) if args.sparse else None
    if args.sparse:
        ref = oracle.gemm_sp_sampled(*host_sparse, B_host, rows.numpy(), cols.numpy(), relu=w.relu)
    else:
        ref = oracle.gemm_sampled(A_host, B_host, rows.numpy(), cols.numpy(), relu=w.relu)
    spot = oracle.compare(got, ref)

    config_name = g.sp_config_name(plan["config"]) if args.sparse else g.config_name(plan["config"])
    out = {
        "metric": SPARSE_METRIC if args.sparse else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": workload_name, "M": w.M, "N": w.N, "K": w.K, "layout": args.layout,
                   "epilogue": epi, "inputs": f"{w.dist} seed {w.seed}" + (", A pruned to 2:4" if args.sparse else ""),
                   "sha256_A": workloads.sha256(a), "sha256_B": workloads.sha256(b),
                   "kernel": config_name},
        "pct_of_peak": round(100.0 * value / PEAK_TFLOPS, 2),
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": round(PEAK_TFLOPS, 1),
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_TFLOPS, 4),
            "traffic": measured_traffic(workload_name, config_name),
            "kernel_ms_mean": round(float(kernel_ms), 5),
            "single_launch_ms_mean": round(float(launch_ms.mean()), 5),
            "kernel_ms_median": round(float(np.median(launch_ms)), 5),
            "kernel_ms_min": round(float(launch_ms.min()), 5),
            "kernel_ms_p90": round(float(np.percentile(launch_ms, 90)), 5),
            "algorithmic_flops": flops,
            "algorithmic_bytes": float(plan["min_bytes"]),
        },
        "spot_check": {"block": f"{len(rows)}x{len(cols)} seeded rows x columns of C",
                       "elements": spot["n"], "n_fail": spot.get("n_fail"), "pass": spot["pass"],
                       "max_ulp_err": spot["max_ulp_err"], "max_abs_err": spot.get("max_abs_err")},
    }
    rec = measured_counters(workload_name, config_name)
    if rec is not None and "gpu_cycles_per_launch" in rec:
        # the shader clock this run sustained: the kernel's GPU cycles (from
        # the committed counter record of the same kernel source) over its
        # live mean duration; and the matrix cores' busy share at that clock
        out["roofline"]["counters"] = {
            "source": os.path.relpath(traffic_file(workload_name), ROOT),
            "gpu_cycles_per_launch": rec["gpu_cycles_per_launch"],
            "sclk_ghz": round(rec["gpu_cycles_per_launch"] / (float(kernel_ms) * 1e-3) / 1e9, 3),
            "mfma_busy_frac": round(rec.get("mfma_busy_frac", float("nan")), 4)}
    if not args.no_ceiling:
        # the matrix cores' sustained rate on register operands alone, for the
        # kernel's MFMA instruction, with constant and with changing random bits
        m16 = (not args.sparse) and "_m16" in config_name
        extra = g.PROBE_MFMA16 if m16 else 0
        rnd = g.probe_mfma_tflops(g.PROBE_RANDOM_CHANGING + extra)
        const = g.probe_mfma_tflops(g.PROBE_CONSTANT + extra)
        out["roofline"]["mfma_only_ceiling"] = {
            "instruction": ("v_mfma_f32_16x16x32_f16" if m16 else "v_mfma_f32_32x32x16_f16")
            + (" (dense; a v_smfmac_f32_32x32x32_f16 does as many kept products per cycle)" if args.sparse else ""),
            "random_operands": round(rnd, 1), "constant_operands": round(const, 1), "unit": "TFLOP/s",
            "achieved_over_random_ceiling": round(achieved / rnd, 3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(a, b, w, args.cpu_budget, sparse=host_sparse)
    print(json.dumps(out), flush=True)
    return 0 if spot["pass"] else 1


if __name__ == "__main__":
    sys.exit(main())
