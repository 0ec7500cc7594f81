"""Offline tuning sweep -> frozen configuration table.

The pages recommend searching tile sizes and stage counts with the
autotuner, freezing the result per machine and power limit, and re-running
the search on new hardware ("TileLang：比 Triton 低一层的 tile 语言",
section "工程上的几个注意点"; "5分钟上手TileLang：GPU内核开发指南", section
"避坑与调参").  This script is that search for this library: on a GPU it
times every configuration that accepts each shape of a grid (four layouts,
aligned and misaligned pitches), unsplit and, where the unsplit grid leaves
CUs idle, with K split 2 to 16 ways, and writes ``csrc/gemm_f16_tuned.inc``, a table the
host planner consults before its analytic model: per shape the fastest
configuration and split count, and the fastest configuration unsplit (what
a call without a workspace runs).  Measurements are logged by configuration
name, so a log stays usable when configurations are added or removed.
Rebuild the library afterwards.

    python -m tiled_dense_gemm_fp16_amd.tune [--layouts nn,nt,tn,tt] [--out PATH] [--log LOG]
    python -m tiled_dense_gemm_fp16_amd.tune --from-log LOG [LOG ...] [--out PATH]
"""
from __future__ import annotations

import argparse
import datetime
import json
import math
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
OUT = os.path.join(HERE, "csrc", "gemm_f16_tuned.inc")

# shape grid per alignment class: aligned pitches (every configuration runs)
# at 2x steps in M and N and 4x steps in K; the misaligned classes (rows
# 4-byte aligned: the direct configurations for such rows and the
# register-staged ones; rows 2-byte aligned: register-staged only) on a
# coarser grid
GRIDS = {
    1: ([256, 512, 1024, 2048, 4096, 8192], [256, 1024, 4096, 8192]),
    0: ([512, 2048, 8192], [512, 2048, 8192]),
    2: ([512, 2048, 8192], [512, 2048, 8192]),
}
SPLIT_BELOW_TILES = 512       # K splits are timed only for grids under two workgroups per CU
LAYOUTS = [(False, False), (False, True), (True, False), (True, True)]
SPLITS = [1, 2, 4, 8, 16]
WORKSPACE_MAX = 256 << 20     # the planner's limit for automatic splits
_SIDE = None                  # one capture stream for the whole sweep


def _time(fn, flops, target_s=0.03):
    """TFLOP/s of fn() (one GEMM launch on torch's current stream).

    Launches are captured into a HIP graph of several calls and the graph is
    replayed, so that small shapes are timed on the GPU rather than at the
    rate Python can issue them."""
    import torch

    global _SIDE
    if _SIDE is None:
        _SIDE = torch.cuda.Stream()
    side = _SIDE
    fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(4):
        fn()
    e.record()
    torch.cuda.synchronize()
    one = max(s.elapsed_time(e) / 4, 1e-3)   # ms, an upper bound for small shapes
    per_graph = max(1, min(64, int(2.0 / one)))
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    s.record()
    graph.replay()
    e.record()
    torch.cuda.synchronize()
    g_ms = max(s.elapsed_time(e), 1e-3)
    reps = max(2, min(100, int(target_s * 1e3 / g_ms)))
    s.record()
    for _ in range(reps):
        graph.replay()
    e.record()
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / (reps * per_graph)
    del graph
    return flops / (ms * 1e-3) / 1e12


def sweep(layouts, log, classes=(1, 0, 2)):
    import torch

    import tiled_dense_gemm_fp16_amd as g

    rows = []
    ws = torch.empty(WORKSPACE_MAX // 4, dtype=torch.float32, device="cuda")   # every split's workspace
    narrow = narrow_configs(g)    # never chosen on aligned shapes, so not timed there
    for aligned in classes:
        sizes_mn, sizes_k = GRIDS[aligned]
        for M in sizes_mn:
            for N in sizes_mn:
                for K in sizes_k:
                    # class 2: every pitch off by 4 elements (8-byte rows);
                    # class 0: every pitch odd (2-byte rows)
                    m, n, k = {1: (M, N, K), 2: (M + 4, N + 4, K + 4), 0: (M + 1, N + 1, K + 1)}[aligned]
                    for ta, tb in layouts:
                        a = torch.randn((k, m) if ta else (m, k), device="cuda").half()
                        b = (torch.randn((n, k) if tb else (k, n), device="cuda") / math.sqrt(k)).half()
                        c = torch.empty((m, n), device="cuda", dtype=torch.float16)
                        best = None
                        results = {}
                        for cfg in range(g.num_configs()):
                            name = g.config_name(cfg)
                            if aligned == 1 and name in narrow:
                                continue
                            for sp in SPLITS:
                                try:
                                    p = g.plan(m, n, k, a.data_ptr(), b.data_ptr(), c.data_ptr(), config=cfg,
                                               trans_a=ta, trans_b=tb, splits=sp)
                                except g.GemmError:
                                    break
                                if sp == 1:
                                    unsplit_grid = p["grid"]
                                elif unsplit_grid >= SPLIT_BELOW_TILES:
                                    break
                                # a split must keep two k tiles and use a new count
                                if sp > 1 and (p["splits"] != sp or p["k_tiles"] < 2
                                               or p["workspace_bytes"] > WORKSPACE_MAX):
                                    continue
                                tf = _time(lambda: g.gemm(a, b, out=c, config=cfg, trans_a=ta, trans_b=tb,
                                                          splits=sp, workspace=ws), 2.0 * m * n * k)
                                key = f"{name}:{sp}"
                                results[key] = round(tf, 1)
                                if best is None or tf > results[best]:
                                    best = key
                        # near-ties (within 5 % of the best) are timed again, three
                        # rounds interleaved, so that clock drift between the first
                        # pass's measurements does not decide them; best median wins
                        retimed = None
                        if best is not None:
                            top = sorted(results, key=results.get, reverse=True)
                            top = [key for key in top if results[key] >= 0.95 * results[best]][:3]
                            if len(top) > 1:
                                again = {key: [] for key in top}
                                index = {g.config_name(i): i for i in range(g.num_configs())}
                                for _ in range(3):
                                    for key in top:
                                        name_r, sp_r = key.split(":")
                                        cfg_r, sp_r = index[name_r], int(sp_r)
                                        again[key].append(_time(
                                            lambda: g.gemm(a, b, out=c, config=cfg_r, trans_a=ta, trans_b=tb,
                                                           splits=sp_r, workspace=ws), 2.0 * m * n * k))
                                retimed = {key: round(statistics.median(v), 1) for key, v in again.items()}
                                best = max(retimed, key=retimed.get)
                        rec = {"M": m, "N": n, "K": k, "trans_a": int(ta), "trans_b": int(tb),
                               "aligned": aligned, "best": best, "tflops": results}
                        if retimed:
                            rec["retimed"] = retimed
                        rows.append(rec)
                        print(json.dumps(rec), file=log, flush=True)
                        if log is not sys.stdout:
                            print(f"{m}x{n}x{k} ta={int(ta)} tb={int(tb)}: {best} "
                                  f"{(retimed or results).get(best, 0.0)} TF/s", flush=True)
                        del a, b, c
    return rows


def narrow_configs(g):
    """Names of the configurations built for rows narrower than 16 bytes
    (vec_a or vec_b below 8 on 16-byte-aligned operands: the fallbacks for
    misaligned pitches)."""
    out = set()
    for c in range(g.num_configs()):
        try:
            p = g.plan(4096, 4096, 4096, 1 << 20, 1 << 20, 1 << 20, config=c)
        except g.GemmError:
            continue
        if p["vec_a"] < 8 or p["vec_b"] < 8:
            out.add(g.config_name(c))
    return out


def choose(r, names, narrow=()):
    """(config, splits, TFLOP/s) of the fastest run and (config, TFLOP/s) of
    the fastest unsplit run of one sweep record, over the configurations in
    ``names`` (the library's current list); None if none of them ran.  Keys
    re-timed in interleaved rounds take their re-timed medians.  On aligned
    shapes the ``narrow`` fallbacks are not chosen (a win there is a near-tie
    with their 16-byte twin)."""
    index = {n: i for i, n in enumerate(names)}
    skip = set(narrow) if r["aligned"] == 1 else set()
    vals = {k: v for k, v in {**r["tflops"], **(r.get("retimed") or {})}.items()
            if k.split(":")[0] in index and k.split(":")[0] not in skip}
    if not vals:
        return None
    retimed = {k: v for k, v in (r.get("retimed") or {}).items() if k in vals}
    best = max(retimed or vals, key=(retimed or vals).get)
    unsplit = {k: v for k, v in vals.items() if k.endswith(":1")}
    best1 = best if best.endswith(":1") else max(unsplit, key=unsplit.get)
    name, sp = best.split(":")
    return (index[name], int(sp), vals[best]), (index[best1.split(":")[0]], unsplit[best1])


def write_table(rows, path, note, names, narrow=()):
    lines = [
        "// gemm_f16_tuned.inc -- measured configuration table, written by",
        "// tiled_dense_gemm_fp16_amd/tune.py; do not edit by hand.",
        f"// {note}",
        "// fields: log2 M, log2 N, log2 K (of the swept shape), trans_a, trans_b,",
        "// rows of both operands 16-byte aligned (1), both at least 4-byte aligned (2), otherwise (0),",
        "// best configuration, K splits, its TFLOP/s, best configuration unsplit, its TFLOP/s",
    ]
    for r in rows:
        picked = choose(r, names, narrow)
        if picked is None:
            continue
        (cfg, sp, tf), (cfg1, tf1) = picked
        lm, ln, lk = (round(math.log2(r[x])) for x in ("M", "N", "K"))
        lines.append(f"{{{lm}, {ln}, {lk}, {r['trans_a']}, {r['trans_b']}, {r['aligned']}, {cfg}, {sp}, "
                     f"{tf:.1f}, {cfg1}, {tf1:.1f}}},")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--layouts", default="nn,nt,tn,tt",
                    help="comma-separated layouts to sweep (n: as stored, t: given transposed)")
    ap.add_argument("--classes", default="1,0,2",
                    help="alignment classes to sweep: 1 aligned, 2 every pitch off by 4, 0 every pitch odd")
    ap.add_argument("--out", default=OUT)
    ap.add_argument("--log", default=None, help="also write every measurement (JSON lines) here")
    ap.add_argument("--from-log", nargs="+", default=None, metavar="LOG",
                    help="write the table from earlier sweeps' logs instead of measuring (a shape in a "
                         "later log replaces its record in an earlier one)")
    args = ap.parse_args()
    import tiled_dense_gemm_fp16_amd as g

    names = [g.config_name(c) for c in range(g.num_configs())]
    if args.from_log:
        # a shape measured again in a later log replaces the earlier record
        latest = {}
        for path in args.from_log:
            for line in open(path):
                if line.strip():
                    r = json.loads(line)
                    latest[(r["M"], r["N"], r["K"], r["trans_a"], r["trans_b"], r["aligned"])] = r
        rows = list(latest.values())
        write_table(rows, args.out, f"combined from {len(args.from_log)} sweep log(s)", names, narrow_configs(g))
        print(f"wrote {args.out} ({len(rows)} shapes)", flush=True)
        return 0
    import torch

    if not torch.cuda.is_available():
        print("tune.py needs a GPU", file=sys.stderr)
        return 2
    codes = {"nn": (False, False), "nt": (False, True), "tn": (True, False), "tt": (True, True)}
    layouts = [codes[x] for x in args.layouts.split(",")]
    log = open(args.log, "w") if args.log else sys.stdout
    rows = sweep(layouts, log, tuple(int(x) for x in args.classes.split(",")))
    dev = torch.cuda.get_device_properties(0)
    note = (f"swept {datetime.date.today().isoformat()} on {dev.name} "
            f"({getattr(dev, 'gcnArchName', '?')}, {dev.multi_processor_count} CUs)")
    write_table(rows, args.out, note, names, narrow_configs(g))
    print(f"wrote {args.out} ({len(rows)} shapes)", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
