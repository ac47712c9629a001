#!/usr/bin/env python3
"""Benchmark of the persistent GEMM on one MI355X.

Metric: GEMM TFLOPS (2*M*N*K / time) and its fraction of the dense MFMA
peak, swept over K, with the non-persistent, static-persistent and
dynamic-persistent modes side by side (the sweeps of the Triton
persistent-matmul issue, "Describe the issue": M = N = 8192, K from 256
to 8192 in steps of 256 -- the default workload, whose last point is the
8192^3 target -- and M = N = 4096, K from 128 to 4096 in steps of 128).

One "step" is one pass of the whole workload: every K of the sweep in
every scheduling mode and grid multiple, inputs already resident in
device memory.
`value` is the step's total algorithmic flops over its total time, from
K steps launched back to back with nothing between the launches. The
per-(K, mode) table and the roofline's launch durations come from a
second pass of the same K steps with HIP events around every launch
(those events add gaps, so they stay out of the timed region).

After the timed workload the default run also measures, in the same
process and outside the timed region: a small-K pass (100 launches per
(K, mode) point, the mode order rotating from launch to launch, for the
persistent-vs-non-persistent crossover), and a summary of the other
configured workloads (fp16 256^3, the 4096^2 sweep at both macro tiles,
fp8 8192^3, the bf16 tail set), each mode's TFLOP/s and fraction of the
dtype's dense peak.

Prints ONE JSON line on stdout; the per-(K, mode) table goes to
--table (JSON) when given.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "e4m3fn": 5033.2}  # dense MFMA, 256 CU x 2.4 GHz
HBM_GBS = 8000.0
ESIZE = {"f16": 2, "bf16": 2, "e4m3fn": 1}
MODE_NAMES = {0: "nonpersistent", 1: "static", 2: "dynamic", 3: "cancel", 4: "streamk"}

WORKLOADS = {
    # name: (description, dtype, M, N, K list, modes, grid multiples, input kind, workload id)
    "small256": ("fp16 GEMM M=N=K=256, uniform[-1,1], fp16 C; non-persistent, static and dynamic (one tile)",
                 "f16", 256, 256, [256], [0, 1, 2], [0], "uniform", 1),
    "sweep4k": ("fp16 GEMM M=N=4096, K=128..4096 step 128, uniform[-1,1], fp32 accumulate, fp16 C; "
                "non-persistent, static and dynamic persistent per K", "f16", 4096, 4096,
                list(range(128, 4097, 128)), [0, 1, 2], [0], "uniform", 2),
    "sweep8k": ("fp16 GEMM M=N=8192, K=256..8192 step 256, uniform[-1,1], fp16 C; non-persistent, and "
                "static / dynamic persistent at grid multiple 1, 2, 3 x CUs", "f16", 8192, 8192,
                list(range(256, 8193, 256)), [0, 1, 2], [1, 2, 3], "uniform", 3),
    "fp8": ("fp8 e4m3 GEMM M=N=K=8192, uniform[-1,1] quantised with scale 1.0, bf16 C; static vs dynamic",
            "e4m3fn", 8192, 8192, [8192], [0, 1, 2], [0], "uniform", 4),
    "tail": ("bf16 GEMM M=N=K in {4000, 6144, 8200}, normal(0,1), bf16 C; non-persistent, static, dynamic "
             "and stream-K (tail effect)", "bf16", None, None, [4000, 6144, 8200], [0, 1, 2, 4], [0], "normal", 5),
    "fewtiles": ("fp16 GEMM M=N=1024, K in {2048, 8192, 32768}, uniform[-1,1], fp16 C: fewer tiles than "
                 "workgroups; non-persistent, static, dynamic and stream-K", "f16", 1024, 1024,
                 [2048, 8192, 32768], [0, 1, 2, 4], [0], "uniform", 6),
    "square8k": ("fp16 GEMM M=N=K=8192, uniform[-1,1], fp16 C; all modes", "f16", 8192, 8192, [8192],
                 [0, 1, 2], [0], "uniform", 3),
    "uneven": ("fp16 GEMM M=N=K=8192, uniform[-1,1], fp16 C; all five scheduling modes, alone and while "
               "--hold-cus CUs are held by a co-running kernel", "f16", 8192, 8192, [8192],
               [0, 1, 2, 3, 4], [0], "uniform", 3),
}


def add_custom_workload(args) -> None:
    """Register the 'custom' workload from the command line (same shape as the configured ones)."""
    lo, hi = args.K_range
    if min(args.M, args.N, lo, args.K_step) < 1 or hi < lo:
        raise SystemExit("custom workload: --M, --N, --K-range and --K-step must be positive, with LO <= HI")
    dtype = {"fp16": "f16", "bf16": "bf16", "fp8": "e4m3fn"}[args.prec]
    modes = [int(x) for x in args.modes.split(",")] if args.modes else [0, 1, 2]
    gms = [int(x) for x in args.grid_multiples.split(",")]
    desc = (f"{args.prec} GEMM M={args.M} N={args.N}, K={lo}..{hi} step {args.K_step}, {args.input} inputs, "
            f"fp32 accumulate; modes {modes}, grid multiples {gms}")
    WORKLOADS["custom"] = (desc, dtype, args.M, args.N, list(range(lo, hi + 1, args.K_step)), modes, gms,
                           args.input, 20)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="sweep8k", choices=sorted(WORKLOADS) + ["custom"],
                    help="a configured workload, or 'custom' built from --prec/--M/--N/--K-range/--K-step")
    ap.add_argument("--prec", default="fp16", choices=["fp16", "bf16", "fp8"],
                    help="custom workload: input precision (fp8 = OCP e4m3, bf16 output)")
    ap.add_argument("--M", type=int, default=4096, help="custom workload: rows of A and C")
    ap.add_argument("--N", type=int, default=4096, help="custom workload: columns of B and C")
    ap.add_argument("--K-range", type=int, nargs=2, default=[128, 4096], metavar=("LO", "HI"),
                    help="custom workload: K from LO to HI inclusive")
    ap.add_argument("--K-step", type=int, default=128, help="custom workload: K step")
    ap.add_argument("--grid-multiples", default="0",
                    help="custom workload: comma-separated grid multiples of the persistent modes (0 = occupancy)")
    ap.add_argument("--input", default="uniform", choices=["uniform", "normal"], help="custom workload: input values")
    ap.add_argument("--table", default=None, help="write the per-(K, mode) table as JSON here")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample duration")
    ap.add_argument("--modes", default=None, help="comma-separated subset of scheduling modes (0..4)")
    ap.add_argument("--no-small-k-latency", action="store_true",
                    help="skip the 100-launch small-K crossover pass (profiled runs: one launch per point)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured once as a HIP graph and replayed (launch overhead removed)")
    ap.add_argument("--hold-cus", type=int, default=64, help="uneven workload: CUs held by the co-running kernel")
    ap.add_argument("--hold-us", type=int, default=6000, help="uneven workload: how long they are held")
    ap.add_argument("--trace", action="store_true",
                    help="after timing, run every (problem, mode) once more with the tile trace on (untimed) and "
                         "report makespan, busy fraction of the workgroup slots and the drain (tail) time")
    ap.add_argument("--trace-out", default=None, metavar="NPZ",
                    help="with --trace: also save the raw traces (int64 [T, 4]: workgroup, XCD, start, end "
                         "ticks; one array per problem and mode) and the clock rate to this .npz file")
    ap.add_argument("--b-layout", default="kn", choices=["kn", "nk"],
                    help="storage of B: kn = K x N row-major (default, the configured workloads' layout), "
                         "nk = N x K row-major (B transposed, as a linear layer stores its weight)")
    ap.add_argument("--tile", default="auto", choices=["auto", "256", "128"],
                    help="macro tile of the fast kernel (auto: the library's default choice)")
    ap.add_argument("--mainloop", default="auto", choices=["auto", "lockstep", "pingpong", "producer"],
                    help="wave schedule of the 256-row tile (auto: the library's default choice; producer: copy waves and MFMA waves, 256 x 128 tiles)")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the summary of the other configured workloads after the timed one")
    ap.add_argument("--small-k-max", type=int, default=None,
                    help="largest K of the small-K crossover pass (default: 2048 for sweep8k, 1024 for sweep4k, "
                         "512 otherwise)")
    ap.add_argument("--oracle-timing", action="store_true",
                    help="only time the CPU oracle in full on every configured problem it can finish in minutes "
                         "(256^3; 8192^3 fp8; the bf16 tail set; 4096^2 at K = 128, 1024, 4096; 8192^2 at "
                         "K = 256, 2048, 8192) and print one JSON line")
    ap.add_argument("--vendor", action="store_true",
                    help="also time torch's own GEMM (hipBLASLt) on the same operands, interleaved with "
                         "pgemm's static mode in the same process (context, not the metric)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (reference for rocprof HBM counters)")
    return ap.parse_args()


CSRC = os.path.join(ROOT, "persistent_tile_scheduling_macro_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def source_digest() -> str:
    """sha256 over the kernel sources' code (comments and blank space removed);
    HBM counters are only reported for the code they came from."""
    import hashlib
    import re

    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name), encoding="utf-8") as f:
                text = f.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            text = " ".join(text.split())
            h.update(name.encode() + b"\0" + text.encode())
    return h.hexdigest()


def measured_traffic(kernel: str, workload: str):
    """Calibrated HBM bytes per launch of `kernel` from a committed rocprofv3
    summary (profiles/hbm_traffic_*.txt: one key line per kernel of the
    workload), or None if there is none for this workload or the kernel
    source changed since."""
    import glob

    digest = source_digest()
    for path in sorted(glob.glob(os.path.join(PROFILES, "hbm_traffic_*.txt"))):
        kv = {}
        try:
            with open(path) as f:
                for line in f:
                    if ":" in line and not line.startswith(("#", " ")):
                        k, v = line.split(":", 1)
                        kv[k.strip()] = v.strip()
        except OSError:
            continue
        if kv.get("workload") != workload or kv.get("source_sha256") != digest:
            continue
        try:
            return float(kv[f"hbm_bytes_per_launch {kernel}"])
        except (KeyError, ValueError):
            return None
    return None


def copy_calibration(mib: int) -> None:
    """A plain device-to-device copy of known size: FETCH_SIZE and WRITE_SIZE of
    this kernel give the scale from counter units to real bytes."""
    import torch

    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": n * 4, "launches": 3}), flush=True)


def problems(wl):
    desc, dtype, M, N, Ks, modes, gms, kind, wid = WORKLOADS[wl]
    out = []
    for K in Ks:
        m = M if M is not None else K
        n = N if N is not None else K
        for mode in modes:
            for gm in (gms if mode != 0 else [0]):
                out.append((m, n, K, mode, gm))
    return desc, dtype, kind, wid, out


SCHED_NAMES = {0: "kNonPersistent", 1: "kStatic", 2: "kDynamic", 3: "kCancel", 4: "kStreamK"}
DT_NAMES = {"f16": "kF16", "bf16": "kBF16", "e4m3fn": "kF8E4M3"}


def kernel_name(dtype, mode, info):
    """Name of the kernel that computes a launch's whole tiles (the key of the traffic profiles)."""
    if not info["fast_path"]:
        return f"gemm_generic_kernel<{DT_NAMES[dtype]}, {SCHED_NAMES[mode]}>"
    if info.get("body") == 3:  # producer waves (never stream-K)
        return f"gemm_pw_kernel<{DT_NAMES[dtype]}, {SCHED_NAMES[mode]}>"
    if info.get("body") == 2:  # ping-pong; stream-K's whole waves run in its static kernel
        return f"gemm_pp_kernel<{DT_NAMES[dtype]}, {SCHED_NAMES[1 if mode == 4 else mode]}>"
    return f"gemm_fast_kernel<{DT_NAMES[dtype]}, {SCHED_NAMES[mode]}, kTile{info['bm']}>"


def variant_name(p):
    return MODE_NAMES[p[3]] + (f"@g{p[4]}" if p[4] else "")


def setup(pg, torch, si, args, workload, tile=None):
    """Operands, outputs, a handle and a launch function for a configured workload."""
    desc, dtype, kind, wid, probs = problems(workload)
    if args.modes and workload == args.workload:
        keep = {int(x) for x in args.modes.split(",")}
        probs = [p for p in probs if p[3] in keep]
    dev = torch.device("cuda:0")
    dt_code = {"f16": pg.PGEMM_F16, "bf16": pg.PGEMM_BF16, "e4m3fn": pg.PGEMM_F8E4M3_BF16}[dtype]
    out_dtype = torch.bfloat16 if dtype in ("bf16", "e4m3fn") else torch.float16
    # Inputs: drawn once at the largest shape, sliced per K (leading columns of A, rows of B).
    shapes = {}
    for (m, n, K, _, _) in probs:
        shapes.setdefault((m, n), []).append(K)
    operands = {}
    for (m, n), ks in shapes.items():
        kmax = max(ks)
        A, B = si.operands(m, n, kmax, dtype, kind, workload=wid)
        Ad, Bd = A.to(dev), B.to(dev)
        for K in set(ks):
            Bk = Bd[:K, :]
            operands[(m, n, K)] = (Ad[:, :K].contiguous(),
                                   Bk.t().contiguous() if args.b_layout == "nk" else Bk.contiguous())
        del A, B, Ad, Bd
    outs = {(m, n): torch.empty((m, n), dtype=out_dtype, device=dev) for (m, n) in shapes}
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    h = pg.pgemm_create(0)
    pg.pgemm_set_stream(h, stream)
    tile = tile or args.tile
    pg.pgemm_set_tile_config(h, {"auto": pg.PGEMM_TILE_AUTO, "256": pg.PGEMM_TILE_256,
                                 "128": pg.PGEMM_TILE_128}[tile])
    pg.pgemm_set_mainloop(h, {"auto": pg.PGEMM_MAINLOOP_AUTO, "lockstep": pg.PGEMM_MAINLOOP_LOCKSTEP,
                              "pingpong": pg.PGEMM_MAINLOOP_PINGPONG, "producer": pg.PGEMM_MAINLOOP_PRODUCER}[args.mainloop])
    pg.pgemm_set_b_layout(h, pg.PGEMM_B_NK if args.b_layout == "nk" else pg.PGEMM_B_KN)

    def launch(p):
        m, n, K, mode, gm = p
        A, B = operands[(m, n, K)]
        pg.pgemm_run(h, A, B, outs[(m, n)], m, n, K, dt_code, mode, gm)

    return dict(desc=desc, dtype=dtype, kind=kind, wid=wid, probs=probs, dt_code=dt_code, operands=operands,
                outs=outs, stream=stream, h=h, launch=launch)


def rotated_launch_times(torch, stream, probs, launch, rounds):
    """`rounds` rounds; each launches every problem once, with an event pair around each
    launch, in an order rotated by one from round to round (so no variant always runs
    first or last in a burst while the clock settles). Returns {problem: [seconds]}."""
    n = len(probs)
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
          for _ in range(rounds)]
    order = []
    for r in range(rounds):
        idx = [(i + r) % n for i in range(n)]
        order.append(idx)
        for i in idx:
            ev[r][i][0].record(stream)
            launch(probs[i])
            ev[r][i][1].record(stream)
    torch.cuda.synchronize()
    out = {p: [] for p in probs}
    for r in range(rounds):
        for i in order[r]:
            out[probs[i]].append(ev[r][i][0].elapsed_time(ev[r][i][1]) * 1e-3)
    return out


def small_k_crossover(torch, np, env, k_max, rounds=100):
    """Persistent vs non-persistent at small K: every (K, mode, grid multiple) point with
    K <= k_max launched `rounds` times, the order rotating from round to round. Per K:
    median, min and max per variant, the fastest variant by median, and whether the
    non-persistent mode's median beats every persistent variant's."""
    probs = [p for p in env["probs"] if p[2] <= k_max]
    if not probs:
        return None
    for p in probs:  # warm every variant once
        env["launch"](p)
    torch.cuda.synchronize()
    times = rotated_launch_times(torch, env["stream"], probs, env["launch"], rounds)
    out = crossover_summary(times, np)
    out["launches_per_point"] = rounds
    return out


def crossover_summary(times, np):
    """The small-K pass's analysis, from {problem: [seconds per launch]}: per K the median, min
    and max of every variant, the fastest variant, the non-persistent median over the best
    persistent one and whether their [min, max] ranges are separated; the K values where each
    side leads; and the crossover K (the smallest K from which non-persistent is at least as
    fast at every larger measured K; None when persistent leads at the largest)."""
    by_k = {}
    for p, ts in times.items():
        us = sorted(t * 1e6 for t in ts)
        by_k.setdefault(p[2], {})[variant_name(p)] = {
            "median_us": round(float(np.median(us)), 2), "min_us": round(us[0], 2), "max_us": round(us[-1], 2),
            "tflops_median": round(2.0 * p[0] * p[1] * p[2] / (np.median(us) * 1e-6) / 1e12, 1)}
    points, ahead = {}, []
    for K in sorted(by_k):
        v = by_k[K]
        fastest = min(v, key=lambda k: v[k]["median_us"])
        pers = {k: x for k, x in v.items() if not k.startswith("nonpersistent")}
        entry = {"variants": v, "fastest": fastest}
        if "nonpersistent" in v and pers:
            best_p = min(pers, key=lambda k: pers[k]["median_us"])
            np_med, p_med = v["nonpersistent"]["median_us"], pers[best_p]["median_us"]
            entry["best_persistent"] = best_p
            entry["nonpersistent_over_best_persistent"] = round(np_med / p_med, 4)
            # the medians' order is settled only when the two ranges [min, max] do not overlap
            entry["separated"] = bool(v["nonpersistent"]["min_us"] > pers[best_p]["max_us"]
                                      or pers[best_p]["min_us"] > v["nonpersistent"]["max_us"])
            ahead.append((K, np_med <= p_med))
        points[f"K={K}"] = entry
    # crossover: the smallest K from which the non-persistent median is at least as fast as the
    # best persistent one at every larger measured K (None: persistent leads at the largest K)
    cross = None
    for K, np_wins in reversed(ahead):
        if not np_wins:
            break
        cross = K
    return {"order": "rotated by one variant per round", "points": points,
            "persistent_ahead_at_K": [K for K, w in ahead if not w],
            "nonpersistent_ahead_at_K": [K for K, w in ahead if w],
            "crossover_K": cross}


def summarize(env, times, np, peak):
    """Per-(K, mode) table, per-mode totals and the best variant per problem."""
    table, mode_tflops = [], {}
    for p in env["probs"]:
        m, n, K, mode, gm = p
        t = float(np.median(times[p]))
        fl = 2.0 * m * n * K
        byts = ESIZE[env["dtype"]] * (m * K + K * n) + 2 * m * n
        table.append({"M": m, "N": n, "K": K, "mode": MODE_NAMES[mode], "grid_multiple": gm,
                      "us": round(t * 1e6, 2), "tflops": round(fl / t / 1e12, 1),
                      "frac_peak": round(fl / t / 1e12 / peak, 4),
                      "frac_roofline": round(fl / t / 1e12 / min(peak, fl / byts * HBM_GBS / 1e3), 4)})
    for name in sorted({variant_name(p) for p in env["probs"]}):
        ps = [p for p in env["probs"] if variant_name(p) == name]
        fl = sum(2.0 * p[0] * p[1] * p[2] for p in ps)
        tt = sum(float(np.median(times[p])) for p in ps)
        mode_tflops[name] = {"tflops": round(fl / tt / 1e12, 1), "frac_peak": round(fl / tt / 1e12 / peak, 4)}
    return table, mode_tflops


def config_summary(pg, torch, np, si, args):
    """The other configured workloads, measured after the timed one with the same
    library defaults: each (problem, mode) launched in rotated order, a few rounds."""
    out = {}
    plan = [("small256", "auto", 20), ("sweep4k", "auto", 5), ("sweep4k", "128", 5), ("fp8", "auto", 8),
            ("tail", "auto", 6)]
    for wl, tile, rounds in plan:
        env = setup(pg, torch, si, args, wl, tile=tile)
        try:
            for p in env["probs"]:
                env["launch"](p)
            torch.cuda.synchronize()
            times = rotated_launch_times(torch, env["stream"], env["probs"], env["launch"], rounds)
            peak = PEAK_TFLOPS[env["dtype"]]
            table, modes = summarize(env, times, np, peak)
            key = wl if tile == "auto" else f"{wl}_tile{tile}"
            entry = {"workload": env["desc"], "rounds": rounds, "modes": modes}
            if wl in ("fp8", "tail", "small256"):
                entry["problems"] = [{k: r[k] for k in ("M", "N", "K", "mode", "us", "tflops", "frac_peak")}
                                     for r in table]
            if wl == "sweep4k":
                info = pg.pgemm_query_launch(env["h"], 4096, 4096, 4096, env["dt_code"], 1, 0)
                entry["tile"] = f'{info["bm"]}x{info["bn"]}'
                entry["tiles"] = info["tiles"]
                entry["tiles_per_wg_static"] = round(info["tiles"] / info["grid"], 2)
                entry["per_K_tflops"] = {}
                for r in table:
                    entry["per_K_tflops"].setdefault(str(r["K"]), {})[r["mode"]] = r["tflops"]
            out[key] = entry
        finally:
            pg.pgemm_destroy(env["h"])
        del env
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)
    if args.oracle_timing:
        print(json.dumps(oracle_timing()), flush=True)
        return
    import numpy as np
    import torch

    import persistent_tile_scheduling_macro_amd as pg
    import seeded_inputs as si

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.workload == "uneven":
        return run_uneven(args, pg, si, torch, np)
    if args.workload == "custom":
        add_custom_workload(args)
    env = setup(pg, torch, si, args, args.workload)
    desc, dtype, kind, wid, probs = env["desc"], env["dtype"], env["kind"], env["wid"], env["probs"]
    h, stream, launch, dt_code = env["h"], env["stream"], env["launch"], env["dt_code"]
    operands, outs = env["operands"], env["outs"]

    # warmup
    for _ in range(args.warmup):
        for p in probs:
            launch(p)
    torch.cuda.synchronize()

    # timed region: exactly K steps, each the whole workload, launched back to back on the
    # library's stream (torch's current stream) with nothing in between; wall clock between
    # two synchronizations, cross-checked by one event pair around the whole region
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record(stream)
    for s in range(args.steps):
        for p in probs:
            launch(p)
    r1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    region_ms = r0.elapsed_time(r1)

    # per-launch pass: the same K steps again, now with an event pair around every launch
    # (same stream). It gives the per-(K, mode) table and the roofline's launch durations;
    # it is kept out of the timed region because each event pair adds several microseconds
    # between launches (measured: 6.7 against 6.1 ms per sweep4k step).
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in probs]
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    for s in range(args.steps):
        for i, p in enumerate(probs):
            ev[s][i][0].record(stream)
            launch(p)
            ev[s][i][1].record(stream)
    torch.cuda.synchronize()
    per = {p: [] for p in probs}
    for s in range(args.steps):
        for i, p in enumerate(probs):
            per[p].append(ev[s][i][0].elapsed_time(ev[s][i][1]) * 1e-3)

    # small-K crossover: 100 launches per (K, mode) point in rotated order
    k_max = args.small_k_max
    if k_max is None:
        k_max = {"sweep8k": 2048, "sweep4k": 1024}.get(args.workload, 512)
    small_k = None if args.no_small_k_latency else small_k_crossover(torch, np, env, k_max)

    graph_info = None
    if args.graph:
        # One step captured as a graph: the launches are capture-safe (no memsets; the claiming
        # modes' counter resets itself in the kernel). Replays timed with events on the stream.
        gstream = torch.cuda.Stream(device=torch.device("cuda:0"))
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=gstream):
            pg.pgemm_set_stream(h, gstream)
            for p in probs:
                launch(p)
        pg.pgemm_set_stream(h, stream)
        g.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record(stream)
        for _ in range(args.steps):
            g.replay()
        g1.record(stream)
        torch.cuda.synchronize()
        gt = g0.elapsed_time(g1) * 1e-3 / args.steps
        graph_info = {"ms_per_step": round(gt * 1e3, 3),
                      "value": round(sum(2.0 * p[0] * p[1] * p[2] for p in probs) / gt / 1e12, 1)}
        del g

    flops = {p: 2.0 * p[0] * p[1] * p[2] for p in probs}
    step_flops = sum(flops.values())
    value = step_flops * args.steps / wall / 1e12
    peak = PEAK_TFLOPS[dtype]
    table, mode_tflops = summarize(env, per, np, peak)
    for row, p in zip(table, probs):
        info = pg.pgemm_query_launch(h, p[0], p[1], p[2], dt_code, p[3], p[4])
        row.update({"tile": f'{info["bm"]}x{info["bn"]}', "body": info["body"], "tiles": info["tiles"],
                    "grid": info["grid"], "tiles_per_wg": round(info["tiles"] / info["grid"], 2)})

    # roofline of the dominant kernel: the kernel (dtype, scheduling mode, tile body) with the
    # most total time over the per-launch pass
    kname_of = {p: kernel_name(dtype, p[3], pg.pgemm_query_launch(h, p[0], p[1], p[2], dt_code, p[3], p[4]))
                for p in probs}
    tot = {}
    for p in probs:
        tot.setdefault(kname_of[p], [0.0, 0.0, 0])
        tot[kname_of[p]][0] += sum(per[p])
        tot[kname_of[p]][1] += flops[p] * len(per[p])
        tot[kname_of[p]][2] += len(per[p])
    kname = max(tot, key=lambda k: tot[k][0])
    dom_time, dom_flops, dom_n = tot[kname]
    achieved = dom_flops / dom_time / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(kname, args.workload),
                "kernel": kname, "launches": dom_n, "avg_us": round(dom_time / dom_n * 1e6, 2),
                "flops_per_launch_avg": dom_flops / dom_n,
                "timing": "HIP events around every launch on the library's stream, in a second pass of "
                          "the same K steps (the timed region itself has no per-launch events)"}
    if any(p[3] == 4 for p in probs if kname_of[p] == kname):
        roofline["note"] = "stream-K: each timed run is the GEMM kernel plus its tail and fix-up launches"

    best = {}
    for row in table:
        key = (row["M"], row["N"], row["K"])
        if key not in best or row["tflops"] > best[key]["tflops"]:
            best[key] = row
    # the largest problem of the workload (8192^3 for sweep8k), every variant
    top = max(best, key=lambda k: k[0] * k[1] * k[2])
    largest = {"problem": f"{top[0]}x{top[1]}x{top[2]}",
               "variants": {r["mode"] + (f"@g{r['grid_multiple']}" if r["grid_multiple"] else ""):
                            {"tflops": r["tflops"], "frac_peak": r["frac_peak"], "us": r["us"]}
                            for r in table if (r["M"], r["N"], r["K"]) == top}}

    vendor_info = None
    if args.vendor:
        vendor_info = vendor_leg(pg, h, probs, operands, outs, dtype, dt_code, args.b_layout, stream, torch, np)

    trace_info = None
    if args.trace:
        trace_info = tile_trace_summary(pg, h, probs, operands, outs, dt_code, torch, np, args.trace_out)

    pg.pgemm_destroy(h)
    del env, operands, outs
    torch.cuda.empty_cache()

    configs = None
    if not args.no_configs and args.workload == "sweep8k" and not args.modes:
        configs = config_summary(pg, torch, np, si, args)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(dtype, kind, wid, probs, args.cpu_seconds)

    result = {
        "metric": "GEMM TFLOPS and % of dense MFMA peak vs K; persistent vs non-persistent",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype if dtype != "e4m3fn" else "e4m3fn->bf16", "data": "synthetic",
        "config": {"workload": desc, "name": args.workload, "tile": args.tile, "mainloop": args.mainloop,
                   "b_layout": args.b_layout, "launches_per_step": len(probs), "flops_per_step": step_flops},
        "frac_of_peak": round(value / peak, 4),
        "mode_tflops": mode_tflops,
        "largest_problem": largest,
        "best": {f"{k[0]}x{k[1]}x{k[2]}": {"mode": v["mode"], "tflops": v["tflops"], "frac_peak": v["frac_peak"]}
                 for k, v in sorted(best.items())[-3:]},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "timing": {"region_gpu_ms_per_step": round(region_ms / args.steps, 3),
                   "per_launch_pass_ms_per_step": round(sum(sum(v) for v in per.values()) / args.steps * 1e3, 3)},
    }
    if small_k:
        result["small_k_crossover"] = small_k
    if configs:
        result["configs"] = configs
    if graph_info:
        result["graph"] = graph_info
    if trace_info:
        result["tile_trace"] = trace_info
    if vendor_info:
        result["vendor"] = vendor_info
    if args.table:
        with open(args.table, "w") as f:
            json.dump({"result": result, "table": table}, f, indent=1)
    print(json.dumps(result), flush=True)


def vendor_leg(pg, h, probs, operands, outs, dtype, dt_code, b_layout, stream, torch, np, rounds=4, reps=5):
    """torch's own GEMM on the workload's operands, beside pgemm's static mode.

    Per distinct (M, N, K): `rounds` alternations of `reps` back-to-back vendor launches and
    `reps` pgemm static launches, one event pair around each group (same stream), so both
    see the same clock and power state. fp16/bf16 use torch.matmul with B as stored (K x N,
    or the transpose of an N x K B). fp8 uses torch._scaled_mm, which takes B column-major
    (K-contiguous): that is the stored N x K B, or an N x K copy made here for a K x N one.
    Returns total TFLOP/s of each side over the distinct shapes (sum of flops over sum of
    median times) and their ratio."""
    one = torch.ones((), dtype=torch.float32, device=outs[next(iter(outs))].device)
    t_v, t_p, fl = 0.0, 0.0, 0.0
    for (m, n, K) in sorted({p[:3] for p in probs}):
        A, B = operands[(m, n, K)]
        C = outs[(m, n)]
        if dtype == "e4m3fn":
            Bnk = B if b_layout == "nk" else B.t().contiguous()
            def vendor():
                torch._scaled_mm(A, Bnk.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        else:
            Bkn = B.t() if b_layout == "nk" else B
            def vendor():
                torch.matmul(A, Bkn, out=C)
        def ours():
            pg.pgemm_run(h, A, B, C, m, n, K, dt_code, 1, 0)
        tv, tp = [], []
        for fn in (vendor, ours):  # untimed first calls (library heuristics, kernel loads)
            fn()
        for _ in range(rounds):
            for fn, acc in ((vendor, tv), (ours, tp)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for _ in range(reps):
                    fn()
                e1.record(stream)
                torch.cuda.synchronize()
                acc.append(e0.elapsed_time(e1) * 1e-3 / reps)
        t_v += float(np.median(tv))
        t_p += float(np.median(tp))
        fl += 2.0 * m * n * K
    lib = "torch._scaled_mm (B column-major)" if dtype == "e4m3fn" else "torch.matmul"
    return {"library": lib, "tflops": round(fl / t_v / 1e12, 1), "pgemm_static_tflops": round(fl / t_p / 1e12, 1),
            "pgemm_over_vendor": round(t_v / t_p, 3),
            "timing": f"{rounds} alternations of {reps} launches per side and shape, events on one stream"}


def drain_start(st, en, slots, np):
    """Time at which the chip stops being full for good: the tiles in flight
    (+1 at each start, -1 at each end, ends first on equal times) last equal
    `slots` before the next event, which is where the drain begins. Returns
    the first start when the slots were never all busy."""
    n = len(st)
    ev = np.concatenate([np.stack([st, np.ones(n, np.int64)], 1), np.stack([en, -np.ones(n, np.int64)], 1)])
    ev = ev[np.lexsort((ev[:, 1], ev[:, 0]))]
    level = np.cumsum(ev[:, 1])
    full = np.flatnonzero(level >= slots)
    if not len(full):
        return int(st.min())
    nxt = full[-1] + 1
    return int(ev[nxt, 0]) if nxt < len(ev) else int(en.max())


def tile_trace_summary(pg, h, probs, operands, outs, dt_code, torch, np, raw_path=None):
    """One untimed run per (problem, mode) with the tile trace on. Per run:
    makespan (first tile start to last tile end), the busy fraction of the
    workgroup slots (CUs x occupancy) over the makespan, and the drain: the
    time from the last moment every slot held a tile to the end -- the tail
    that the last, partial wave of tiles leaves (KernelWiki "Persistent
    Kernels with Cluster Launch Control", "Choosing between static and CLC
    scheduling"). Stream-K tail pieces are not traced (the fix-up stores
    their tiles), so its busy fraction counts only whole tiles and fix-ups."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    khz = pg.pgemm_clock_khz(0)
    out = {}
    raw = {"clock_khz": np.array(khz)}
    for p in probs:
        m, n, K, mode, gm = p
        info = pg.pgemm_query_launch(h, m, n, K, dt_code, mode, gm)
        T = info["tiles"]
        slots = cus * info["occupancy"]
        tr = torch.zeros(4 * T, dtype=torch.int64, device="cuda:0")
        A, B = operands[(m, n, K)]
        pg.pgemm_set_tile_trace(h, tr)
        try:
            pg.pgemm_run(h, A, B, outs[(m, n)], m, n, K, dt_code, mode, gm)
            torch.cuda.synchronize()
        finally:
            pg.pgemm_set_tile_trace(h, None)
        t = tr.view(T, 4).cpu().numpy()
        raw[f"{m}x{n}x{K}_{MODE_NAMES[mode]}" + (f"_g{gm}" if gm else "")] = t
        wg, xcd, st, en = t[:, 0], t[:, 1], t[:, 2], t[:, 3]
        t0, t1 = int(st.min()), int(en.max())
        us = 1e3 / khz  # microseconds per tick
        busy = float((en - st).sum())
        drain_from = drain_start(st, en, slots, np)
        own = wg >= 0
        key = f"{m}x{n}x{K}"
        out.setdefault(key, {})[MODE_NAMES[mode] + (f"@g{gm}" if gm else "")] = {
            "tiles": T, "grid": info["grid"], "slots": slots,
            "makespan_us": round((t1 - t0) * us, 1),
            "busy_frac": round(busy / (slots * (t1 - t0)), 4) if t1 > t0 else None,
            "drain_us": round((t1 - drain_from) * us, 1),
            "tile_us_median": round(float(np.median(en - st)) * us, 1),
            # workgroups are dealt round-robin over the 8 XCDs from a starting XCD that carries over
            # between launches: the fraction of tiles on XCD (w + r) mod 8 for the launch's rotation r
            "xcd_round_robin": (round(float(np.bincount((xcd[own] - wg[own]) % 8, minlength=8).max() / own.sum()), 4)
                                if own.any() else None),
        }
    if raw_path:
        np.savez(raw_path, **raw)
    return out


def run_uneven(args, pg, si, torch, np):
    """The schedulers when part of the GPU is busy (KernelWiki "Persistent Kernels
    with Cluster Launch Control", "Choosing between static and CLC scheduling": a
    static mapping assumes every CU is available). Each timed GEMM is launched while
    a kernel on a second stream holds `--hold-cus` CUs for `--hold-us`; the same
    GEMMs are also timed alone. Timing is per launch with HIP events on the GEMM's
    stream, which include any wait for CUs."""
    desc, dtype, kind, wid, probs = problems("uneven")
    M = N = K = 8192
    dev = torch.device("cuda:0")
    A, B = si.operands(M, N, K, dtype, kind, workload=wid)
    A, B = A.to(dev), B.to(dev)
    C = torch.empty((M, N), dtype=torch.float16, device=dev)
    stream = torch.cuda.current_stream(dev)
    side = torch.cuda.Stream(device=dev)  # default priority
    h = pg.pgemm_create(0)
    pg.pgemm_set_stream(h, stream)
    modes = list(WORKLOADS["uneven"][5])
    if args.modes:
        modes = [m for m in modes if m in {int(x) for x in args.modes.split(",")}]
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    held_set = [0, min(args.hold_cus, cus - 1)]
    times = {(hc, m): [] for hc in held_set for m in modes}

    def one(hc, m):
        if hc:
            pg.pgemm_hold_cus(side, 0, hc, args.hold_us)
            time.sleep(0.0005)  # let the holding workgroups take their CUs first
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        pg.pgemm_run(h, A, B, C, M, N, K, pg.PGEMM_F16, m, 0)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    # The clock sags over a burst of 8192^3 launches (power limit: a launch late in a
    # step's burst measured up to 30% slower than the first), so a fixed order would
    # favour whichever mode runs first: the order rotates every step, and the step count
    # is rounded up to whole rotations so that every mode takes every position equally
    # often.
    def order(s):
        r = s % len(modes)
        return modes[r:] + modes[:r]

    steps = -(-args.steps // len(modes)) * len(modes)
    for s in range(args.warmup):
        for hc in held_set:
            for m in order(s):
                one(hc, m)
    for s in range(steps):
        for hc in held_set:
            for m in order(s):
                times[(hc, m)].append(one(hc, m))
    flops = 2.0 * M * N * K
    trace_info = None
    if args.trace:
        # one untimed run per (held CUs, mode) with the tile trace on, the CUs held as above
        khz = pg.pgemm_clock_khz(0)
        trace_info, raw = {}, {"clock_khz": np.array(khz)}
        for hc in held_set:
            for m in modes:
                T = pg.pgemm_query_launch(h, M, N, K, pg.PGEMM_F16, m, 0)["tiles"]
                tr = torch.zeros(4 * T, dtype=torch.int64, device=dev)
                pg.pgemm_set_tile_trace(h, tr)
                try:
                    one(hc, m)
                finally:
                    pg.pgemm_set_tile_trace(h, None)
                t = tr.view(T, 4).cpu().numpy()
                raw[f"held{hc}_{MODE_NAMES[m]}"] = t
                wg, st, en = t[:, 0], t[:, 2], t[:, 3]
                t0 = int(st.min())
                us = 1e3 / khz
                own = wg >= 0
                per_wg = np.bincount(wg[own]) if own.any() else np.zeros(1, np.int64)
                per_wg = per_wg[per_wg > 0]
                first_start = {int(w): int(st[wg == w].min()) for w in np.unique(wg[own])}
                trace_info.setdefault(f"held{hc}", {})[MODE_NAMES[m]] = {
                    "makespan_us": round((int(en.max()) - t0) * us, 1),
                    "workgroups_with_tiles": int(len(per_wg)),
                    "tiles_per_wg_min": int(per_wg.min()), "tiles_per_wg_max": int(per_wg.max()),
                    "last_first_start_us": round((max(first_start.values()) - t0) * us, 1) if first_start else None,
                    "drain_us": round((int(en.max()) - drain_start(st, en, cus - hc, np)) * us, 1),
                }
        if args.trace_out:
            np.savez(args.trace_out, **raw)
    table = []
    for (hc, m), ts in times.items():
        t = float(np.median(ts))
        info = pg.pgemm_query_launch(h, M, N, K, pg.PGEMM_F16, m, 0)
        table.append({"held_cus": hc, "mode": MODE_NAMES[m], "us": round(t * 1e6, 1),
                      "tflops": round(flops / t / 1e12, 1), "tiles": info["tiles"], "grid": info["grid"]})
    pg.pgemm_destroy(h)
    tot_t = sum(sum(ts) for ts in times.values())
    n_runs = sum(len(ts) for ts in times.values())
    value = flops * n_runs / tot_t / 1e12
    result = {
        "metric": "GEMM TFLOPS and % of dense MFMA peak vs K; persistent vs non-persistent",
        "value": round(value, 1), "unit": "TFLOP/s", "n_gpus": 1, "steps": steps, "warmup": args.warmup,
        "ms_per_step": round(tot_t / steps * 1e3, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic",
        "config": {"workload": desc, "name": "uneven", "hold_cus": held_set[1], "hold_us": args.hold_us,
                   "cus": cus},
        "by_mode": {f"{r['mode']}@held{r['held_cus']}": r["tflops"] for r in table},
        "roofline": None, "cpu_baseline": None,
    }
    if trace_info:
        result["tile_trace"] = trace_info
    if args.table:
        with open(args.table, "w") as f:
            json.dump({"result": result, "table": table}, f, indent=1)
    print(json.dumps(result), flush=True)


def oracle_timing():
    """The CPU oracle in full (every row, every column) on each configured problem
    it finishes in minutes, on all of the host's cores, plus one thread at 256^3.
    A reported baseline only: seconds and fp64 GFLOP/s per problem."""
    import numpy as np  # noqa: F401

    import oracle
    import seeded_inputs as si

    cores = oracle.default_threads()
    # (label, dtype, input kind, workload id (seeds), M, N, K, K of the drawn operands)
    plan = [("fp16 256^3", "f16", "uniform", 1, 256, 256, 256, 256)]
    plan += [(f"fp16 4096^2 x K={K}", "f16", "uniform", 2, 4096, 4096, K, 4096) for K in (128, 1024, 4096)]
    plan += [(f"fp16 8192^2 x K={K}", "f16", "uniform", 3, 8192, 8192, K, 8192) for K in (256, 2048, 8192)]
    plan += [("fp8 e4m3 8192^3", "e4m3fn", "uniform", 4, 8192, 8192, 8192, 8192)]
    plan += [(f"bf16 {n}^3", "bf16", "normal", 5, n, n, n, n) for n in (4000, 6144, 8200)]
    out = []
    drawn = {}
    for label, dtype, kind, wid, M, N, K, kmax in plan:
        key = (dtype, kind, wid, M, N, kmax)
        if key not in drawn:
            drawn.clear()
            A, B = si.operands(M, N, kmax, dtype, kind, workload=wid)
            drawn[key] = (A, B)
        A, B = drawn[key]
        Ab, Bb = si.bits(A[:, :K].contiguous()), si.bits(B[:K, :].contiguous())
        t0 = time.perf_counter()
        oracle.gemm(Ab, Bb, dtype, nthreads=cores)
        dt = time.perf_counter() - t0
        out.append({"problem": label, "seconds": round(dt, 3), "gflops_fp64": round(2.0 * M * N * K / dt / 1e9, 2)})
        print(f"oracle {label}: {dt:.2f} s", file=sys.stderr, flush=True)
    A1, B1 = si.operands(256, 256, 256, "f16", "uniform", workload=1)
    t0 = time.perf_counter()
    oracle.gemm(si.bits(A1), si.bits(B1), "f16", nthreads=1)
    single = time.perf_counter() - t0
    return {"oracle_timing": out, "threads": cores, "host_cpus": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)), "single_thread_256cubed_s": round(single, 4),
            "kind": "oracle", "what": "fp64 triple loop over the decoded inputs, rows split over threads"}


def cpu_baseline(dtype, kind, wid, probs, seconds):
    """Time the CPU oracle (as it stands) on a bounded sample of the same workload:
    whole problems of the sweep, largest K first, until about `seconds` have
    been spent (row-sampled when even the first problem would take far longer)."""
    import numpy as np

    import oracle
    import seeded_inputs as si

    cores = oracle.default_threads()
    shapes = {}
    for (m, n, K, _, _) in probs:
        shapes.setdefault((m, n), set()).add(K)
    todo = sorted({(m, n, K) for (m, n), ks in shapes.items() for K in ks}, key=lambda x: -x[2])
    drawn = {}

    def bits_of(m, n, K):
        kmax = max(shapes[(m, n)])
        if (m, n) not in drawn:
            drawn.clear()
            drawn[(m, n)] = si.operands(m, n, kmax, dtype, kind, workload=wid)
        A, B = drawn[(m, n)]
        return si.bits(A[:, :K].contiguous()), si.bits(B[:K, :].contiguous())

    # cost of the first (largest) problem from two row counts (each call also decodes all of B)
    m, n, K = todo[0]
    Ab, Bb = bits_of(m, n, K)

    def timed_rows(r):
        t0 = time.perf_counter()
        oracle.gemm(Ab, Bb, dtype, rows=np.arange(r) * (m // r), nthreads=cores)
        return time.perf_counter() - t0

    r1, r2 = 16, 64
    t1, t2 = timed_rows(r1), timed_rows(r2)
    per_row = max((t2 - t1) / (r2 - r1), t2 / r2 / 4, 1e-9)
    fixed = max(t1 - r1 * per_row, 0.0)
    flops = 0.0
    spent = 0.0
    done = []
    if fixed + m * per_row > 2 * seconds:  # one problem is too big: sample its rows
        nrows = int(min(m, max(r2, (seconds - fixed) / per_row)))
        rows = np.sort(np.random.default_rng(0).choice(m, size=nrows, replace=False))
        t0 = time.perf_counter()
        oracle.gemm(Ab, Bb, dtype, rows=rows, nthreads=cores)
        spent = time.perf_counter() - t0
        flops = 2.0 * nrows * n * K
        sample = f"{nrows} of {m} rows of the {m}x{n}x{K} {dtype} problem, all {n} columns"
    else:
        for (m, n, K) in todo:
            if spent >= seconds:
                break
            Ab, Bb = bits_of(m, n, K)
            t0 = time.perf_counter()
            oracle.gemm(Ab, Bb, dtype, nthreads=cores)
            spent += time.perf_counter() - t0
            flops += 2.0 * m * n * K
            done.append(f"{m}x{n}x{K}")
        sample = f"{len(done)} of the {len(todo)} problems of the workload in full ({', '.join(done)})"
    # one thread on the smallest configured problem (256^3, the correctness configuration)
    A1, B1 = si.operands(256, 256, 256, dtype, kind, workload=1)
    a1, b1 = si.bits(A1), si.bits(B1)
    t0 = time.perf_counter()
    oracle.gemm(a1, b1, dtype, nthreads=1)
    single = time.perf_counter() - t0
    return {"value": round(flops / spent / 1e12, 6), "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{sample}, fp64 triple loop, {spent:.1f} s",
            "seconds": round(spent, 2), "gflops_fp64": round(flops / spent / 1e9, 2),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "single_thread_256cubed_s": round(single, 4)}


if __name__ == "__main__":
    main()
