#!/usr/bin/env python3
"""Benchmark of the int4-dequantizing GEMV on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

One step is the matmul set of one Phi-3-mini decode layer at batch 1, run
back to back through the C ABI: QKV [9216x3072], O-proj [3072x3072], gate_up
[16384x3072] and down [3072x8192] GEMVs, int4 codes + one f16 scale per 32
weights, x f16 ~ N(0,1), f16 out (synthetic seeded inputs of those shapes).
Weights are rotated over enough distinct device copies (>= 1 GiB) that every
step streams them from HBM rather than from the 256 MB Infinity Cache.

Printed (one JSON line): effective GB/s over the step (algorithmic bytes:
codes + scales + x + y, divided by the wall time of K steps), the per-kernel
roofline of the dominant kernel (gate_up) from HIP events around each of its
launches, the oracle's own rate on the host, and the other variants of the
matmul (single 3072^2 GEMV, fused gate/up SiLU FFN + down, f32 LM head with
argmax, skinny GEMM at M = 16/64/256) as sub-objects.
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

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, published
PEAK_F16_TFLOPS = 2500.0       # MI355X dense f16 MFMA, published
ROTATE_BYTES = 1 << 30         # distinct weight bytes cycled through (4x the MALL)
PROFILE_DIR = os.path.join(ROOT, "profiles")


def weight_bytes(n: int, k: int) -> int:
    return n * k // 2 + n * (k // 32) * 2


def gemv_bytes(n: int, k: int, out_bytes: int = 2) -> int:
    return weight_bytes(n, k) + 2 * k + out_bytes * n


def weight3_bytes(n: int, k: int) -> int:
    """int3: 3-bit codes plus one f16 scale per 32."""
    return n * k * 3 // 8 + n * (k // 32) * 2


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--only", choices=["all", "layer", "variants", "gemm"], default="all",
                    help="layer: the headline step only; gemm: the prefill GEMM at --gemm-m "
                         "only (both for profiling)")
    ap.add_argument("--gemm-m", type=int, default=256,
                    help="with --only gemm: activation rows of the 16384x3072 GEMM")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate host time budget of the oracle baseline")
    ap.add_argument("--summarize", metavar="RESULTS_DB",
                    help="print per-kernel duration statistics of a rocprofv3 "
                         "--kernel-trace database (grouped by kernel and grid) and exit")
    ap.add_argument("--roles", metavar="NAMES",
                    help="with --summarize or --counters: comma-separated names of the GEMVs one step "
                         "launches, in order (a --only layer run: qkv,o_proj,gate_up,down)")
    ap.add_argument("--counters", nargs="+", metavar="PMC_DB",
                    help="print the median per dispatch of every counter in rocprofv3 --pmc "
                         "databases, per q4 kernel and grid, and exit")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="print the HBM traffic summary of the gate_up GEMV from two "
                         "rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of --only layer, "
                         "calibrated on the 256 MiB copy that run makes, and exit")
    return ap.parse_args()


CALIBRATION_BYTES = 256 << 20   # device-to-device copy made in --only layer runs


LAYER_ROLES = ("qkv", "o_proj", "gate_up", "down")   # launch order of one layer step


def label_roles(seq, roles):
    """Roles of the q4 GEMV dispatches of a profiled run, in dispatch order:
    a dispatch with the same (kernel, grid) as the previous GEMV dispatch keeps
    its role (a loop over one GEMV), any other takes the next role in step
    order.  This matches the launch order of bench.py's layer part: the timed
    steps, then one timing loop per GEMV in step order.  Non-GEMV dispatches
    get None."""
    out, ri, prev = [], -1, None
    for name, grid in seq:
        if not name.startswith("void q4::gemv_"):
            out.append(None)
            continue
        if (name, grid) != prev:
            ri = (ri + 1) % len(roles)
            prev = (name, grid)
        out.append(roles[ri])
    return out


def pmc_medians(db_path: str, counter: str):
    """{role or (kernel name, grid): median value per dispatch} of one counter;
    layer GEMV dispatches are keyed by their role."""
    import sqlite3
    import statistics
    db = sqlite3.connect(db_path)
    rows = db.execute("select dispatch_id, kernel_name, grid_size, sum(value) from "
                      "counters_collection where counter_name = ? group by dispatch_id "
                      "order by dispatch_id", (counter,)).fetchall()
    labels = label_roles([(name, grid) for _, name, grid, _ in rows], LAYER_ROLES)
    groups = {}
    for (_, name, grid, v), role in zip(rows, labels):
        groups.setdefault(role or (name, grid), []).append(v)
    return {key: statistics.median(v) for key, v in groups.items()}


def pmc_max_dispatch(db_path: str, counter: str):
    """(kernel name, value) of the single dispatch with the largest value."""
    import sqlite3
    db = sqlite3.connect(db_path)
    rows = db.execute("select kernel_name, sum(value) as v from counters_collection where "
                      "counter_name = ? group by dispatch_id order by v desc limit 1",
                      (counter,)).fetchall()
    return rows[0]


def counters_summary(db_paths, roles=None) -> int:
    """Median per dispatch of every counter of the library's kernels in one or
    more rocprofv3 --pmc databases (one pass each), grouped by kernel and grid;
    with `roles` the layer GEMV dispatches are grouped by role (label_roles)."""
    import sqlite3
    import statistics
    groups = {}
    for path in db_paths:
        db = sqlite3.connect(path)
        rows = db.execute("select dispatch_id, kernel_name, grid_size, counter_name, sum(value) from "
                          "counters_collection group by dispatch_id, counter_name "
                          "order by dispatch_id").fetchall()
        role_of = {}
        if roles:
            order = []
            for d, name, grid, _, _ in rows:
                if not order or order[-1][0] != d:
                    order.append((d, name, grid))
            labels = label_roles([(name, grid) for _, name, grid in order], roles)
            role_of = {d: lab for (d, _, _), lab in zip(order, labels)}
        for d, name, grid, counter, v in rows:
            if "q4::" in name:
                key = (f"{role_of[d]}: {name}", grid) if role_of.get(d) else (name, grid)
                groups.setdefault(key, {}).setdefault(counter, []).append(v)
        print(f"# rocprofv3 --pmc: {path}")
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            if any(c == counter for *_, c, _ in rows):
                # the run's calibration copy moves by far the most bytes
                cal = pmc_max_dispatch(path, counter)
                print(f"# calibration: {cal[0][:40]} copying {CALIBRATION_BYTES} B reads {counter} "
                      f"{cal[1]:.1f} KiB -> {counter.lower()}_scale "
                      f"{CALIBRATION_BYTES / (cal[1] * 1024.0):.4f}")
    for (name, grid), cs in sorted(groups.items()):
        print(f"# kernel {name[:110]}  grid {grid}")
        for counter, v in sorted(cs.items()):
            print(f"{counter}: {statistics.median(v):.6g}   (dispatches: {len(v)})")
    return 0


def traffic_summary(fetch_db: str, write_db: str) -> int:
    fetch = pmc_medians(fetch_db, "FETCH_SIZE")
    write = pmc_medians(write_db, "WRITE_SIZE")
    # the calibration copy is the single dispatch that moves by far the most bytes
    cal_f = pmc_max_dispatch(fetch_db, "FETCH_SIZE")
    cal_w = pmc_max_dispatch(write_db, "WRITE_SIZE")
    kf = CALIBRATION_BYTES / (cal_f[1] * 1024.0)
    kw = CALIBRATION_BYTES / (cal_w[1] * 1024.0)
    import seeded_inputs as si
    print("# HBM traffic per launch of the layer-set GEMVs, from rocprofv3 PMC; the gate_up")
    print("# GEMV (16384 x 3072) is the kernel bench.py reports in its roofline object")
    print(f"# FETCH_SIZE run: {fetch_db}")
    print(f"# WRITE_SIZE run: {write_db}")
    print(f"# calibration: {cal_f[0][:40]} copying {CALIBRATION_BYTES} B reads "
          f"FETCH_SIZE {cal_f[1]:.1f} KiB and WRITE_SIZE {cal_w[1]:.1f} KiB")
    print(f"fetch_scale: {kf:.4f}")
    print(f"write_scale: {kw:.4f}")
    for role in LAYER_ROLES:
        n, k = si.LAYER_SHAPES[role]
        f_bytes = fetch[role] * 1024.0 * kf
        w_bytes = write.get(role, 0.0) * 1024.0 * kw
        tag = "" if role == "gate_up" else f"{role}."
        print(f"# {role} {n} x {k}: FETCH_SIZE median {fetch[role]:.1f} KiB, "
              f"WRITE_SIZE median {write.get(role, 0.0):.1f} KiB")
        print(f"{tag}hbm_read_bytes_per_launch: {f_bytes:.0f}")
        print(f"{tag}hbm_write_bytes_per_launch: {w_bytes:.0f}")
        print(f"{tag}hbm_bytes_per_launch: {f_bytes + w_bytes:.0f}")
        print(f"{tag}algorithmic_bytes_per_launch: {gemv_bytes(n, k)}")
    print(f"kernel_sources_sha256_16: {kernels_hash()}")
    return 0


def summarize(db_path: str, roles=None) -> int:
    """Kernel-trace statistics from a rocprofv3 results database: one row per
    (kernel, grid size), durations in microseconds.  With `roles` (the names
    of the GEMVs one step launches, in launch order) the q4 GEMV dispatches
    are labelled by label_roles, so two layers that run the same kernel with
    the same grid get separate rows."""
    import sqlite3
    import statistics
    db = sqlite3.connect(db_path)
    rows = db.execute("select name, grid_x, workgroup_x, vgpr_count, accum_vgpr_count, "
                      "sgpr_count, lds_size, duration from kernels order by start").fetchall()
    labels = label_roles([(r[0], r[1]) for r in rows], roles) if roles else [None] * len(rows)
    groups = {}
    for (name, gx, wx, vg, ag, sg, lds, dur), role in zip(rows, labels):
        groups.setdefault((role or "-", name, gx, wx, vg, ag, sg, lds), []).append(dur / 1000.0)
    print(f"# rocprofv3 kernel trace: {db_path}")
    print("# calls  avg_us  median_us  min_us  p10_us  p90_us  grid  block  vgpr  agpr  sgpr  lds  role  kernel")
    for key, d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        role, name, gx, wx, vg, ag, sg, lds = key
        d.sort()
        p10 = d[int(0.1 * (len(d) - 1))]
        p90 = d[min(len(d) - 1, int(0.9 * len(d)))]
        print(f"{len(d):6d} {statistics.fmean(d):8.3f} {statistics.median(d):8.3f} {d[0]:8.3f} "
              f"{p10:8.3f} {p90:8.3f} {gx:8d} {wx:5d} {vg:4d} {ag:4d} {sg:4d} {lds:6d}  {role:8s} {name[:100]}")
    return 0


def kernels_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "int4_quantized_decode_q4_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel_tag: str):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    path = os.path.join(PROFILE_DIR, f"traffic_{kernel_tag}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                key, _, v = line.partition(":")
                vals[key.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernels_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Rotation:
    """C distinct device copies of a packed weight (same bytes, different
    addresses): the first is packed from the seeded inputs, the rest are
    device-side clones."""

    def __init__(self, q4, pw, copies: int):
        self.items = [pw]
        for _ in range(copies - 1):
            self.items.append(pw.clone())

    def __getitem__(self, i):
        return self.items[i % len(self.items)]


def dev_f16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.float16)).cuda()


def dev_u16(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def dev_u32(a):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).cuda()


def copies_for(nbytes: int) -> int:
    return max(2, -(-ROTATE_BYTES // nbytes))


def capture(torch, fn, first: int, count: int):
    """A HIP graph of fn(first), ..., fn(first + count - 1), captured on a side
    stream (the library launches on torch's current stream, which is the
    capture stream inside the block)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn(first)                       # one eager call before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(first, first + count):
            fn(i)
    return g


HOLD_CYCLES = 4_000_000   # device-side delay in front of a timed region


def timed(torch, fn, steps: int, warmup: int):
    """Device time per call (ms) of exactly `steps` calls fn(warmup), ...,
    replayed from one HIP graph, after `warmup` untimed calls (their own
    graph), with synchronisation on both sides.  The first replay of a newly
    instantiated graph costs about 18 us more on this platform (one-time
    set-up), so the timed graph is replayed once, untimed, beforehand.  The
    warmup graph is then queued behind a short bounded spin of the device
    (torch.cuda._sleep) and the timed graph straight behind the warmup one,
    so when the timed region opens the graph is already submitted and the
    device is busy and warm: the region holds the steps' device work and the
    gaps between them, not the host's submission or a cold start, and the
    figure does not depend on `steps`."""
    gw = capture(torch, fn, 0, max(1, warmup))
    gt = capture(torch, fn, warmup, steps)
    gw.replay()
    gt.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(HOLD_CYCLES)
    gw.replay()
    start.record()
    gt.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps


PER_LAUNCH_MIN = 200   # launches behind every per-kernel figure


def per_launch_us(torch, fn, launches: int = 200, warmup: int = 20):
    """Average device time (us) of one launch of fn: at least PER_LAUNCH_MIN
    back-to-back launches (rotating weight copies, so each copy comes back
    after >= 1 GiB of other bytes) replayed from a HIP graph, bracketed by HIP
    events on the launching stream."""
    return 1000.0 * timed(torch, fn, max(launches, PER_LAUNCH_MIN), warmup)


def main():
    args = parse()
    if args.summarize:
        return summarize(args.summarize, args.roles.split(",") if args.roles else None)
    if args.traffic:
        return traffic_summary(*args.traffic)
    if args.counters:
        return counters_summary(args.counters, args.roles.split(",") if args.roles else None)
    if args.gpus != 1:
        print("bench.py measures one GPU: the int4 GEMV path has no multi-GPU part in this "
              "library (run with --gpus 1)", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import int4_quantized_decode_q4_amd as q4
    import seeded_inputs as si

    torch.cuda.set_device(0)
    K, W = args.steps, args.warmup
    result = {}
    if args.only == "gemm":
        return gemm_only(torch, q4, si, np, K, W, args.gemm_m)

    # ---------------------------------------------------------------- layer
    inp = si.workload(si.LAYER_SET, seed=0)
    x3, x8 = dev_f16(inp["x3072"]), dev_f16(inp["x8192"])
    set_bytes = sum(weight_bytes(n, k) for n, k in si.LAYER_SHAPES.values())
    C = copies_for(set_bytes)
    rot = {}
    outs = {}
    for key, (n, k) in si.LAYER_SHAPES.items():
        w, s = inp[key]
        rot[key] = Rotation(q4, q4.pack(dev_u32(w), dev_u16(s)), C)
        outs[key] = torch.empty(n, dtype=torch.float16, device="cuda")
    xin = {"qkv": x3, "o_proj": x3, "gate_up": x3, "down": x8}

    def launch(key):
        return lambda i: q4.gemv(rot[key][i], xin[key], outs[key])

    launches = {key: launch(key) for key in si.LAYER_SHAPES}

    def step(i):
        for fn in launches.values():
            fn(i)

    step_bytes = sum(gemv_bytes(n, k) for n, k in si.LAYER_SHAPES.values())
    if args.only == "layer":
        # a device copy of known size, for calibrating HBM byte counters
        src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)
        torch.cuda.synchronize()
        del src
    ms = timed(torch, step, K, W)
    # each GEMV alone, over its own rotation of >= 1 GiB of distinct copies
    # (the layer set's copies plus more clones), so no single-matrix figure is
    # served from the Infinity Cache
    kus = {}
    for key, (n, k) in si.LAYER_SHAPES.items():
        own = rot[key].items + [rot[key][0].clone()
                                for _ in range(copies_for(weight_bytes(n, k)) - C)]
        kus[key] = per_launch_us(torch, lambda i, own=own, key=key:
                                 q4.gemv(own[i % len(own)], xin[key], outs[key]), K, W)
        del own
    gbs = step_bytes / (ms * 1e-3) / 1e9
    dom = "gate_up"
    dn, dk = si.LAYER_SHAPES[dom]
    dom_bytes = gemv_bytes(dn, dk)
    achieved = dom_bytes / (kus[dom] * 1e-6) / 1e9
    traffic = committed_traffic("phi3_layer_set")
    result.update({
        "metric": "int4 GEMV effective HBM GB/s (% of peak) + us per Phi-3-mini decode layer",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "phi3_mini_layer_set",
            "matrices": {k: list(v) for k, v in si.LAYER_SHAPES.items()},
            "batch": 1, "group": 32, "weights": "int4 codes + f16 scale per 32 (q4f16_1)",
            "accumulate": "f32", "rotation_copies": C,
            "bytes_per_step": step_bytes,
        },
        "us_per_layer_wall": round(ms * 1000, 3),
        "us_per_layer_kernel_sum": round(sum(kus.values()), 3),
        "pct_of_peak_hbm": round(100 * gbs / PEAK_HBM_GBS, 2),
        "per_kernel_us": {k: round(v, 3) for k, v in kus.items()},
        "per_kernel_gbs": {k: round(gemv_bytes(*si.LAYER_SHAPES[k]) / (kus[k] * 1e-6) / 1e9, 1)
                           for k in kus},
        "roofline": {
            "kernel": "q4 GEMV gate_up 16384x3072 (gemv_block_kernel<32,3,f16>)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
            "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": dom_bytes,
        },
    })

    # the same four GEMVs as one q4_chain launch, gate_up after O-proj and
    # down after gate_up (the order a decode layer imposes on them)
    chain_sets = [[q4.Stage(rot["qkv"][i], x=x3, out=outs["qkv"]),
                   q4.Stage(rot["o_proj"][i], x=x3, out=outs["o_proj"]),
                   q4.Stage(rot["gate_up"][i], x=x3, after=1, out=outs["gate_up"]),
                   q4.Stage(rot["down"][i], x=x8, after=2, out=outs["down"])] for i in range(C)]
    ms_chain = timed(torch, lambda i: q4.chain(chain_sets[i % C]), K, W)
    result["layer_set_one_chain_launch"] = {
        "us": round(ms_chain * 1000, 3), "gbs": round(step_bytes / (ms_chain * 1e-3) / 1e9, 1),
        "frac": round(step_bytes / (ms_chain * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
    del chain_sets

    probe_sizes = {"gemv_3072x3072": gemv_bytes(3072, 3072)}
    probe_sizes.update({key: gemv_bytes(n, k) for key, (n, k) in si.LAYER_SHAPES.items()})
    probe_sizes.update({"layer_set": step_bytes,
                        "lm_head_32064x3072": gemv_bytes(32064, 3072, out_bytes=4) + 4})
    probe = read_probe_leg(torch, q4, probe_sizes, K, W)
    result["read_probe"] = probe
    result["per_kernel_frac_of_read_probe"] = {
        key: round(probe[key]["us"] / kus[key], 4) for key in kus}
    result["layer_set_frac_of_read_probe"] = round(probe["layer_set"]["us"] / (ms * 1000), 4)

    if args.only in ("all", "variants"):
        result["variants"] = variants(torch, q4, si, np, K, W)
        v = result["variants"]
        v["gemv_3072x3072"]["frac_of_read_probe"] = round(
            probe["gemv_3072x3072"]["us"] / v["gemv_3072x3072"]["us"], 4)
        v["lm_head_32064x3072_f32_argmax"]["frac_of_read_probe"] = round(
            probe["lm_head_32064x3072"]["us"] / v["lm_head_32064x3072_f32_argmax"]["us"], 4)

    if not args.no_cpu_baseline and args.only == "all":
        result["cpu_baseline"] = cpu_baseline(si, inp, args.cpu_seconds)
    result["library"] = library_stamp(q4)

    print(json.dumps(result), flush=True)
    return 0


def library_stamp(q4) -> dict:
    """The source digest stamped into the loaded libq4.so against the digest
    of the sources in this tree (the build script's sources_digest)."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "q4_build", os.path.join(ROOT, "int4_quantized_decode_q4_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    built, tree = q4.source_hash(), b.sources_digest()
    return {"source_hash": built, "tree_hash": tree, "matches_sources": built == tree}


def read_probe_leg(torch, q4, sizes: dict, K: int, W: int) -> dict:
    """The plain streaming read (q4_read_probe) of each size in one launch,
    over rotating offsets of a buffer >= 1 GiB larger than the size (so the
    bytes come from HBM), timed as the kernels are: the ceiling each
    HBM-bound matmul is read against."""
    big = max(sizes.values())
    pool = torch.empty(ROTATE_BYTES + big + 4096, dtype=torch.uint8, device="cuda")
    sink = torch.empty(2048, dtype=torch.int32, device="cuda")
    out = {}
    for name, nb in sizes.items():
        nb = (nb + 15) // 16 * 16          # the probe reads whole 16-byte words
        stride = (nb + 4095) // 4096 * 4096
        slots = max(2, ROTATE_BYTES // stride)
        views = [pool[i * stride:i * stride + nb] for i in range(slots)]
        us = per_launch_us(torch, lambda i, views=views: q4.read_probe(views[i % len(views)], sink),
                           K, W)
        out[name] = {"bytes": nb, "us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                     "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4)}
    del pool
    return out


def decode_layer(torch, q4, si, np, K, W, ctx):
    """One whole Phi-3-mini decoder layer per step, in 5 launches (+1 to
    combine the attention chunks): add + RMSNorm + QKV + RoPE + K/V append,
    paged attention over ctx positions, O-proj, add + RMSNorm + gate/up +
    SiLU, down-proj.  Layer copies (weights and cache) rotated over >= 1 GiB."""
    inp = si.workload(si.LAYER_SET, seed=0)
    rng = np.random.default_rng(13)
    (qw, qs), (ow, os_), (dw, ds) = inp["qkv"], inp["o_proj"], inp["down"]
    fi = si.workload(si.FFN, seed=0)
    (gw, gs), (uw, us_) = fi["gate"], fi["up"]
    pages = ctx // 16 + 1
    layer_bytes = (weight_bytes(9216, 3072) + weight_bytes(3072, 3072) +
                   2 * weight_bytes(8192, 3072) + weight_bytes(3072, 8192))
    kv_read = ctx * 2 * 3072 * 2
    copies = copies_for(layer_bytes + pages * 2 * 16 * 3072 * 2)
    base = {"qkv": q4.pack_rope(dev_u32(qw), dev_u16(qs), 96),
            "o": q4.pack(dev_u32(ow), dev_u16(os_)),
            "gu": q4.pack_gate_up(dev_u32(gw), dev_u16(gs), dev_u32(uw), dev_u16(us_)),
            "down": q4.pack(dev_u32(dw), dev_u16(ds))}
    layers = []
    for c in range(copies):
        lw = {key: (pw if c == 0 else pw.clone()) for key, pw in base.items()}
        lw["cache"] = torch.empty((pages, 2, 32, 16, 96), dtype=torch.float16,
                                  device="cuda").normal_()
        layers.append(lw)
    pt = torch.arange(pages, dtype=torch.int32, device="cuda")
    g1 = dev_f16(si.f16_bits(rng.uniform(0.5, 1.5, 3072)))
    g2 = dev_f16(si.f16_bits(rng.uniform(0.5, 1.5, 3072)))
    f16 = dict(dtype=torch.float16, device="cuda")
    x = dev_f16(inp["x3072"])                     # the previous layer's down-proj output
    res = [dev_f16(si.f16_bits(rng.normal(0.0, 2.0, 3072))), torch.empty(3072, **f16)]
    res2 = torch.empty(3072, **f16)
    qkv, att = torch.empty(9216, **f16), torch.empty((32, 96), **f16)
    o, h, y = torch.empty(3072, **f16), torch.empty(8192, **f16), torch.empty(3072, **f16)
    ws = q4.workspace(x.device, int(q4.lib.q4_workspace_bytes(q4.OP_ATTENTION, ctx, 32, 96)))

    def step(i):
        L = layers[i % copies]
        pos = ctx - 1
        q4.qkv_rope_append(L["qkv"], x, 32, pos, 10000.0, L["cache"], pt, out=qkv,
                           norm=(res[0], g1, 1e-5, res[1]))
        q4.attention_decode(qkv[:3072], L["cache"], pt, ctx, 32, 96 ** -0.5, out=att, ws=ws)
        q4.gemv(L["o"], att.view(-1), out=o)
        q4.add_rmsnorm_ffn_gate_up_silu(L["gu"], o, res[1], g2, 1e-5, residual_out=res2, out=h)
        q4.gemv(L["down"], h, out=y)

    ms = timed(torch, step, K, W)
    nb = layer_bytes + kv_read

    # the same layer with O-proj -> add + RMSNorm -> gate/up + SiLU -> down
    # as one q4_chain launch (each stage reads the previous one's output)
    for L in layers:
        L["chain"] = [q4.Stage(L["o"], x=att.view(-1), out=o),
                      q4.Stage(L["gu"], src=0, residual=res[1], gamma=g2, eps=1e-5,
                               residual_out=res2, out=h),
                      q4.Stage(L["down"], src=1, out=y)]

    def step_chain(i):
        L = layers[i % copies]
        pos = ctx - 1
        q4.qkv_rope_append(L["qkv"], x, 32, pos, 10000.0, L["cache"], pt, out=qkv,
                           norm=(res[0], g1, 1e-5, res[1]))
        q4.attention_decode(qkv[:3072], L["cache"], pt, ctx, 32, 96 ** -0.5, out=att, ws=ws)
        q4.chain(L["chain"])

    ms_c = timed(torch, step_chain, K, W)
    return {"us": round(ms * 1000, 3), "ctx": ctx, "launches": 6 if ctx > 256 else 5,
            "weight_bytes": layer_bytes, "kv_bytes_read": kv_read,
            "gbs": round(nb / (ms * 1e-3) / 1e9, 1),
            "frac": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "layer_copies": copies,
            "with_chain": {"us": round(ms_c * 1000, 3), "launches": 4 if ctx > 256 else 3,
                           "gbs": round(nb / (ms_c * 1e-3) / 1e9, 1),
                           "frac": round(nb / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}}


def variants(torch, q4, si, np, K, W):
    out = {}
    # single GEMV 3072^2
    inp = si.workload(si.GEMV_3072, seed=0)
    nb = gemv_bytes(3072, 3072)
    rot = Rotation(q4, q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"])),
                   copies_for(weight_bytes(3072, 3072)))
    x = dev_f16(inp["x"])
    y = torch.empty(3072, dtype=torch.float16, device="cuda")
    us = per_launch_us(torch, lambda i: q4.gemv(rot[i], x, y), K, W)
    out["gemv_3072x3072"] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                             "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4), "bytes": nb}
    del rot

    # the int3 variant of the matmul on the layer set's shapes (uniform random
    # codes), one GEMV at a time and the four back to back
    rng = np.random.default_rng(3)
    i3 = {}
    for key, (n, k) in si.LAYER_SHAPES.items():
        w3, s3 = si.draw_weight3(rng, n, k)
        i3[key] = (Rotation(q4, q4.pack_int3(dev_u32(w3), dev_u16(s3)),
                            copies_for(weight3_bytes(n, k))),
                   dev_f16(si.draw_x(rng, k)), torch.empty(n, dtype=torch.float16, device="cuda"))
    rec = {}
    tot_bytes = 0
    for key, (n, k) in si.LAYER_SHAPES.items():
        r3, xk, yk = i3[key]
        nb3 = weight3_bytes(n, k) + 2 * k + 2 * n
        tot_bytes += nb3
        us3 = per_launch_us(torch, lambda i, r3=r3, xk=xk, yk=yk: q4.gemv(r3[i], xk, yk), K, W)
        rec[key] = {"us": round(us3, 3), "gbs": round(nb3 / us3 / 1e3, 1),
                    "frac": round(nb3 / us3 / 1e3 / PEAK_HBM_GBS, 4), "bytes": nb3}

    def int3_step(i):
        for r3, xk, yk in i3.values():
            q4.gemv(r3[i], xk, yk)

    us_set = per_launch_us(torch, int3_step, K, W)
    rec["set"] = {"us": round(us_set, 3), "gbs": round(tot_bytes / us_set / 1e3, 1),
                  "frac": round(tot_bytes / us_set / 1e3 / PEAK_HBM_GBS, 4), "bytes": tot_bytes}
    out["int3_gemv_phi3_layer_set"] = rec
    del i3
    # int3 fused gate/up + SiLU (2 x 8192 x 3072) and LM head (32064 x 3072, f32 + argmax)
    gw, gs = si.draw_weight3(rng, 8192, 3072)
    uw, us = si.draw_weight3(rng, 8192, 3072)
    gu3_bytes = 2 * weight3_bytes(8192, 3072) + 2 * 3072 + 2 * 8192
    r3 = Rotation(q4, q4.pack_int3_gate_up(dev_u32(gw), dev_u16(gs), dev_u32(uw), dev_u16(us)),
                  copies_for(gu3_bytes))
    x3 = dev_f16(si.draw_x(rng, 3072))
    h3 = torch.empty(8192, dtype=torch.float16, device="cuda")
    us3 = per_launch_us(torch, lambda i: q4.ffn_gate_up_silu(r3[i], x3, h3), K, W)
    del r3
    lw, ls = si.draw_weight3(rng, 32064, 3072)
    lm3_bytes = weight3_bytes(32064, 3072) + 2 * 3072 + 4 * 32064 + 4
    r3 = Rotation(q4, q4.pack_int3(dev_u32(lw), dev_u16(ls)), copies_for(lm3_bytes))
    lg = torch.empty(32064, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    usl = per_launch_us(torch, lambda i: q4.lmhead_f32(r3[i], x3, lg, am), K, W)
    del r3
    out["int3_ffn_and_lm_head"] = {
        "ffn_us": round(us3, 3), "ffn_gbs": round(gu3_bytes / us3 / 1e3, 1), "ffn_bytes": gu3_bytes,
        "lm_head_us": round(usl, 3), "lm_head_gbs": round(lm3_bytes / usl / 1e3, 1),
        "lm_head_bytes": lm3_bytes, "lm_head_launches": 1}

    # fused gate/up + SiLU, then down
    inp = si.workload(si.FFN, seed=0)
    g, u, d = inp["gate"], inp["up"], inp["down"]
    gu_bytes = 2 * weight_bytes(8192, 3072) + 2 * 3072 + 2 * 8192
    rot_gu = Rotation(q4, q4.pack_gate_up(dev_u32(g[0]), dev_u16(g[1]), dev_u32(u[0]),
                                          dev_u16(u[1])), copies_for(gu_bytes))
    rot_d = Rotation(q4, q4.pack(dev_u32(d[0]), dev_u16(d[1])), copies_for(weight_bytes(3072, 8192)))
    x = dev_f16(inp["x"])
    h = torch.empty(8192, dtype=torch.float16, device="cuda")
    yd = torch.empty(3072, dtype=torch.float16, device="cuda")
    kus = {"ffn": per_launch_us(torch, lambda i: q4.ffn_gate_up_silu(rot_gu[i], x, h), K, W),
           "down": per_launch_us(torch, lambda i: q4.gemv(rot_d[i], h, yd), K, W)}
    dbytes = gemv_bytes(3072, 8192)
    out["ffn_fused_8192x3072_plus_down"] = {
        "ffn_us": round(kus["ffn"], 3), "ffn_gbs": round(gu_bytes / kus["ffn"] / 1e3, 1),
        "ffn_frac": round(gu_bytes / kus["ffn"] / 1e3 / PEAK_HBM_GBS, 4),
        "down_us": round(kus["down"], 3), "down_gbs": round(dbytes / kus["down"] / 1e3, 1),
        "bytes": [gu_bytes, dbytes]}
    del rot_gu, rot_d

    # residual add + RMSNorm fused into the QKV GEMV (9216 x 3072), next to
    # the plain GEMV on the same weights: the prologue's cost inside the launch
    inp = si.workload(si.LAYER_SET, seed=0)
    w, s_ = inp["qkv"]
    rng = np.random.default_rng(11)
    rot = Rotation(q4, q4.pack(dev_u32(w), dev_u16(s_)), copies_for(weight_bytes(9216, 3072)))
    x = dev_f16(inp["x3072"])
    res = dev_f16(si.f16_bits(rng.normal(0.0, 2.0, 3072)))
    gam = dev_f16(si.f16_bits(rng.uniform(0.5, 1.5, 3072)))
    hout = torch.empty(3072, dtype=torch.float16, device="cuda")
    y = torch.empty(9216, dtype=torch.float16, device="cuda")
    nb = gemv_bytes(9216, 3072) + 4 * 2 * 3072   # + residual, gamma, residual out
    us_n = per_launch_us(torch, lambda i: q4.add_rmsnorm_gemv(rot[i], x, res, gam, 1e-5, hout, y), K, W)
    us_p = per_launch_us(torch, lambda i: q4.gemv(rot[i], x, y), K, W)
    out["add_rmsnorm_qkv_9216x3072"] = {"us": round(us_n, 3), "plain_gemv_us": round(us_p, 3),
                                        "gbs": round(nb / us_n / 1e3, 1),
                                        "frac": round(nb / us_n / 1e3 / PEAK_HBM_GBS, 4),
                                        "bytes": nb}
    del rot
    # the fused QKV step: RoPE on the 32 q and 32 k heads (96 dims) at
    # position 1000 and the K/V append into a 64-page cache, with and without
    # the add + RMSNorm prologue
    rot = Rotation(q4, q4.pack_rope(dev_u32(w), dev_u16(s_), 96), copies_for(weight_bytes(9216, 3072)))
    cache = torch.zeros((64, 2, 32, 16, 96), dtype=torch.float16, device="cuda")
    pt = torch.arange(64, dtype=torch.int32, device="cuda")
    us_r = per_launch_us(torch, lambda i: q4.qkv_rope_append(rot[i], x, 32, 1000, 10000.0, cache, pt, out=y), K, W)
    us_rn = per_launch_us(torch, lambda i: q4.qkv_rope_append(rot[i], x, 32, 1000, 10000.0, cache, pt, out=y,
                                                              norm=(res, gam, 1e-5, hout)), K, W)
    nb = gemv_bytes(9216, 3072) + 2 * 2 * 3072   # + the K and V rows appended
    out["qkv_rope_append_9216x3072"] = {"us": round(us_r, 3), "with_norm_us": round(us_rn, 3),
                                        "gbs": round(nb / us_r / 1e3, 1),
                                        "frac": round(nb / us_r / 1e3 / PEAK_HBM_GBS, 4),
                                        "bytes": nb}
    del rot, cache

    # paged-attention decode, Phi-3 heads (32 x 96), 4096 positions; caches
    # rotated over >= 1 GiB so the K/V rows come from HBM
    ctx = 4096
    pages = ctx // 16
    kv_bytes = pages * 2 * 16 * 3072 * 2
    ncache = copies_for(kv_bytes)
    caches = [torch.empty((pages, 2, 32, 16, 96), dtype=torch.float16, device="cuda").normal_()
              for _ in range(ncache)]
    pt = torch.randperm(pages, device="cuda").to(torch.int32)
    qv = torch.randn(32 * 96, device="cuda").to(torch.float16)
    ao = torch.empty((32, 96), dtype=torch.float16, device="cuda")
    ws = q4.workspace(qv.device, int(q4.lib.q4_workspace_bytes(q4.OP_ATTENTION, ctx, 32, 96)))
    us = per_launch_us(torch, lambda i: q4.attention_decode(qv, caches[i % ncache], pt, ctx, 32,
                                                            96 ** -0.5, out=ao, ws=ws), K, W)
    nb = kv_bytes + 2 * 2 * 3072 + 4 * pages
    out["attention_decode_32x96_ctx4096"] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                                             "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4),
                                             "bytes": nb, "launches": 2}
    del caches

    # the same attention over the int8 cache (codes + one f32 scale per row),
    # and the quantise-and-append of one token's k and v heads
    pb8 = q4.kv_int8_page_bytes(32, 96)
    kv8_bytes = pages * pb8
    n8 = copies_for(kv8_bytes)
    caches8 = []
    for _ in range(n8):
        c8 = torch.randint(-127, 128, (pages, pb8), dtype=torch.int8, device="cuda").view(torch.uint8)
        sc = c8.view(pages, 2, 32, 16 * 96 + 64)[:, :, :, 16 * 96:]
        sc.copy_(torch.full((pages, 2, 32, 16), 0.01, device="cuda").view(torch.uint8).view(pages, 2, 32, 64))
        caches8.append(c8)
    us8 = per_launch_us(torch, lambda i: q4.attention_decode_int8(qv, caches8[i % n8], pt, ctx, 32, 32, 96,
                                                                   96 ** -0.5, out=ao, ws=ws), K, W)
    nb8 = kv8_bytes + 2 * 2 * 3072 + 4 * pages
    out["attention_decode_int8_32x96_ctx4096"] = {"us": round(us8, 3), "gbs": round(nb8 / us8 / 1e3, 1),
                                                  "frac": round(nb8 / us8 / 1e3 / PEAK_HBM_GBS, 4),
                                                  "bytes": nb8, "launches": 2}
    qkv = torch.randn(9216, device="cuda").to(torch.float16)
    usa = per_launch_us(torch, lambda i: q4.kv_append_int8(qkv, 32, 32, 96, 1000, caches8[i % n8], pt), K, W)
    out["kv_append_int8_32x96"] = {"us": round(usa, 3)}
    del caches8
    out["decode_layer_phi3_ctx1024"] = decode_layer(torch, q4, si, np, K, W, 1024)

    # LM head, f32 logits + argmax
    inp = si.workload(si.LM_HEAD, seed=0)
    nb = gemv_bytes(32064, 3072, out_bytes=4) + 4
    rot = Rotation(q4, q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"])),
                   copies_for(weight_bytes(32064, 3072)))
    x = dev_f16(inp["x"])
    logits = torch.empty(32064, dtype=torch.float32, device="cuda")
    am = torch.empty(1, dtype=torch.int32, device="cuda")
    us = per_launch_us(torch, lambda i: q4.lmhead_f32(rot[i], x, logits, am), K, W)
    out["lm_head_32064x3072_f32_argmax"] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                                            "frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4),
                                            "bytes": nb}
    del rot

    # skinny GEMM (prefill, batched decode): M = 1, 8, 16, 64, 128, 256 on the
    # default path, and the VALU-vs-MFMA crossover over small M
    gm = {}
    inp = si.workload(si.GEMM, seed=0, m=256)
    rot = Rotation(q4, q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"])),
                   copies_for(weight_bytes(16384, 3072)))

    def gemm_us(m, path, steps):
        X = dev_f16(np.ascontiguousarray(inp["X"][:m]))
        Y = torch.empty((m, 16384), dtype=torch.float16, device="cuda")
        return per_launch_us(torch, lambda i: q4.gemm(rot[i], X, Y, path=path), steps, 5)

    for m in (1, 8, 16, 64, 128, 256):
        us = gemm_us(m, q4.GEMM_AUTO, max(20, K // 4))
        nb = weight_bytes(16384, 3072) + 2 * m * 3072 + 2 * m * 16384
        fl = 2.0 * m * 16384 * 3072
        gm[str(m)] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                      "hbm_frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4),
                      "tflops": round(fl / us / 1e6, 2),
                      "mfma_frac": round(fl / us / 1e6 / PEAK_F16_TFLOPS, 4)}
    cross = {}
    for m in (1, 2, 4, 8, 12, 16, 24, 32, 64, 128, 256):
        cross[str(m)] = {"valu_us": round(gemm_us(m, q4.GEMM_VALU, 20), 3),
                         "mfma_us": round(gemm_us(m, q4.GEMM_MFMA, 20), 3)}
    faster = [int(m) for m, v in cross.items() if v["mfma_us"] < v["valu_us"]]
    gm["crossover"] = {"per_m": cross, "smallest_m_mfma_faster": min(faster) if faster else None}
    out["gemm_16384x3072"] = gm
    del rot

    # the same prefill GEMM over int3 weights (uniform random codes)
    w3, s3 = si.draw_weight3(np.random.default_rng(5), 16384, 3072)
    rot = Rotation(q4, q4.pack_int3(dev_u32(w3), dev_u16(s3)), copies_for(weight3_bytes(16384, 3072)))
    g3 = {}
    for m in (1, 8, 16, 64, 128, 256):
        us = gemm_us(m, q4.GEMM_AUTO, max(20, K // 4))
        nb = weight3_bytes(16384, 3072) + 2 * m * 3072 + 2 * m * 16384
        fl = 2.0 * m * 16384 * 3072
        g3[str(m)] = {"us": round(us, 3), "gbs": round(nb / us / 1e3, 1),
                      "hbm_frac": round(nb / us / 1e3 / PEAK_HBM_GBS, 4),
                      "tflops": round(fl / us / 1e6, 2),
                      "mfma_frac": round(fl / us / 1e6 / PEAK_F16_TFLOPS, 4)}
    out["int3_gemm_16384x3072"] = g3
    return out


def gemm_only(torch, q4, si, np, K, W, m: int) -> int:
    """The prefill GEMM (W 16384 x 3072, X [m][3072], default path) alone, for
    rocprofv3 counter runs; prints one JSON line.  Makes the same calibration
    copy as --only layer."""
    if not 1 <= m <= 256:
        print("--gemm-m must be in 1..256", file=sys.stderr)
        return 2
    src = torch.empty(CALIBRATION_BYTES, dtype=torch.uint8, device="cuda")
    torch.empty_like(src).copy_(src)
    torch.cuda.synchronize()
    del src
    inp = si.workload(si.GEMM, seed=0, m=256)
    rot = Rotation(q4, q4.pack(dev_u32(inp["words"]), dev_u16(inp["scales"])),
                   copies_for(weight_bytes(16384, 3072)))
    X = dev_f16(np.ascontiguousarray(inp["X"][:m]))
    Y = torch.empty((m, 16384), dtype=torch.float16, device="cuda")
    us = per_launch_us(torch, lambda i: q4.gemm(rot[i], X, Y), K, W)
    nb = weight_bytes(16384, 3072) + 2 * m * 3072 + 2 * m * 16384
    fl = 2.0 * m * 16384 * 3072
    print(json.dumps({"workload": "gemm_16384x3072", "m": m, "steps": K, "us": round(us, 3),
                      "gbs": round(nb / us / 1e3, 1), "tflops": round(fl / us / 1e6, 2),
                      "mfma_frac": round(fl / us / 1e6 / PEAK_F16_TFLOPS, 4)}), flush=True)
    return 0


def host_cpu():
    """(usable host threads, CPU model name)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS")
    if cap and cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return n, model


def oracle_layer_set(orc, si, inp, threads: int) -> float:
    """Seconds for the oracle to compute the four layer-set GEMVs once, the
    rows of each split over `threads` host threads (each thread one call of
    the oracle on its row range; ctypes releases the interpreter lock, and
    the rows are independent, so the results are the same bits)."""
    from concurrent.futures import ThreadPoolExecutor
    jobs = []
    for key, (n, k) in si.LAYER_SHAPES.items():
        w, s = inp[key]
        x = inp["x8192"] if key == "down" else inp["x3072"]
        step = -(-n // threads)
        jobs += [(w[r:r + step], s[r:r + step], x) for r in range(0, n, step)]
    t = time.perf_counter()
    if threads == 1:
        for w, s, x in jobs:
            orc.gemv(w, s, x)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda j: orc.gemv(*j), jobs))
    return time.perf_counter() - t


def cpu_baseline(si, inp, budget_s: float):
    """The oracle (plain C, f64) on the host cores: whole layer sets (the four
    GEMVs), once on one thread and as many times as fit the budget on every
    usable host thread; the rate is in the metric's unit (effective GB/s of
    the same algorithmic bytes).  `value` is the all-thread rate."""
    import oracle
    orc = oracle.load()
    threads, model = host_cpu()
    set_bytes = sum(gemv_bytes(n, k) for n, k in si.LAYER_SHAPES.values())
    t1 = oracle_layer_set(orc, si, inp, 1)
    runs, tn = [], 0.0
    while tn < budget_s and len(runs) < 20:
        runs.append(oracle_layer_set(orc, si, inp, threads))
        tn += runs[-1]
    best = min(runs)
    return {"value": round(set_bytes / best / 1e9, 5), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the four layer-set GEMVs ({set_bytes} algorithmic bytes), {len(runs)} runs "
                      f"on {threads} threads (fastest taken, {tn:.1f} s in all) and 1 run on one "
                      f"thread ({t1:.1f} s)",
            "us_per_layer": round(best * 1e6, 1),
            "one_thread": {"value": round(set_bytes / t1 / 1e9, 5), "unit": "GB/s",
                           "us_per_layer": round(t1 * 1e6, 1)},
            "host": {"threads_usable": threads, "cpu_model": model, "nproc": os.cpu_count()}}


if __name__ == "__main__":
    sys.exit(main())
