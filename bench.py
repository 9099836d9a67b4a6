"""Benchmark: FMM force evaluation throughput on one MI355X.

A step is one fmm_build + fmm_eval (Morton keys, radix sort, octree, dual-tree
walk, P2M, M2M, M2L, L2L, L2P, P2P, combine) over the headline workload:
N = 10^6 particles, 64-Plummer clustered set (seed 1005), fp64, order 4,
theta 0.7, leaf 32, inputs resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FMM force eval particles/s at N=10^6 fp64 order 4; % FP64 peak (M2L, P2P)"
WORKLOAD = "clustered_1e6_p4"
FP64_VECTOR_PEAK_TFLOPS = 78.6  # MI355X: 256 CU x 2.4 GHz x 64 lanes x 2 (FMA)
FP32_VECTOR_PEAK_TFLOPS = 157.3


def binom(n, k):
    return math.comb(n, k)


def m2l_flops_per_pair(p: int) -> int:
    """Algorithmic flops of one multipole-to-local translation at order p.

    Contraction: |n|+|m| <= p terms, one multiply-add each: 2 C(p+6, 6).
    Derivative tensor of 1/R by the recurrence over levels j = p..0: every entry
    of multi-index k != 0 costs a multiply (one source) or a multiply plus a
    multiply-add (two sources, when the split axis index is >= 2); plus the
    offset (3), |R|^2 (5), the inverse square root (1) and the g_j chain (2p).
    """
    contraction = 2 * binom(p + 6, 6)
    d = 3 + 5 + 1 + 1 + 2 * p
    for j in range(p, -1, -1):
        for deg in range(1, p - j + 1):
            for a in range(deg, -1, -1):
                for b in range(deg - a, -1, -1):
                    c = deg - a - b
                    kk = a if a > 0 else (b if b > 0 else c)
                    d += 3 if kk >= 2 else 1
    return contraction + d


P2P_FLOPS_PER_PAIR = 19  # 3 sub, |r|^2 5, rsqrt 1, 3 mul, 1 add, 3 FMA (6)


def roofline_obj(flops_per_launch, ms, dtype_peak, traffic=None):
    achieved = flops_per_launch / (ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 3), "peak": dtype_peak, "unit": "TFLOP/s",
            "frac": round(achieved / dtype_peak, 4), "traffic": traffic}


def cpu_baseline(pos, mass, cfg):
    from oracle import oracle as orc
    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)
    t0 = time.perf_counter()
    orc.fmm(pos, mass, cfg["order"], cfg["theta"], cfg["leaf"])
    dt = time.perf_counter() - t0
    return {"value": round(cfg["n"] / dt, 1), "unit": "particles/s", "cores": cores, "kind": "oracle",
            "sample": f"the full workload ({cfg['n']} particles, one oracle build+eval, {dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--workload", default=WORKLOAD)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from multipole_body_gravity_amd import Plan, workloads

    cfg = workloads.CONFIGS[args.workload]
    pos, mass = workloads.make(cfg["dist"], cfg["n"], cfg["seed"])
    tdt = torch.float64 if cfg["dtype"] == "f64" else torch.float32
    dev = torch.device("cuda:0")
    tpos = torch.from_numpy(pos).to(dev, tdt)
    tmass = torch.from_numpy(mass).to(dev, tdt)
    plan = Plan(cfg["n"], order=cfg["order"], theta=cfg["theta"], leaf_size=cfg["leaf"], dtype=tdt,
                device=dev)
    phi = torch.empty(cfg["n"], dtype=tdt, device=dev)
    acc = torch.empty(cfg["n"], 3, dtype=tdt, device=dev)

    for _ in range(args.warmup):
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
    torch.cuda.synchronize()

    # work counts of this workload (outside the timed region)
    st = plan.stats()
    lists = plan.copy_lists()
    tree = plan.copy_tree()
    cnt = tree["count"].astype(np.int64)
    tgt = np.repeat(np.arange(st["n_nodes"]), np.diff(lists["p2p_off"]))
    p2p_pairs = int(np.sum(cnt[tgt] * cnt[lists["p2p_src"]]) - cfg["n"])  # minus self terms
    n_m2l = st["n_m2l"]

    plan.set_timing(True)
    stage_sum = {k: 0.0 for k in st["stage_ms"]}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
        s = plan.stats()  # reads the step's HIP-event stage times (synchronizes)
        for k, v in s["stage_ms"].items():
            stage_sum[k] += v
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_avg = {k: v / args.steps for k, v in stage_sum.items()}
    ms_step = wall / args.steps * 1e3

    m2l_flops = n_m2l * m2l_flops_per_pair(cfg["order"])
    p2p_flops = p2p_pairs * P2P_FLOPS_PER_PAIR
    peak = FP64_VECTOR_PEAK_TFLOPS if cfg["dtype"] == "f64" else FP32_VECTOR_PEAK_TFLOPS
    rl = {"m2l": roofline_obj(m2l_flops, stage_avg["m2l"], peak),
          "p2p": roofline_obj(p2p_flops, stage_avg["p2p"], peak)}
    dominant = "m2l" if stage_avg["m2l"] >= stage_avg["p2p"] else "p2p"
    roof = dict(rl[dominant])
    roof["kernel"] = dominant

    out = {
        "metric": METRIC,
        "value": round(cfg["n"] * args.steps / wall, 1),
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "distribution": cfg["dist"], "n": cfg["n"],
                   "order": cfg["order"], "theta": cfg["theta"], "leaf_size": cfg["leaf"],
                   "seed": cfg["seed"]},
        "roofline": roof,
        "roofline_other": rl["p2p" if dominant == "m2l" else "m2l"] | {
            "kernel": "p2p" if dominant == "m2l" else "m2l"},
        "stage_ms": {k: round(v, 4) for k, v in stage_avg.items()},
        "work": {"n_m2l": n_m2l, "p2p_pairs": p2p_pairs, "n_nodes": st["n_nodes"],
                 "n_leaves": st["n_leaves"], "depth": st["depth"],
                 "m2l_flops_per_pair": m2l_flops_per_pair(cfg["order"])},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pos, mass, cfg)
    plan.close()
    print(json.dumps(out))


if __name__ == "__main__":
    main()
