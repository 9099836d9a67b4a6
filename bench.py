"""Benchmark: FMM force evaluation throughput on one MI355X.

A step is one fmm_build + fmm_eval (Morton keys, radix sort, octree, dual-tree
walk, P2M, M2M, M2L, L2L, L2P, P2P, combine) over the headline workload:
N = 10^6 particles, 64-Plummer clustered set (seed 1005), fp64, order 4,
theta 0.7, leaf 32, inputs resident in HBM.  Prints one JSON line: the
throughput over the timed steps, the per-step best of 3 and median of 10, the
roofline of the dominant kernel (and of the other compute kernels) against the
published and the measured peaks, the HBM rates of the memory-bound stages,
and, outside the timed region, the accuracy (p99 and largest relative
acceleration error against direct summation at 4096 seeded targets, the
momentum residual), the cheapest setting that meets the 1e-3 p99 bar on the
same particles, and the CPU oracle's time and its agreement with the GPU.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
    python bench.py --sweep [--sweep-n N] [--sweep-orders 2,4,6,8] [--sweep-thetas ...]
    python bench.py --vjp [--steps K] [--warmup W]   (forward + VJP steps, same workload)
    python bench.py --lattice [--steps K] [--warmup W] (reversible lattice steps, same workload)
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


def _dtensor_flops(p: int, max_kz: int) -> int:
    """Derivative tensor of 1/R by the recurrence over levels j = p..0, for the
    entries with k_z <= max_kz: a multiply (one source) or a multiply plus a
    multiply-add (two sources, when the split axis index is >= 2); plus the
    offset (3), |R|^2 (5), the inverse square root (1) and the g_j chain (2p)."""
    d = 3 + 5 + 1 + 1 + 2 * p
    for j in range(p, -1, -1):
        for deg in range(1, p - j + 1):
            for a in range(deg, -1, -1):
                for b in range(deg - a, -1, -1):
                    c = deg - a - b
                    if c > max_kz:
                        continue
                    kk = a if a > 0 else (b if b > 0 else c)
                    d += 3 if kk >= 2 else 1
    return d


def m2l_flops_per_pair(p: int) -> int:
    """Algorithmic flops of one multipole-to-local translation at order p, in the
    traceless form the kernels evaluate (the same result as the plain Cartesian
    sum: D is harmonic, so moments are folded onto m_z <= 1 once per node and
    locals with n_z >= 2 are rebuilt once per target): one multiply-add for
    every n, m with n_z, m_z <= 1 and |n| + |m| <= p, i.e.
    2 sum_(dn+dm<=p) (2dn+1)(2dm+1), plus the derivative entries with k_z <= 2.
    """
    contraction = 2 * sum((2 * dn + 1) * (2 * dm + 1)
                          for dn in range(p + 1) for dm in range(p + 1 - dn))
    return contraction + _dtensor_flops(p, 2)


def m2l_flops_per_pair_plain(p: int) -> int:
    """The same translation as the plain Cartesian sum over |n| + |m| <= p."""
    return 2 * binom(p + 6, 6) + _dtensor_flops(p, p)


P2P_FLOPS_PER_PAIR = 19  # 3 sub, |r|^2 5, rsqrt 1, 3 mul, 1 add, 3 FMA (6)
# VJP pair: 3 sub, |r|^2 5, rsqrt 1, 1/r^2 and 1/r^3 2, s 3, w 9, r.w 5,
# coefficient 3, coef r + w 6, accumulate 6, ab_j . r 5, Psi 4
P2P_VJP_FLOPS_PER_PAIR = 52


HBM_PEAK_GBS = 8000.0  # MI355X HBM3E


def hbm_stages(cfg, st, stage_ms, kernel_ms):
    """Algorithmic HBM bytes of the memory-bound steps over their measured
    times: the keys stage (bounding box + keys) and the sort stage (seven 9-bit
    radix passes + gather into sorted records) from the stage events, P2M and
    L2P from their kernel events.  Bytes count each array element once: per
    particle, the box reads x, y, z, m and the keys kernel reads x, y, z and
    writes key + index; a radix pass reads the key (histogram) and the key and
    index (scatter) and writes both; the gather reads the index and the input
    and writes the record; P2M reads the records and writes K moments per
    leaf; L2P reads the record, the leaf index, and per leaf the centre and K
    locals, and writes four results."""
    n, nl, nn = cfg["n"], st["n_leaves"], st["n_nodes"]
    w = 8 if cfg["dtype"] == "f64" else 4
    K = (cfg["order"] + 1) * (cfg["order"] + 2) * (cfg["order"] + 3) // 6
    passes = 7
    items = {
        "keys": (n * (4 * w + 3 * w + 8 + 4), stage_ms["keys"], "stage"),
        "sort": (n * (passes * (8 + 12 + 12) + 4 + 4 * w + 4 * w), stage_ms["sort"], "stage"),
        # the sorted keys read once, the leaf index of every particle written,
        # and the node arrays written (level 1, prefix 8, begin, count, parent,
        # first child 4 each, child count 1, centre 24, cell coords 8, criterion
        # record 16: 74 B per node)
        "tree": (n * (8 + 4) + nn * 74, stage_ms["tree"], "stage"),
        # 8 B per emitted list entry (a source id written and read back once)
        # and 16 B per node (its criterion record read once per level)
        "walk": ((st["n_m2l"] + st["n_p2p"]) * 8 + nn * 16, stage_ms["walk"], "stage"),
        "p2m": (n * 4 * w + nl * (12 + 24 + K * w), kernel_ms["p2m"], "kernel"),
        "l2p": (n * (4 * w + 4 + 4 * w) + nl * (24 + K * w), kernel_ms["l2p"], "kernel"),
    }
    out = {}
    for k, (b, ms, how) in items.items():
        if ms > 0:
            gbs = b / (ms * 1e-3) / 1e9
            out[k] = {"bound": "hbm", "bytes": int(b), "ms": round(ms, 4), "achieved": round(gbs, 1),
                      "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                      "timed": how}
    return out


def roofline_obj(flops_per_launch, ms, dtype_peak, traffic=None):
    achieved = flops_per_launch / (ms * 1e-3) / 1e12
    return {"bound": "alu", "achieved": round(achieved, 3), "peak": dtype_peak, "unit": "TFLOP/s",
            "frac": round(achieved / dtype_peak, 4), "traffic": traffic}


# kernel -> (source file whose text the traffic figure is tied to, profile summary)
KERNEL_SOURCES = {
    "p2p": "multipole_body_gravity_amd/csrc/fmm_p2p.hip",
    "m2l_sib": "multipole_body_gravity_amd/csrc/fmm_m2l.hip",
    "m2l_tail": "multipole_body_gravity_amd/csrc/fmm_m2l.hip",
    "vjp_p2p": "multipole_body_gravity_amd/csrc/fmm_p2p.hip",
    "vjp_m2l_sib": "multipole_body_gravity_amd/csrc/fmm_m2l.hip",
}


def source_sha(kernel):
    import hashlib
    path = os.path.join(ROOT, KERNEL_SOURCES[kernel])
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None.

    The summary (profiles/traffic_<kernel>_<workload>.md) holds one line
    'traffic_json: {...}' with the calibrated FETCH_SIZE + WRITE_SIZE bytes and
    the hash of the kernel's source file when the counters were taken; a
    different hash means the kernel changed since, and no figure is reported.
    """
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic_json:"):
                rec = json.loads(line.split(":", 1)[1])
                if rec.get("source_sha") == source_sha(kernel):
                    return rec["bytes_per_launch"]
    return None


def copy_probe(nbytes=1 << 30, reps=5):
    """A plain device copy of known size, for calibrating HBM byte counters."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_read": nbytes, "copy_probe_bytes_written": nbytes,
                      "reps": reps}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def copy_rate_gbs(nbytes=1 << 30, reps=5):
    """A plain 1 GiB device-to-device copy, best of `reps` after one warm-up:
    bytes read + bytes written over its event time."""
    import torch
    dev = torch.device("cuda:0")
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    best = 1e30
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        best = min(best, a.elapsed_time(b))
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (best * 1e-3) / 1e9


def measured_peaks():
    from multipole_body_gravity_amd import fmm
    f64, f32 = fmm.measure_peaks()
    return {"fp64_vector_tflops": round(f64, 2), "fp32_vector_unpacked_tflops": round(f32, 2),
            "hbm_copy_gbs": round(copy_rate_gbs(), 1),
            "how": "fma-chain kernel (fmm_measure_peaks, best of 3) and a 1 GiB device copy "
                   "(read + write bytes, best of 5)"}


def _rel(got, ref):
    nref = np.linalg.norm(ref, axis=-1) if ref.ndim == 2 else np.abs(ref)
    d = np.linalg.norm(got - ref, axis=-1) if ref.ndim == 2 else np.abs(got - ref)
    return d / nref


def direct_reference(tpos, tmass, n, n_targets=4096, seed=4242):
    """fp64 direct sums (fmm_direct) at a seeded sample of targets."""
    import torch

    from multipole_body_gravity_amd import direct
    tg = np.sort(np.random.default_rng(seed).choice(n, min(n_targets, n), replace=False))
    ttg = torch.from_numpy(tg).to(tpos.device)
    rphi, racc = direct(tpos, tmass, ttg)
    return tg, rphi.double().cpu().numpy(), racc.double().cpu().numpy()


def accuracy_vs_direct(ref, phi, acc):
    tg, rphi, racc = ref
    ea = _rel(acc[tg].double().cpu().numpy(), racc)
    ep = _rel(phi[tg].double().cpu().numpy(), rphi)
    return {"targets": int(tg.size), "acc_rel_err_p99": float(np.percentile(ea, 99)),
            "acc_rel_err_max": float(ea.max()), "phi_rel_err_p99": float(np.percentile(ep, 99))}


def momentum_residual(acc, mass):
    """|sum_i m_i a_i| / sum_i m_i |a_i| of the evaluated accelerations (fp64)."""
    a = acc.double()
    m = mass.double()[:, None]
    return float(((m * a).sum(0).norm() / (m[:, 0] * a.norm(dim=1)).sum()).item())


def accuracy_matched(cfg, tpos, tmass, ref, bar=1e-3, steps=5):
    """The cheapest (order, theta) among a few candidates whose p99 relative
    acceleration error against direct summation is within `bar` on the same
    particles: build + eval time (mean of `steps` after two untimed steps) and
    the error of each candidate."""
    import torch

    from multipole_body_gravity_amd import Plan
    n = cfg["n"]
    rows = []
    for order, theta in [(5, 0.6), (6, 0.6), (5, 0.5), (6, 0.5)]:
        plan = Plan(n, order=order, theta=theta, leaf_size=cfg["leaf"], dtype=tpos.dtype,
                    device=tpos.device)
        phi = torch.empty(n, dtype=tpos.dtype, device=tpos.device)
        acc = torch.empty(n, 3, dtype=tpos.dtype, device=tpos.device)
        for _ in range(2):
            plan.build(tpos, tmass)
            plan.eval(phi, acc)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            plan.build(tpos, tmass)
            plan.eval(phi, acc)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) / steps * 1e3
        err = accuracy_vs_direct(ref, phi, acc)
        rows.append({"order": order, "theta": theta, "ms_per_step": round(ms, 3),
                     "value": round(n / (ms * 1e-3), 1), "acc_rel_err_p99": err["acc_rel_err_p99"],
                     "acc_rel_err_max": err["acc_rel_err_max"]})
        plan.close()
        del phi, acc
    ok = [r for r in rows if r["acc_rel_err_p99"] <= bar]
    best = min(ok, key=lambda r: r["ms_per_step"]) if ok else None
    return {"bar_p99": bar, "chosen": best, "candidates": rows,
            "how": f"mean of {steps} build+eval steps each, errors at the same targets as 'accuracy'"}


def cpu_baseline(pos, mass, cfg, phi=None, acc=None):
    """The oracle on the same workload on the host's cores; also the largest
    per-particle relative error of the GPU's outputs (phi, acc: host arrays in
    the caller's order, or None) against it."""
    from oracle import oracle as orc
    cores = len(os.sched_getaffinity(0))
    orc.set_threads(cores)
    t0 = time.perf_counter()
    ref = orc.fmm(pos, mass, cfg["order"], cfg["theta"], cfg["leaf"])
    dt = time.perf_counter() - t0
    out = {"value": round(cfg["n"] / dt, 1), "unit": "particles/s", "cores": cores,
           "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"the full workload ({cfg['n']} particles, one oracle build+eval, {dt:.1f} s)"}
    if acc is not None:
        ea = _rel(acc, ref.acc)
        ep = _rel(phi, ref.phi)
        out["gpu_vs_oracle"] = {"particles": int(cfg["n"]), "acc_rel_err_max": float(ea.max()),
                                "phi_rel_err_max": float(ep.max()),
                                "tolerance": 1e-11 if cfg["dtype"] == "f64" else 1e-4}
    return out


def sweep(args):
    """Accuracy-runtime sweep over order and opening angle on a Hernquist sphere
    (the jz-fmm page's accuracy-runtime comparison, replayed on one GPU): per
    (p, theta) the build+eval time and the acceleration and potential errors
    against direct summation (fmm_direct) at seeded sample particles.  One JSON
    line per configuration."""
    import torch

    from multipole_body_gravity_amd import Plan, direct, workloads
    dev = torch.device("cuda:0")
    n = args.sweep_n
    pos, mass = workloads.make("hernquist", n, 1007)
    tpos = torch.from_numpy(pos).to(dev)
    tmass = torch.from_numpy(mass).to(dev)
    del pos, mass
    smp = np.random.default_rng(77).choice(n, min(args.sweep_targets, n), replace=False)
    tsmp = torch.from_numpy(smp).to(dev)
    rphi, racc = direct(tpos, tmass, tsmp)
    rphi, racc = rphi.cpu().numpy(), racc.cpu().numpy()

    def rel(got, ref):
        nref = np.linalg.norm(ref, axis=-1) if ref.ndim == 2 else np.abs(ref)
        d = np.linalg.norm(got - ref, axis=-1) if ref.ndim == 2 else np.abs(got - ref)
        return d / nref

    for order in [int(x) for x in args.sweep_orders.split(",")]:
        for theta in [float(x) for x in args.sweep_thetas.split(",")]:
            plan = Plan(n, order=order, theta=theta, leaf_size=32, dtype=torch.float64, device=dev)
            phi = torch.empty(n, dtype=torch.float64, device=dev)
            acc = torch.empty(n, 3, dtype=torch.float64, device=dev)
            plan.build(tpos, tmass)
            plan.eval(phi, acc)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                plan.build(tpos, tmass)
                plan.eval(phi, acc)
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / args.steps
            st = plan.stats()
            ea = rel(acc[tsmp].cpu().numpy(), racc)
            ep = rel(phi[tsmp].cpu().numpy(), rphi)
            print(json.dumps({"sweep": "hernquist", "n": n, "order": order, "theta": theta,
                              "leaf_size": 32, "dtype": "f64", "steps": args.steps,
                              "ms_per_step": round(dt * 1e3, 3),
                              "value": round(n / dt, 1), "unit": "particles/s",
                              "acc_rel_err_p99": float(np.percentile(ea, 99)),
                              "acc_rel_err_max": float(ea.max()),
                              "phi_rel_err_p99": float(np.percentile(ep, 99)),
                              "targets": int(smp.size), "n_nodes": st["n_nodes"],
                              "n_m2l": st["n_m2l"], "n_p2p": st["n_p2p"]}), flush=True)
            plan.close()
            del phi, acc
            torch.cuda.empty_cache()


def work_counts(plan, n):
    """Near-field particle pairs and own / transposed M2L entries of the built plan."""
    st = plan.stats()
    lists = plan.copy_lists()
    tree = plan.copy_tree()
    cnt = tree["count"].astype(np.int64)
    tgt = np.repeat(np.arange(st["n_nodes"]), np.diff(lists["p2p_off"]))
    p2p_pairs = int(np.sum(cnt[tgt] * cnt[lists["p2p_src"]]) - n)  # minus self terms
    # own M2L entries (source at the target's level or coarser: the sibling kernel)
    # and transposed ones (deeper sources: the tail kernel)
    lvl = tree["level"].astype(np.int64)
    mt = np.repeat(np.arange(st["n_nodes"]), np.diff(lists["m2l_off"]))
    n_m2l_tr = int(np.sum(lvl[lists["m2l_src"]] > lvl[mt]))
    return st, p2p_pairs, st["n_m2l"] - n_m2l_tr, n_m2l_tr


def vjp_bench(args):
    """Forward and backward on the headline workload: a step is fmm_build +
    fmm_eval + fmm_vjp (the VJP with seeded standard-normal sensitivities), K
    timed steps after W warm-up steps, HIP events around every stage and main
    kernel of each step (collected at the next build's first synchronization,
    so the loop carries no extra synchronization).  One JSON line."""
    import torch

    from multipole_body_gravity_amd import Plan, workloads
    cfg = workloads.CONFIGS[args.workload]
    n = cfg["n"]
    pos, mass = workloads.make(cfg["dist"], n, cfg["seed"])
    rng = np.random.default_rng(2024)
    pb = rng.standard_normal(n)
    ab = rng.standard_normal((n, 3))
    tdt = torch.float64 if cfg["dtype"] == "f64" else torch.float32
    dev = torch.device("cuda:0")
    tpos, tmass = torch.from_numpy(pos).to(dev, tdt), torch.from_numpy(mass).to(dev, tdt)
    tpb, tab = torch.from_numpy(pb).to(dev, tdt), torch.from_numpy(ab).to(dev, tdt)
    plan = Plan(n, order=cfg["order"], theta=cfg["theta"], leaf_size=cfg["leaf"], dtype=tdt,
                device=dev)
    phi = torch.empty(n, dtype=tdt, device=dev)
    acc = torch.empty(n, 3, dtype=tdt, device=dev)
    xb = torch.empty(n, 3, dtype=tdt, device=dev)
    mb = torch.empty(n, dtype=tdt, device=dev)
    for _ in range(args.warmup):
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
        plan.vjp(tpb, tab, xb, mb)
    torch.cuda.synchronize()

    plan.set_timing(2)  # the main kernels and the fmm_vjp call, not every stage
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
        plan.vjp(tpb, tab, xb, mb)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s = plan.stats()
    assert s["timed_vjps"] == args.steps and s["timed_evals"] == args.steps, s
    kern = s["kernel_ms"]
    # work counts of the last build (every build of these inputs is the same)
    st, p2p_pairs, n_m2l_own, n_m2l_tr = work_counts(plan, n)

    fpp = m2l_flops_per_pair(cfg["order"])
    peak = FP64_VECTOR_PEAK_TFLOPS if cfg["dtype"] == "f64" else FP32_VECTOR_PEAK_TFLOPS
    flops = {"vjp_p2p": p2p_pairs * P2P_VJP_FLOPS_PER_PAIR, "vjp_m2l_sib": n_m2l_own * fpp,
             "p2p": p2p_pairs * P2P_FLOPS_PER_PAIR, "m2l_sib": n_m2l_own * fpp,
             "m2l_tail": n_m2l_tr * fpp}
    rl = {k: roofline_obj(f, kern[k], peak, measured_traffic(k, args.workload))
          for k, f in flops.items() if kern[k] > 0}
    dominant = max(rl, key=lambda k: kern[k])
    roof = dict(rl[dominant])
    roof["kernel"] = dominant
    out = {
        "metric": "FMM forward + VJP step particles/s at N=10^6 fp64 order 4",
        "value": round(n * args.steps / wall, 1),
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "ms_vjp": round(s["stage_ms"]["vjp"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "distribution": cfg["dist"], "n": n,
                   "order": cfg["order"], "theta": cfg["theta"], "leaf_size": cfg["leaf"],
                   "seed": cfg["seed"], "sensitivities": "standard normal, seed 2024"},
        "roofline": roof,
        "roofline_other": {k: v for k, v in rl.items() if k != dominant},
        "kernel_ms": {k: round(v, 4) for k, v in kern.items()},
        "work": {"p2p_pairs": p2p_pairs, "n_m2l_own": n_m2l_own, "n_m2l_transposed": n_m2l_tr,
                 "p2p_vjp_flops_per_pair": P2P_VJP_FLOPS_PER_PAIR,
                 "p2p_flops_per_pair": P2P_FLOPS_PER_PAIR, "m2l_flops_per_pair": fpp},
    }
    if not args.no_cpu_baseline:
        from oracle import oracle as orc
        cores = len(os.sched_getaffinity(0))
        orc.set_threads(cores)
        t2 = time.perf_counter()
        orc.fmm_vjp(pos, mass, pb, ab, cfg["order"], cfg["theta"], cfg["leaf"])
        dt = time.perf_counter() - t2
        out["cpu_baseline"] = {"value": round(n / dt, 1), "unit": "particles/s", "cores": cores,
                               "kind": "oracle",
                               "sample": f"the full workload ({n} particles, one oracle forward "
                                         f"and VJP, {dt:.1f} s)"}
    plan.close()
    print(json.dumps(out))


def lattice_bench(args):
    """Reversible integer-lattice kick-drift-kick steps (fmm_lattice_steps) on
    the headline workload's positions with velocities N(0, 0.1), dt = 1e-3,
    dx = dv = 2^-32: one call of K steps timed (K + 1 force evaluations, two
    kicks and a drift per step), then K backward steps outside the timed region
    that must restore the state bit for bit.  One JSON line."""
    import torch

    from multipole_body_gravity_amd import Plan, workloads
    cfg = workloads.CONFIGS[args.workload]
    n = cfg["n"]
    pos, mass = workloads.make(cfg["dist"], n, cfg["seed"])
    q0, u0 = workloads.lattice_state(pos, 301)
    tdt = torch.float64 if cfg["dtype"] == "f64" else torch.float32
    dev = torch.device("cuda:0")
    tq, tu = torch.from_numpy(q0).to(dev), torch.from_numpy(u0).to(dev)
    tmass = torch.from_numpy(mass).to(dev, tdt)
    plan = Plan(n, order=cfg["order"], theta=cfg["theta"], leaf_size=cfg["leaf"], dtype=tdt,
                device=dev)
    dx, dv, dt = workloads.LATTICE_DX, workloads.LATTICE_DV, 1e-3
    if args.warmup:
        plan.lattice_steps(tq, tu, tmass, dx, dv, dt, args.warmup, +1)
    torch.cuda.synchronize()
    qs, us = tq.clone(), tu.clone()
    plan.set_timing(2)  # the main kernels only: stage events slow the step
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    plan.lattice_steps(tq, tu, tmass, dx, dv, dt, args.steps, +1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    s = plan.stats()
    plan.set_timing(False)
    # work counts of the last step's build (outside the timed region)
    st, p2p_pairs, n_m2l_own, n_m2l_tr = work_counts(plan, n)
    plan.lattice_steps(tq, tu, tmass, dx, dv, dt, args.steps, -1)
    torch.cuda.synchronize()
    reversible = bool(torch.equal(tq, qs) and torch.equal(tu, us))
    kern = s["kernel_ms"]
    fpp = m2l_flops_per_pair(cfg["order"])
    peak = FP64_VECTOR_PEAK_TFLOPS if cfg["dtype"] == "f64" else FP32_VECTOR_PEAK_TFLOPS
    flops = {"m2l_sib": n_m2l_own * fpp, "m2l_tail": n_m2l_tr * fpp,
             "p2p": p2p_pairs * P2P_FLOPS_PER_PAIR}
    rl = {k: roofline_obj(flops[k], kern[k], peak) for k in flops if kern[k] > 0}
    dominant = max(rl, key=lambda k: kern[k])
    roof = dict(rl[dominant])
    roof["kernel"] = dominant
    out = {
        "metric": "reversible lattice KDK step particles/s at N=10^6 fp64 order 4",
        "value": round(n * args.steps / wall, 1),
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "ms_per_force_eval": round(wall / (args.steps + 1) * 1e3, 4),
        "reversible": reversible,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "distribution": cfg["dist"], "n": n,
                   "order": cfg["order"], "theta": cfg["theta"], "leaf_size": cfg["leaf"],
                   "seed": cfg["seed"], "dt": dt, "dx": dx, "dv": dv,
                   "velocities": "N(0, 0.1) per component, seed 301"},
        "roofline": roof,
        "kernel_ms": {k: round(v, 4) for k, v in kern.items() if not k.startswith("vjp")},
    }
    plan.close()
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mutual", action="store_true",
                    help="sum the sibling leaves' near field mutually (fmm_set_mutual_near_field)")
    ap.add_argument("--no-accuracy-matched", action="store_true",
                    help="skip the search for the cheapest setting within the 1e-3 p99 bar")
    ap.add_argument("--workload", default=WORKLOAD)
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a 1 GiB device copy (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="accuracy-runtime sweep on a Hernquist sphere instead of the headline line")
    ap.add_argument("--sweep-n", type=int, default=40_000_000)
    ap.add_argument("--sweep-orders", default="2,4,6,8")
    ap.add_argument("--sweep-thetas", default="0.4,0.5,0.6,0.7")
    ap.add_argument("--sweep-targets", type=int, default=2048)
    ap.add_argument("--lattice", action="store_true",
                    help="time reversible integer-lattice steps instead of the forward step")
    ap.add_argument("--vjp", action="store_true",
                    help="time forward + VJP steps (build, eval, fmm_vjp) instead of the forward step")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on one GPU only (no multi-GPU path); use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.copy_probe:
        copy_probe()
        return
    if args.sweep:
        if args.steps == ap.get_default("steps"):
            args.steps = 3
        sweep(args)
        return
    if args.vjp:
        vjp_bench(args)
        return
    if args.lattice:
        lattice_bench(args)
        return

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
    if args.mutual:
        plan.set_mutual_near_field(True)
    phi = torch.empty(cfg["n"], dtype=tdt, device=dev)
    acc = torch.empty(cfg["n"], 3, dtype=tdt, device=dev)

    for _ in range(args.warmup):
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
    torch.cuda.synchronize()

    # HIP events around the near-field kernels of each step (timing mode 3), on
    # the stream they are launched on; the library reads them at the
    # synchronizations a build makes anyway, so the timed loop carries no
    # extra synchronization.  Every event is a marker that slows the step a
    # little by itself, so the other kernels' times (mode 2) and the stage
    # times (mode 1) come from separate passes after the timed one.
    plan.set_timing(3)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for e0, e1 in evs:  # torch creates an event at its first record: not in the timed loop
        e0.record()
        e1.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        evs[k][0].record()
        plan.build(tpos, tmass)
        plan.eval(phi, acc)
        evs[k][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = [a.elapsed_time(b) for a, b in evs]
    s = plan.stats()  # means over the K timed steps
    assert s["timed_builds"] == args.steps and s["timed_evals"] == args.steps, s
    kern_timed = s["kernel_ms"]
    ms_step = wall / args.steps * 1e3
    # side passes: every main kernel's events, then the stages'
    k_side = min(args.steps, 20)
    side_ms = {}
    for mode in (2, 1):
        plan.set_timing(mode)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for _ in range(k_side):
            plan.build(tpos, tmass)
            plan.eval(phi, acc)
        torch.cuda.synchronize()
        side_ms[mode] = (time.perf_counter() - t1) / k_side * 1e3
        if mode == 2:
            kern_avg = dict(plan.stats()["kernel_ms"])
        else:
            stage_avg = plan.stats()["stage_ms"]
    plan.set_timing(0)
    for k in ("p2p", "p2p_combine"):  # the near field: from the timed steps
        kern_avg[k] = kern_timed[k]
    # work counts of the last build (every build of these inputs is the same);
    # taken after the timed steps, so that the GPU does not sit idle between
    # the warm-up and the timed steps
    st, p2p_pairs, n_m2l_own, n_m2l_tr = work_counts(plan, cfg["n"])
    n_m2l = st["n_m2l"]

    # accuracy of the last step's outputs, outside the timed region
    ref = direct_reference(tpos, tmass, cfg["n"])
    accuracy = accuracy_vs_direct(ref, phi, acc)
    accuracy["bar_p99"] = 1e-3
    accuracy["bar_met"] = bool(accuracy["acc_rel_err_p99"] <= 1e-3)
    accuracy["momentum_residual"] = momentum_residual(acc, tmass)
    peaks = measured_peaks()

    # algorithmic flops per launch of each compute kernel, over its measured
    # average launch time (HIP events recorded on the launch stream)
    fpp = m2l_flops_per_pair(cfg["order"])
    flops = {"m2l_sib": n_m2l_own * fpp, "m2l_tail": n_m2l_tr * fpp,
             "p2p": p2p_pairs * P2P_FLOPS_PER_PAIR}
    peak = FP64_VECTOR_PEAK_TFLOPS if cfg["dtype"] == "f64" else FP32_VECTOR_PEAK_TFLOPS
    rl = {k: roofline_obj(flops[k], kern_avg[k], peak, measured_traffic(k, args.workload))
          for k in flops if kern_avg[k] > 0}
    mpeak = peaks["fp64_vector_tflops"] if cfg["dtype"] == "f64" else \
        peaks["fp32_vector_unpacked_tflops"]
    for v in rl.values():
        v["frac_of_measured_peak"] = round(v["achieved"] / mpeak, 4)
    dominant = max(rl, key=lambda k: kern_avg[k])
    roof = dict(rl[dominant])
    roof["kernel"] = dominant
    sorted_ms = sorted(step_ms)

    out = {
        "metric": METRIC,
        "value": round(cfg["n"] * args.steps / wall, 1),
        "unit": "particles/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "step_ms": {"best_of_3": round(min(step_ms[:3]), 4),
                    "median_of_10": round(float(np.median(step_ms[:10])), 4),
                    "min": round(sorted_ms[0], 4), "max": round(sorted_ms[-1], 4),
                    "how": "HIP events on the launch stream around each timed build + eval; "
                           "best of the first 3, median of the first 10"},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "distribution": cfg["dist"], "n": cfg["n"],
                   "order": cfg["order"], "theta": cfg["theta"], "leaf_size": cfg["leaf"],
                   "seed": cfg["seed"], "near_field": "mutual siblings" if args.mutual else "directed"},
        "roofline": roof,
        "roofline_other": {k: v for k, v in rl.items() if k != dominant},
        "hbm": hbm_stages(cfg, st, stage_avg, kern_avg),
        "accuracy": accuracy,
        "measured_peaks": peaks,
        "stage_ms": {k: round(v, 4) for k, v in stage_avg.items() if k != "vjp"},
        "stage_ms_how": f"a separate pass of {k_side} steps with the stage events on "
                        f"({side_ms[1]:.4f} ms per step there)",
        "kernel_ms_how": "p2p and p2p_combine from the timed steps (their events are the only "
                         f"ones there); the others from a pass of {k_side} steps with every main "
                         f"kernel's events ({side_ms[2]:.4f} ms per step there)",
        "kernel_ms": {k: round(v, 4) for k, v in kern_avg.items() if not k.startswith("vjp")},
        "work": {"n_m2l": n_m2l, "n_m2l_own": n_m2l_own, "n_m2l_transposed": n_m2l_tr,
                 "p2p_pairs": p2p_pairs, "n_nodes": st["n_nodes"],
                 "n_leaves": st["n_leaves"], "depth": st["depth"],
                 "m2l_flops_per_pair": fpp, "p2p_flops_per_pair": P2P_FLOPS_PER_PAIR,
                 "m2l_flops_per_pair_plain_cartesian": m2l_flops_per_pair_plain(cfg["order"])},
    }
    plan.close()
    if not args.no_accuracy_matched:
        out["accuracy_matched"] = accuracy_matched(cfg, tpos, tmass, ref)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pos, mass, cfg, phi.double().cpu().numpy(),
                                           acc.double().cpu().numpy())
    print(json.dumps(out))


if __name__ == "__main__":
    main()
