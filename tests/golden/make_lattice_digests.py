"""Writes tests/golden/lattice_256_digests.txt: per tree level, the totals of
the oracle's per-target list digests for the two 256^3 displaced-lattice
workloads (fp32 order 4 theta 0.7 leaf 64; fp64 order 8 theta 0.5 leaf 64).

Calls only the oracle (digest-mode walk) and the seeded input generators.  A
target's digest is its entry count and the sum mod 2^64 of SplitMix64 hashes
of its sources; a level's line holds the number of targets there and the sums
of their counts and hashes (mod 2^64), for the M2L and P2P lists.

    python tests/golden/make_lattice_digests.py
"""
from __future__ import annotations

import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from multipole_body_gravity_amd import workloads as W  # noqa: E402
from oracle import oracle as orc  # noqa: E402

OUT = os.path.join(HERE, "lattice_256_digests.txt")
NAMES = ["lattice_256_f32", "lattice_256_p8"]


def level_totals(level, dig):
    rows = []
    with np.errstate(over="ignore"):
        for lv in range(int(level.max()) + 1):
            sel = level == lv
            rows.append((lv, int(sel.sum()),
                         int(dig["m2l_cnt"][sel].sum(dtype=np.uint64)),
                         int(dig["m2l_hash"][sel].sum(dtype=np.uint64)),
                         int(dig["p2p_cnt"][sel].sum(dtype=np.uint64)),
                         int(dig["p2p_hash"][sel].sum(dtype=np.uint64))))
    return rows


def main():
    lines = ["# Per-level totals of the oracle's per-target interaction-list digests",
             "# (count, and sum mod 2^64 of SplitMix64(seed 0) outputs number src+1) for the",
             "# 256^3 displaced-lattice workloads; written by make_lattice_digests.py.",
             "# workload level n_targets m2l_entries m2l_hash p2p_entries p2p_hash"]
    for name in NAMES:
        c = W.CONFIGS[name]
        pos, mass = W.make(c["dist"], c["n"], c["seed"])
        if c["dtype"] == "f32":  # the values the fp32 path is given
            pos = pos.astype(np.float32).astype(np.float64)
            mass = mass.astype(np.float32).astype(np.float64)
        r = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], digests="walk")
        for lv, nt, mc, mh, pc, ph in level_totals(r.level, r.digests):
            lines.append(f"{name} {lv} {nt} {mc} {mh:016x} {pc} {ph:016x}")
        print(name, "m2l", r.n_m2l, "p2p", r.n_p2p, flush=True)
    with open(OUT, "w") as f:
        f.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    main()
