"""GPU path vs CPU oracle, element by element, through the C-ABI.

Keys, permutation, tree and interaction lists must be bit-identical; potential
and acceleration must agree per particle to 1e-11 relative in fp64 and 1e-4 in
fp32 (max over particles of |a - a_ref| / |a_ref|; a particle whose reference
acceleration is below 1e-3 of the median is normalised by that floor instead
and counted separately).
"""
import sys

import numpy as np
import pytest

from multipole_body_gravity_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = {"f64": 1e-11, "f32": 1e-4}


def _torch():
    import torch
    return torch


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu_run(pos, mass, order, theta, leaf, dt, timing=False, mutual=None):
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    tdt = torch.float64 if dt == "f64" else torch.float32
    dev = torch.device("cuda:0")
    plan = Plan(pos.shape[0], order=order, theta=theta, leaf_size=leaf, dtype=tdt, device=dev)
    if mutual is not None:
        plan.set_mutual_near_field(mutual)
    if timing:
        plan.set_timing(True)
    plan.build(torch.from_numpy(pos).to(dev, tdt), torch.from_numpy(mass).to(dev, tdt))
    phi, acc = plan.eval()
    torch.cuda.synchronize()
    return plan, phi.double().cpu().numpy(), acc.double().cpu().numpy()


def inputs(dist, n, seed, dt):
    pos, mass = W.make(dist, n, seed)
    if dt == "f32":  # the oracle sees exactly the values the GPU gets
        pos = pos.astype(np.float32).astype(np.float64)
        mass = mass.astype(np.float32).astype(np.float64)
    return pos, mass


def rel_err(got, ref, floor_frac=1e-3):
    nref = np.linalg.norm(ref, axis=-1) if ref.ndim == 2 else np.abs(ref)
    diff = np.linalg.norm(got - ref, axis=-1) if ref.ndim == 2 else np.abs(got - ref)
    med = np.median(nref) if nref.size else 0.0
    floor = floor_frac * med
    small = nref < floor
    e = diff / np.where(small, floor, np.where(nref > 0, nref, 1.0))
    return e, int(small.sum())


def check_structure(plan, ref, sample_targets=None):
    keys, perm = plan.copy_keys()
    assert np.array_equal(keys, ref.keys), "sorted keys differ"
    assert np.array_equal(perm, ref.perm), "permutation differs"
    tree = plan.copy_tree()
    for f in ("level", "prefix", "begin", "count", "parent", "first_child", "n_child"):
        assert np.array_equal(tree[f], getattr(ref, f)), f"tree field {f} differs"
    lists = plan.copy_lists()
    if sample_targets is None:
        for f in ("m2l_off", "m2l_src", "p2p_off", "p2p_src"):
            assert np.array_equal(lists[f], getattr(ref, f)), f"list {f} differs"
    else:
        for a in sample_targets:
            for k in ("m2l", "p2p"):
                g = lists[k + "_src"][lists[k + "_off"][a]:lists[k + "_off"][a + 1]]
                r = getattr(ref, k + "_src")[getattr(ref, k + "_off")[a]:getattr(ref, k + "_off")[a + 1]]
                assert np.array_equal(g, r), f"{k} list of node {a} differs"


def check_values(phi, acc, ref, dt, idx=None, no_floor=False):
    """Per-particle relative errors against the oracle.  no_floor: the
    benchmark workloads, where no particle may need the small-reference floor
    (every particle is held to the plain relative bar)."""
    if idx is None:
        idx = np.arange(phi.shape[0])
    ea, na = rel_err(acc[idx], ref.acc[idx])
    ep, npf = rel_err(phi[idx], ref.phi[idx])
    say(f"    max rel err acc {ea.max():.3g} phi {ep.max():.3g} (floored {na} acc, {npf} phi)")
    assert ea.max() <= TOL[dt], f"acc rel err {ea.max():.3g}"
    assert ep.max() <= TOL[dt], f"phi rel err {ep.max():.3g}"
    if no_floor:
        assert na == 0 and npf == 0, f"floored particles on a benchmark workload: {na}, {npf}"


CASES = [
    # dist, n, seed, order, theta, leaf, dtype
    ("uniform", 4096, 1001, 4, 0.7, 32, "f64"),
    ("plummer", 10000, 1002, 4, 0.7, 32, "f64"),
    ("clustered", 20000, 31, 4, 0.7, 32, "f64"),
    ("clustered", 20000, 31, 4, 0.7, 32, "f32"),
    ("plummer", 6000, 32, 6, 0.5, 16, "f64"),
    ("uniform", 1037, 33, 3, 0.6, 7, "f64"),
    ("plummer", 777, 34, 2, 0.4, 1, "f64"),
    ("clustered", 5000, 35, 5, 0.55, 100, "f32"),
    ("uniform", 3000, 36, 0, 0.7, 20, "f64"),
    ("uniform", 3000, 36, 1, 0.7, 20, "f64"),
    ("plummer", 3000, 37, 7, 0.7, 40, "f64"),
    ("plummer", 3000, 37, 8, 0.5, 40, "f64"),
    ("plummer", 3000, 37, 8, 0.5, 40, "f32"),
    ("plummer", 3000, 38, 9, 0.6, 24, "f64"),
    ("clustered", 4000, 39, 10, 0.5, 32, "f64"),
    ("uniform", 2500, 40, 9, 0.7, 16, "f32"),
    ("plummer", 2000, 41, 10, 0.6, 40, "f32"),
    # 4041, 4104 and 5233 transposed entries: the one-block walk tail on the
    # second build with one and two sort passes (131, 290 and 157 nodes)
    ("plummer", 1500, 42, 4, 0.7, 64, "f64"),
    ("clustered", 3000, 44, 4, 0.7, 64, "f32"),
    ("plummer", 2500, 46, 2, 0.7, 128, "f64"),
    # the one-block front: the largest set of its first instance (every
    # thread holds eight particles, the last ones partly), the smallest and
    # the largest of its second (8-bit digits), and the smallest set of the
    # multi-block path
    ("uniform", 8000, 47, 4, 0.7, 32, "f64"),
    ("clustered", 8001, 48, 3, 0.6, 16, "f32"),
    ("plummer", 11264, 49, 4, 0.7, 32, "f64"),
    ("clustered", 11264, 50, 5, 0.6, 24, "f32"),
    ("uniform", 11265, 51, 4, 0.7, 32, "f64"),
]


@pytest.mark.parametrize("dist,n,seed,order,theta,leaf,dt", CASES)
def test_parity_small(orc, dist, n, seed, order, theta, leaf, dt):
    """Structure and values against the oracle after the first build (the
    walk's multi-block path for the transposed keys) and after a second build
    on the same plan (the one-block path wherever the first walk found at most
    3/4 of its capacity, 6144 keys, with 17-bit node ids at most)."""
    say(f"  case {dist} n={n} p={order} theta={theta} leaf={leaf} {dt}")
    pos, mass = inputs(dist, n, seed, dt)
    plan, phi, acc = gpu_run(pos, mass, order, theta, leaf, dt)
    ref = orc.fmm(pos, mass, order, theta, leaf)
    assert not plan.stats()["walk_one_block"]
    check_structure(plan, ref)
    check_values(phi, acc, ref, dt, no_floor=(seed in (1001, 1002)))
    torch = _torch()
    phi1, acc1 = phi, acc
    tdt = torch.float64 if dt == "f64" else torch.float32
    dev = torch.device("cuda:0")
    plan.build(torch.from_numpy(pos).to(dev, tdt), torch.from_numpy(mass).to(dev, tdt))
    p2, a2 = plan.eval()
    torch.cuda.synchronize()
    st = plan.stats()
    # the transposed entries: sources deeper than their target
    lev = ref.level.astype(np.int64)
    n_tr = 0
    for k in ("m2l", "p2p"):
        off, src = getattr(ref, k + "_off"), getattr(ref, k + "_src")
        tgt = np.repeat(np.arange(len(off) - 1), np.diff(off))
        n_tr += int(np.count_nonzero(lev[src] > lev[tgt]))
    say(f"    second build: one-block walk tail {st['walk_one_block']} ({n_tr} transposed entries)")
    nn = len(ref.level)
    assert st["walk_one_block"] == (n_tr <= 6144 and nn <= 65536), "walk tail path"
    check_structure(plan, ref)
    phi2, acc2 = p2.double().cpu().numpy(), a2.double().cpu().numpy()
    assert np.array_equal(phi2, phi1) and np.array_equal(acc2, acc1), "second build differs"
    plan.close()


def test_walk_one_block_overflow(orc):
    """A plan whose last walk had no transposed entries takes the one-block
    path; the next positions have 58637 of them, more than it holds: the walk
    is repeated on the multi-block path and the lists and values match the
    oracle."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    n = 10000
    plan = Plan(n, order=4, theta=0.7, leaf_size=32, dtype=torch.float64, device=dev)
    pos_u, mass_u = inputs("uniform", n, 1001, "f64")
    for _ in range(2):
        plan.build(torch.from_numpy(pos_u).to(dev), torch.from_numpy(mass_u).to(dev))
    pos, mass = inputs("plummer", n, 1002, "f64")
    say(f"  after uniform builds: one-block {plan.stats()['walk_one_block']}")
    plan.build(torch.from_numpy(pos).to(dev), torch.from_numpy(mass).to(dev))
    phi, acc = plan.eval()
    torch.cuda.synchronize()
    st = plan.stats()
    say(f"  plummer build: one-block {st['walk_one_block']}, walk repeats {st['walk_retries']}")
    assert st["walk_retries"] >= 1 and not st["walk_one_block"]
    ref = orc.fmm(pos, mass, 4, 0.7, 32)
    check_structure(plan, ref)
    check_values(phi.double().cpu().numpy(), acc.double().cpu().numpy(), ref, "f64",
                 no_floor=True)
    plan.close()


MUTUAL_CASES = [
    # dist, n, seed, order, theta, leaf, dtype
    ("uniform", 4096, 1001, 4, 0.7, 32, "f64"),
    ("clustered", 20000, 31, 4, 0.7, 32, "f32"),
    ("plummer", 6000, 32, 6, 0.5, 16, "f64"),
    ("uniform", 1037, 33, 3, 0.6, 7, "f64"),
    ("plummer", 777, 34, 2, 0.4, 1, "f64"),
    ("clustered", 5000, 35, 5, 0.55, 100, "f64"),  # groups over 256 particles stay directed
    ("uniform", 300, 36, 4, 0.7, 1000, "f64"),      # the root is the only leaf
]


@pytest.mark.parametrize("dist,n,seed,order,theta,leaf,dt", MUTUAL_CASES)
def test_mutual_near_field_parity(orc, dist, n, seed, order, theta, leaf, dt):
    """The mutual near field of sibling groups (fmm_set_mutual_near_field):
    the same lists and tree as the oracle, values to the same tolerance,
    bitwise repeatable, and equal to the directed form to rounding."""
    say(f"  mutual case {dist} n={n} p={order} theta={theta} leaf={leaf} {dt}")
    pos, mass = inputs(dist, n, seed, dt)
    plan, phi, acc = gpu_run(pos, mass, order, theta, leaf, dt, mutual=True)
    ref = orc.fmm(pos, mass, order, theta, leaf)
    check_structure(plan, ref)
    check_values(phi, acc, ref, dt)
    phi2, acc2 = (t.double().cpu().numpy() for t in plan.eval())
    assert np.array_equal(phi, phi2) and np.array_equal(acc, acc2)
    plan.close()
    _, dphi, dacc = gpu_run(pos, mass, order, theta, leaf, dt, mutual=False)
    ea, _ = rel_err(acc, dacc)
    assert ea.max() <= TOL[dt]


def test_two_body_and_single(orc):
    rows = np.array([[0, 0, 0, 2.0], [3, 4, 0, 0.5]])
    plan, phi, acc = gpu_run(rows[:, :3].copy(), rows[:, 3].copy(), 4, 0.7, 2, "f64")
    assert np.allclose(phi, [-0.1, -0.4], rtol=1e-15)
    assert np.allclose(acc, [[0.012, 0.016, 0], [-0.048, -0.064, 0]], rtol=1e-14, atol=1e-18)
    plan.close()
    plan, phi, acc = gpu_run(np.array([[0.3, 0.2, 0.1]]), np.array([1.0]), 4, 0.7, 1, "f64")
    assert phi[0] == 0.0 and np.all(acc == 0.0)
    plan.close()


@pytest.mark.parametrize("kind", ["line", "plane", "tight_cluster", "leaf_eq_n", "leaf_n_plus_1",
                                  "root_leaf_big", "leaf_1500", "leaf_2500"])
def test_degenerate_inputs(orc, kind):
    rng = np.random.default_rng(41)
    leaf = 8
    if kind == "line":
        pos = np.zeros((500, 3))
        pos[:, 0] = rng.random(500)
    elif kind == "plane":
        pos = np.zeros((800, 3))
        pos[:, :2] = rng.random((800, 2))
        pos[:, 2] = 0.25
    elif kind == "tight_cluster":  # 150 particles inside one level-21 cell
        pos = np.vstack([rng.random((400, 3)), 0.5 + 1e-9 * rng.random((150, 3))])
    elif kind == "leaf_eq_n":
        pos = rng.random((8, 3))
    elif kind == "leaf_n_plus_1":
        pos = rng.random((9, 3))
    elif kind in ("leaf_1500", "leaf_2500"):
        # leaf windows of 1501 and 2501 keys: the widest span the tree's
        # one-launch window maximum takes, and one past it (sparse-table passes)
        pos = np.vstack([rng.random((3000, 3)), 0.3 + 0.01 * rng.random((3000, 3))])
        leaf = int(kind[5:])
    else:
        pos = rng.random((300, 3))
        leaf = 1000
    mass = 0.5 + rng.random(pos.shape[0])
    say(f"  case {kind} n={pos.shape[0]}")
    plan, phi, acc = gpu_run(pos, mass, 4, 0.6, leaf, "f64")
    ref = orc.fmm(pos, mass, 4, 0.6, leaf)
    check_structure(plan, ref)
    check_values(phi, acc, ref, "f64")
    plan.close()


def test_tree_room_regrowth(orc):
    """The tree's second phase is queued with the previous build's node count
    plus slack as room, before the count is read back: a set with many more
    nodes (pairs 1e-6 apart, whose cells go down to the deepest level) on a
    plan sized by a uniform set takes the repeat with room, and the uniform
    set after it the queued phase again; structure and values against the
    oracle each time."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(73)
    n = 4096
    uni = rng.random((n, 3))
    centres = rng.random((n // 2, 3))
    d = rng.standard_normal((n // 2, 3))
    d *= 1e-6 / np.linalg.norm(d, axis=1, keepdims=True)
    pairs = np.empty((n, 3))
    pairs[0::2] = centres
    pairs[1::2] = centres + d
    mass = 0.5 + rng.random(n)
    plan = Plan(n, order=4, theta=0.6, leaf_size=1, dtype=torch.float64, device=dev)
    counts = []
    for label, pos in (("uniform", uni), ("pairs", pairs), ("uniform again", uni)):
        say(f"  tree room: {label}")
        plan.build(torch.from_numpy(pos).to(dev), torch.from_numpy(mass).to(dev))
        phi, acc = plan.eval()
        torch.cuda.synchronize()
        ref = orc.fmm(pos, mass, 4, 0.6, 1)
        check_structure(plan, ref)
        check_values(phi.cpu().numpy(), acc.cpu().numpy(), ref, "f64")
        counts.append(plan.stats()["n_nodes"])
    # the pairs' tree outgrows the room the first build left (n + n/8 + 1024)
    assert counts[1] > counts[0] + counts[0] // 8 + 1024, counts
    plan.close()


@pytest.mark.parametrize("n,dist,dt", [(131072, "clustered", "f64"), (131073, "clustered", "f32"),
                                         (131072, "uniform", "f32")])
def test_particle_sort_paths(orc, n, dist, dt):
    """The particle sort places each digit in one launch (look-back over the
    tiles) up to 2^17 keys and in three launches (histograms, scan, scatter)
    above: keys, permutation, tree and lists against the oracle at both
    sides of the threshold, twice on one plan (the second sort's status words
    meet the first's)."""
    say(f"  sort paths {dist} n={n} {dt}")
    pos, mass = inputs(dist, n, 61, dt)
    plan, _, _ = gpu_run(pos, mass, 4, 0.7, 32, dt)
    ref = orc.fmm(pos, mass, 4, 0.7, 32, numeric=False)
    check_structure(plan, ref)
    torch = _torch()
    tdt = torch.float64 if dt == "f64" else torch.float32
    dev = torch.device("cuda:0")
    plan.build(torch.from_numpy(pos).to(dev, tdt), torch.from_numpy(mass).to(dev, tdt))
    torch.cuda.synchronize()
    check_structure(plan, ref)
    plan.close()


@pytest.mark.parametrize("name", ["plummer_1e5", "uniform_1e5", "hernquist_1e5"])
def test_parity_1e5(orc, name):
    c = W.CONFIGS[name]
    say(f"  case {name}")
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    plan, phi, acc = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"])
    check_structure(plan, ref)
    check_values(phi, acc, ref, c["dtype"], no_floor=True)
    plan.close()


@pytest.mark.timeout(300)
def test_parity_headline_full(orc):
    """The benchmarked workload (10^6 clustered, fp64, order 4, theta 0.7, leaf
    32) against the full oracle: every key, node, list entry and particle."""
    c = W.CONFIGS["clustered_1e6_p4"]
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    plan, phi, acc = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    say("  oracle (full)")
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"])
    check_structure(plan, ref)
    check_values(phi, acc, ref, c["dtype"], no_floor=True)
    plan.close()


@pytest.mark.timeout(400)
@pytest.mark.parametrize("name,n_sample", [("clustered_1e6_f32", 512), ("clustered_1e6_p6", 128)])
def test_parity_1e6_sampled(orc, name, n_sample):
    """Full-size workloads: complete structure check, values on a seeded sample
    of particles (the oracle computes their leaves' exact lists and expansions)."""
    c = W.CONFIGS[name]
    say(f"  case {name}")
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    plan, phi, acc = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    full = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], numeric=False)
    check_structure(plan, full)
    del full
    smp = np.random.default_rng(77).choice(c["n"], n_sample, replace=False)
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], sample=smp)
    check_values(phi, acc, ref, c["dtype"], idx=smp, no_floor=True)
    plan.close()


def test_deterministic_and_reusable(orc):
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    pos, mass = W.make("clustered", 50000, 51)
    plan = Plan(50000, order=4, theta=0.7, leaf_size=32, dtype=torch.float64, device=dev)
    tp, tm = torch.from_numpy(pos).to(dev), torch.from_numpy(mass).to(dev)
    plan.build(tp, tm)
    p1, a1 = plan.eval()
    p2, a2 = plan.eval()
    plan.build(tp, tm)
    p3, a3 = plan.eval()
    assert torch.equal(p1, p2) and torch.equal(a1, a2)
    assert torch.equal(p1, p3) and torch.equal(a1, a3)
    # a different particle set through the same plan (workspace regrowth)
    pos2, mass2 = W.make("plummer", 50000, 52)
    plan.build(torch.from_numpy(pos2).to(dev), torch.from_numpy(mass2).to(dev))
    p4, a4 = plan.eval()
    ref = orc.fmm(pos2, mass2, 4, 0.7, 32)
    check_structure(plan, ref)
    check_values(p4.cpu().numpy(), a4.cpu().numpy(), ref, "f64")
    plan.close()


@pytest.mark.parametrize("hint", [0, 3])
def test_walk_pool_regrowth(orc, hint):
    """Walk pools started far too small (hint entries per node) overflow, are
    regrown from the measured use and the walk repeated: the lists, the tree
    and the values are those of the oracle all the same, and a later build
    with the automatic size needs no repeat."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    pos, mass = W.make("clustered", 40000, 55)
    plan = Plan(40000, order=4, theta=0.6, leaf_size=16, dtype=torch.float64, device=dev)
    plan.set_walk_pool_hint(hint)
    tp, tm = torch.from_numpy(pos).to(dev), torch.from_numpy(mass).to(dev)
    plan.build(tp, tm)
    phi, acc = plan.eval()
    torch.cuda.synchronize()
    retries = plan.stats()["walk_retries"]
    say(f"    walk repeats {retries}")
    assert retries > 0
    ref = orc.fmm(pos, mass, 4, 0.6, 16)
    check_structure(plan, ref)
    check_values(phi.cpu().numpy(), acc.cpu().numpy(), ref, "f64")
    plan.set_walk_pool_hint(-1)
    plan.build(tp, tm)
    phi2, acc2 = plan.eval()
    torch.cuda.synchronize()
    assert plan.stats()["walk_retries"] == 0
    assert torch.equal(phi, phi2) and torch.equal(acc, acc2)
    plan.close()


def test_nonfinite_input_rejected():
    torch = _torch()
    from multipole_body_gravity_amd import FmmError, Plan
    dev = torch.device("cuda:0")
    pos = torch.rand(1000, 3, dtype=torch.float64, device=dev)
    mass = torch.ones(1000, dtype=torch.float64, device=dev)
    pos[17, 2] = float("nan")
    plan = Plan(1000, dtype=torch.float64, device=dev)
    with pytest.raises(FmmError) as ei:
        plan.build(pos, mass)
    assert ei.value.code == -5
    with pytest.raises(FmmError) as ei:
        plan.eval()
    assert ei.value.code == -2
    pos[17, 2] = 0.5
    mass[3] = float("inf")
    with pytest.raises(FmmError) as ei:
        plan.build(pos, mass)
    assert ei.value.code == -5
    mass[3] = 1.0
    plan.build(pos, mass)
    p1, a1 = plan.eval()
    # again with a plan that has room from a good build: the tree's second
    # phase is queued before the check and runs on the rejected set's keys
    pos[17, 2] = float("nan")
    with pytest.raises(FmmError) as ei:
        plan.build(pos, mass)
    assert ei.value.code == -5
    pos[17, 2] = 0.5
    plan.build(pos, mass)
    p2, a2 = plan.eval()
    assert torch.equal(p1, p2) and torch.equal(a1, a2)
    plan.close()


@pytest.mark.parametrize("order", [5, 6, 7, 10])
def test_expansions_match_oracle(orc, order):
    """Moments and locals of every cell (after the downward pass): orders 5
    and 6 take the one-launch downward pass (internal locals rebuilt on a
    copy), orders 7 and 10 the level-by-level one (order 10 with the
    wave-per-node upward and downward kernels)."""
    pos, mass = W.make("plummer", 4000, 61)
    plan, phi, acc = gpu_run(pos, mass, order, 0.6, 16, "f64")
    mp, lc = plan.copy_expansions()
    ref = orc.fmm(pos, mass, order, 0.6, 16, expansions=True)
    scale_m = np.abs(ref.mpole).max(axis=1, keepdims=True)
    assert np.max(np.abs(mp - ref.mpole) / scale_m) < 1e-12
    scale_l = np.abs(ref.local).max(axis=1, keepdims=True) + 1e-300
    assert np.max(np.abs(lc - ref.local) / scale_l) < 1e-11
    plan.close()


def golden_level_totals(name):
    """Per-level totals of the oracle's list digests for a lattice workload
    (tests/golden/lattice_256_digests.txt, written by make_lattice_digests.py)."""
    import os
    rows = {}
    path = os.path.join(os.path.dirname(__file__), "golden", "lattice_256_digests.txt")
    for ln in open(path):
        if ln.startswith("#") or not ln.strip():
            continue
        w, lv, nt, mc, mh, pc, ph = ln.split()
        if w == name:
            rows[int(lv)] = (int(nt), int(mc), int(mh, 16), int(pc), int(ph, 16))
    return rows


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["lattice_256_f32", "lattice_256_p8"])
def test_parity_lattice_full_lists(orc, name):
    """256^3 displaced lattice (fp32 order 4 theta 0.7 leaf 64; fp64 order 8
    theta 0.5 leaf 64), in the launch configuration the benchmark uses: keys,
    permutation and tree in full; every target's M2L and P2P lists through
    their digests (entry count and order-independent source hash, formed here
    from the GPU's copied lists and by the oracle's digest-mode walk), target
    by target, and their per-level totals against the stored ones; values at
    256 seeded particles."""
    from listdigest import csr_digests
    c = W.CONFIGS[name]
    say(f"  case {name}: generating")
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    say("  gpu")
    plan, phi, acc = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    say("  oracle digest walk")
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], digests="walk")
    keys, perm = plan.copy_keys()
    assert np.array_equal(keys, ref.keys) and np.array_equal(perm, ref.perm)
    tree = plan.copy_tree()
    for f in ("level", "prefix", "begin", "count", "parent", "first_child", "n_child"):
        assert np.array_equal(tree[f], getattr(ref, f)), f"tree field {f} differs"
    say("  gpu lists -> digests")
    lists = plan.copy_lists()
    st = plan.stats()
    assert st["n_m2l"] == ref.n_m2l and st["n_p2p"] == ref.n_p2p
    gold = golden_level_totals(name)
    level = tree["level"]
    for kind in ("m2l", "p2p"):
        cnt, h = csr_digests(lists[kind + "_off"], lists[kind + "_src"])
        assert np.array_equal(cnt, ref.digests[kind + "_cnt"]), f"{kind} entry counts differ"
        bad = np.nonzero(h != ref.digests[kind + "_hash"])[0]
        assert bad.size == 0, f"{kind} lists of {bad.size} targets differ (first {bad[:5]})"
        col = 1 if kind == "m2l" else 3
        with np.errstate(over="ignore"):
            for lv, row in gold.items():
                sel = level == lv
                assert int(sel.sum()) == row[0], (kind, lv)
                assert int(cnt[sel].sum(dtype=np.uint64)) == row[col], (kind, lv)
                assert int(h[sel].sum(dtype=np.uint64)) == row[col + 1], (kind, lv)
        assert set(gold) == set(range(int(level.max()) + 1))
    del lists, ref
    smp = np.random.default_rng(78).choice(c["n"], 256, replace=False)
    say("  oracle (sampled values)")
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], sample=smp)
    check_values(phi, acc, ref, c["dtype"], idx=smp, no_floor=True)
    plan.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_sample", [("hernquist_4e7", 64)])
def test_parity_large_sampled(orc, name, n_sample):
    """The 4e7-particle Hernquist sphere of the accuracy-runtime sweep: keys,
    permutation and tree in full; lists and values for the leaves of a seeded
    particle sample (the oracle's walk is restricted to those targets)."""
    c = W.CONFIGS[name]
    say(f"  case {name}: generating")
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    say("  gpu")
    plan, phi, acc = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    smp = np.random.default_rng(78).choice(c["n"], n_sample, replace=False)
    say("  oracle (sampled)")
    ref = orc.fmm(pos, mass, c["order"], c["theta"], c["leaf"], sample=smp)
    check_structure(plan, ref, sample_targets=np.nonzero(ref.mark)[0])
    check_values(phi, acc, ref, c["dtype"], idx=smp)
    plan.close()


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_direct_matches_oracle(orc, dt):
    """fmm_direct (the accuracy reference) against the oracle's direct sum on
    the same values, targets including the first and last particle."""
    torch = _torch()
    from multipole_body_gravity_amd import direct
    pos, mass = inputs("plummer", 20000, 81, dt)
    tdt = torch.float64 if dt == "f64" else torch.float32
    dev = torch.device("cuda:0")
    tg = np.concatenate([[0, 19999], np.random.default_rng(5).choice(20000, 700, replace=False)])
    phi, acc = direct(torch.from_numpy(pos).to(dev, tdt), torch.from_numpy(mass).to(dev, tdt),
                      torch.from_numpy(tg).to(dev))
    rphi, racc = orc.direct(pos, mass, tg)
    ea, _ = rel_err(acc.double().cpu().numpy(), racc)
    ep, _ = rel_err(phi.double().cpu().numpy(), rphi)
    tol = 1e-12 if dt == "f64" else 2e-7  # fp64 sums; fp32 only in the output
    assert ea.max() <= tol and ep.max() <= tol, (ea.max(), ep.max())


# --------------------------------------------------------------------------
# VJP (fmm_vjp) against the oracle's fast multipole VJP on the same tree and
# lists: dS/dpos and dS/dmass per particle, same tolerances as the forward
# --------------------------------------------------------------------------

def sensitivities(n, seed, dt):
    rng = np.random.default_rng(seed)
    pb = rng.standard_normal(n)
    ab = rng.standard_normal((n, 3))
    if dt == "f32":  # the oracle sees exactly the values the GPU gets
        pb = pb.astype(np.float32).astype(np.float64)
        ab = ab.astype(np.float32).astype(np.float64)
    return pb, ab


def gpu_vjp(plan, pb, ab, dt):
    torch = _torch()
    tdt = torch.float64 if dt == "f64" else torch.float32
    dev = torch.device("cuda:0")
    xb, mb = plan.vjp(torch.from_numpy(pb).to(dev, tdt), torch.from_numpy(ab).to(dev, tdt))
    torch.cuda.synchronize()
    return xb.double().cpu().numpy(), mb.double().cpu().numpy()


def abs_scales(pos, mass, pb, ab, idx):
    """Per target, the sums of the absolute values of the pair terms of
    dS/dmass (|pb_j|/r + |ab_j . r|/r^3) and of dS/dpos (|s|/r^2 + 4 |w|/r^3,
    s = pb_i m_j + m_i pb_j, w = m_i ab_j - m_j ab_i), by brute force."""
    am = np.zeros(idx.size)
    ax = np.zeros(idx.size)
    step = max(1, int(2e7 // pos.shape[0]))
    for c0 in range(0, idx.size, step):
        t = idx[c0:c0 + step]
        d = pos[t, None, :] - pos[None, :, :]
        r = np.sqrt((d ** 2).sum(-1))
        r[np.arange(t.size), t] = np.inf  # self term omitted
        am[c0:c0 + step] = (np.abs(pb)[None, :] / r + np.abs((ab[None] * d).sum(-1)) / r ** 3).sum(1)
        sabs = np.abs(pb[t, None] * mass[None, :] + mass[t, None] * pb[None, :])
        w = mass[t, None, None] * ab[None] - mass[None, :, None] * ab[t, None, :]
        ax[c0:c0 + step] = (sabs / r ** 2 + 4.0 * np.linalg.norm(w, axis=-1) / r ** 3).sum(1)
    return ax, am


def check_vjp(xb, mb, rx, rm, dt, idx=None, inputs=None):
    """The sensitivities have both signs, so dS/dmass and dS/dpos are sums with
    cancellation: their rounding error scales with the sum of the absolute pair
    terms A_i >= |result_i|, not with the result.  The bar is the forward's
    tolerance relative to A_i (which is the plain relative error where the
    terms do not cancel); A_i is formed, by brute force, only for the
    particles whose plain relative error is above the bar."""
    if idx is None:
        idx = np.arange(mb.shape[0])
    tol = TOL[dt]
    dx = np.linalg.norm(xb[idx] - rx[idx], axis=-1)
    dm = np.abs(mb[idx] - rm[idx])
    ex = dx / np.linalg.norm(rx[idx], axis=-1)
    em = dm / np.abs(rm[idx])
    bad = ~((ex <= tol) & (em <= tol))
    say(f"    max rel err pos_bar {ex.max():.3g} mass_bar {em.max():.3g}; {int(bad.sum())} above {tol:g}")
    if bad.any():
        pos, mass, pb, ab = inputs
        ax, am = abs_scales(pos, mass, pb, ab, idx[bad])
        ex_a, em_a = dx[bad] / ax, dm[bad] / am
        say(f"    of those, max err / sum|terms| pos_bar {ex_a.max():.3g} mass_bar {em_a.max():.3g}")
        assert ex_a.max() <= tol, f"pos_bar err {ex_a.max():.3g}"
        assert em_a.max() <= tol, f"mass_bar err {em_a.max():.3g}"


VJP_CASES = [
    # dist, n, seed, order, theta, leaf, dtype
    ("uniform", 4096, 1001, 4, 0.7, 32, "f64"),
    ("plummer", 10000, 1002, 5, 0.7, 32, "f64"),
    ("clustered", 20000, 31, 4, 0.7, 32, "f32"),
    ("plummer", 6000, 32, 6, 0.5, 16, "f64"),
    ("uniform", 1037, 33, 3, 0.6, 7, "f64"),
    ("plummer", 777, 34, 2, 0.4, 1, "f64"),
    ("uniform", 3000, 36, 0, 0.7, 20, "f64"),
    ("plummer", 3000, 37, 8, 0.5, 40, "f64"),
    ("plummer", 3000, 37, 8, 0.5, 40, "f32"),
    ("clustered", 3000, 42, 10, 0.6, 24, "f64"),
]


@pytest.mark.parametrize("dist,n,seed,order,theta,leaf,dt", VJP_CASES)
def test_vjp_parity(orc, dist, n, seed, order, theta, leaf, dt):
    say(f"  vjp case {dist} n={n} p={order} theta={theta} leaf={leaf} {dt}")
    pos, mass = inputs(dist, n, seed, dt)
    pb, ab = sensitivities(n, seed + 100, dt)
    plan, _, _ = gpu_run(pos, mass, order, theta, leaf, dt)
    xb, mb = gpu_vjp(plan, pb, ab, dt)
    rx, rm = orc.fmm_vjp(pos, mass, pb, ab, order, theta, leaf)
    check_vjp(xb, mb, rx, rm, dt, inputs=(pos, mass, pb, ab))
    plan.close()


def test_vjp_repeatable(orc):
    """A VJP right after the build (no eval) equals one after an eval bit for
    bit, a repeated VJP too, and an eval after a VJP still gives the forward's
    results bit for bit."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    pos, mass = W.make("clustered", 30000, 91)
    pb, ab = sensitivities(30000, 92, "f64")
    tp, tm = torch.from_numpy(pos).to(dev), torch.from_numpy(mass).to(dev)
    tpb, tab = torch.from_numpy(pb).to(dev), torch.from_numpy(ab).to(dev)
    plan = Plan(30000, order=4, theta=0.6, leaf_size=24, dtype=torch.float64, device=dev)
    plan.build(tp, tm)
    x0, m0 = (t.clone() for t in plan.vjp(tpb, tab))
    phi1, acc1 = (t.clone() for t in plan.eval())
    x1, m1 = (t.clone() for t in plan.vjp(tpb, tab))
    x2, m2 = plan.vjp(tpb, tab)
    phi2, acc2 = plan.eval()
    torch.cuda.synchronize()
    assert torch.equal(x0, x1) and torch.equal(m0, m1)
    assert torch.equal(x1, x2) and torch.equal(m1, m2)
    assert torch.equal(phi1, phi2) and torch.equal(acc1, acc2)
    rx, rm = orc.fmm_vjp(pos, mass, pb, ab, 4, 0.6, 24)
    check_vjp(x2.cpu().numpy(), m2.cpu().numpy(), rx, rm, "f64", inputs=(pos, mass, pb, ab))
    plan.close()


@pytest.mark.timeout(300)
def test_vjp_parity_1e5(orc):
    c = W.CONFIGS["plummer_1e5"]
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    pb, ab = sensitivities(c["n"], 93, c["dtype"])
    plan, _, _ = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    xb, mb = gpu_vjp(plan, pb, ab, c["dtype"])
    rx, rm = orc.fmm_vjp(pos, mass, pb, ab, c["order"], c["theta"], c["leaf"])
    check_vjp(xb, mb, rx, rm, c["dtype"], inputs=(pos, mass, pb, ab))
    plan.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,n_sample", [("clustered_1e6_p4", 256), ("clustered_1e6_f32", 256)])
def test_vjp_1e6_sampled(orc, name, n_sample):
    """The VJP at the 10^6-particle clustered workload, in the launch
    configuration the benchmark times, on the leaves of a seeded sample."""
    c = W.CONFIGS[name]
    pos, mass = inputs(c["dist"], c["n"], c["seed"], c["dtype"])
    pb, ab = sensitivities(c["n"], 94, c["dtype"])
    plan, _, _ = gpu_run(pos, mass, c["order"], c["theta"], c["leaf"], c["dtype"])
    xb, mb = gpu_vjp(plan, pb, ab, c["dtype"])
    smp = np.random.default_rng(95).choice(c["n"], n_sample, replace=False)
    rx, rm = orc.fmm_vjp(pos, mass, pb, ab, c["order"], c["theta"], c["leaf"], sample=smp)
    check_vjp(xb, mb, rx, rm, c["dtype"], idx=smp, inputs=(pos, mass, pb, ab))
    plan.close()


@pytest.mark.parametrize("kind", ["single", "two_body", "all_near", "order0"])
def test_vjp_degenerate(orc, kind):
    """One particle (no sensitivity reaches anything), two bodies, a single
    leaf holding everything (all pairs direct: equal to the exact chain-rule
    gradient of the direct sum) and order 0."""
    pos, mass = W.make("plummer", 3000, 96)
    order, theta, leaf = 4, 0.7, 32
    if kind == "single":
        pos, mass = pos[:1], mass[:1]
    elif kind == "two_body":
        pos, mass = pos[:2], mass[:2]
    elif kind == "all_near":
        pos, mass, leaf = pos[:700], mass[:700], 700
    else:
        order = 0
    n = pos.shape[0]
    pb, ab = sensitivities(n, 97, "f64")
    plan, _, _ = gpu_run(pos, mass, order, theta, leaf, "f64")
    xb, mb = gpu_vjp(plan, pb, ab, "f64")
    plan.close()
    if kind == "single":
        assert np.all(xb == 0.0) and np.all(mb == 0.0)
        return
    rx, rm = orc.fmm_vjp(pos, mass, pb, ab, order, theta, leaf)
    check_vjp(xb, mb, rx, rm, "f64", inputs=(pos, mass, pb, ab))
    if kind in ("two_body", "all_near"):
        dx, dm = orc.direct_vjp(pos, mass, pb, ab)
        assert np.abs(xb - dx).max() <= 1e-12 * np.abs(dx).max()
        assert np.abs(mb - dm).max() <= 1e-12 * np.abs(dm).max()


def test_vjp_matches_forward_differences():
    """The VJP against central differences of the GPU's own forward
    evaluation, S = sum pb.phi + ab.a: masses (S is linear in each, so the
    difference is exact up to rounding) and positions of particles whose keys
    and lists do not change under the step.  At order 8, theta 0.3 the two
    differ only by the expansions' truncation."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    n, order, theta, leaf = 2000, 8, 0.3, 16
    pos, mass = W.make("plummer", n, 98)
    pb, ab = sensitivities(n, 99, "f64")
    plan = Plan(n, order=order, theta=theta, leaf_size=leaf, dtype=torch.float64, device=dev)
    tpb, tab = torch.from_numpy(pb).to(dev), torch.from_numpy(ab).to(dev)

    def S(p, m):
        plan.build(torch.from_numpy(p).to(dev), torch.from_numpy(m).to(dev))
        phi, acc = plan.eval()
        torch.cuda.synchronize()
        return float((tpb * phi).sum() + (tab * acc).sum())

    S(pos, mass)
    keys0, _ = plan.copy_keys()
    lists0 = plan.copy_lists()
    xb, mb = plan.vjp(tpb, tab)
    xb, mb = xb.cpu().numpy(), mb.cpu().numpy()
    gscale = np.abs(xb).max()
    for i in (3, 500, 1999):
        h = 1e-3 * mass[i]
        mp, mm = mass.copy(), mass.copy()
        mp[i] += h
        mm[i] -= h
        fd = (S(pos, mp) - S(pos, mm)) / (2 * h)
        assert abs(fd - mb[i]) <= 1e-6 * np.abs(mb).max(), (i, fd, mb[i])
    checked = 0
    for i in range(0, n, 97):
        for a in range(3):
            h = 1e-7
            pp, pm = pos.copy(), pos.copy()
            pp[i, a] += h
            pm[i, a] -= h
            sp = S(pp, mass)
            same = np.array_equal(plan.copy_keys()[0], keys0) and \
                np.array_equal(plan.copy_lists()["p2p_src"], lists0["p2p_src"])
            sm = S(pm, mass)
            same = same and np.array_equal(plan.copy_keys()[0], keys0) and \
                np.array_equal(plan.copy_lists()["p2p_src"], lists0["p2p_src"])
            if not same:
                continue
            fd = (sp - sm) / (2 * h)
            assert abs(fd - xb[i, a]) <= 1e-5 * gscale, (i, a, fd, xb[i, a])
            checked += 1
        if checked >= 12:
            break
    assert checked >= 6
    plan.close()


def test_vjp_rejects_bad_arguments():
    torch = _torch()
    from multipole_body_gravity_amd import FmmError, Plan
    dev = torch.device("cuda:0")
    plan = Plan(100, order=3, dtype=torch.float64, device=dev)
    pb = torch.zeros(100, dtype=torch.float64, device=dev)
    ab = torch.zeros(100, 3, dtype=torch.float64, device=dev)
    with pytest.raises(FmmError) as e:  # not built
        plan.vjp(pb, ab)
    assert e.value.code == -2
    with pytest.raises(FmmError):
        plan.vjp(pb[:50], ab)
    with pytest.raises(FmmError):
        plan.vjp(pb.float(), ab)
    plan.close()


# --------------------------------------------------------------------------
# reversible integer-lattice steps (fmm_lattice_steps)
# --------------------------------------------------------------------------

def gpu_lattice(plan, q, u, mass, dt, n_steps, direction, tdt, dv=W.LATTICE_DV):
    torch = _torch()
    dev = torch.device("cuda:0")
    tq = torch.from_numpy(q).to(dev)
    tu = torch.from_numpy(u).to(dev)
    plan.lattice_steps(tq, tu, torch.from_numpy(mass).to(dev, tdt), W.LATTICE_DX, dv,
                       dt, n_steps, direction)
    torch.cuda.synchronize()
    return tq.cpu().numpy(), tu.cpu().numpy()


@pytest.mark.parametrize("dist,n,seed,order,theta,leaf", [
    ("plummer", 4096, 201, 4, 0.7, 32), ("clustered", 10000, 202, 5, 0.6, 16),
    ("uniform", 777, 203, 2, 0.5, 3)])
def test_lattice_parity(orc, dist, n, seed, order, theta, leaf):
    """Three steps from the same integer state give the same integers as the
    oracle.  The drift is exact.  A kick rounds a * dt/2 / dv, and the two
    accelerations agree only to the evaluation's tolerance (1e-11), so a kick
    whose quantity lies within 1e-11 |a dt/2/dv| of a rounding boundary could
    go either way: the velocity lattice here is dv = 2^-16 (kicks of tens of
    units, rather than the 2^-32 of the reversibility runs, where a kick of
    ~10^9 units is uncertain in its last digit), and the test checks that no
    kick of the seeded cases comes within 1e-10 (relative) of a boundary, so
    every integer must agree."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    pos, mass = W.make(dist, n, seed)
    dv = 2.0 ** -16
    q0, u0 = W.lattice_state(pos, seed + 1, dv=dv)
    dt = 1e-3
    plan = Plan(n, order=order, theta=theta, leaf_size=leaf, dtype=torch.float64,
                device=torch.device("cuda:0"))
    qg, ug = gpu_lattice(plan, q0, u0, mass, dt, 3, +1, torch.float64, dv=dv)
    qr, ur, margin = orc.lattice_steps(q0, u0, mass, W.LATTICE_DX, dv, dt, 3, +1,
                                       order, theta, leaf)
    say(f"    smallest rounding margin {margin:.3g}")
    assert margin > 1e-10
    assert np.array_equal(qg, qr) and np.array_equal(ug, ur)
    plan.close()


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name,steps", [("clustered_1e6_p4", 4), ("clustered_1e6_f32", 4),
                                        ("plummer_1e5", 10)])
def test_lattice_reversible(name, steps):
    """Forward steps then as many backward steps return the exact initial
    integer state, at the benchmark's workload in fp64 and fp32."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    c = W.CONFIGS[name]
    pos, mass = W.make(c["dist"], c["n"], c["seed"])
    q0, u0 = W.lattice_state(pos, 301)
    tdt = torch.float64 if c["dtype"] == "f64" else torch.float32
    plan = Plan(c["n"], order=c["order"], theta=c["theta"], leaf_size=c["leaf"], dtype=tdt,
                device=torch.device("cuda:0"))
    q1, u1 = gpu_lattice(plan, q0, u0, mass, 1e-3, steps, +1, tdt)
    assert (q1 != q0).mean() > 0.9 and (u1 != u0).mean() > 0.9
    q2, u2 = gpu_lattice(plan, q1, u1, mass, 1e-3, steps, -1, tdt)
    assert np.array_equal(q2, q0) and np.array_equal(u2, u0)
    plan.close()


def test_lattice_edge_cases(orc):
    """No steps leaves the state alone; a lone particle drifts by exactly
    round(u dt dv / dx) per step (as the oracle); a bad direction is an
    argument error."""
    torch = _torch()
    from multipole_body_gravity_amd import FmmError, Plan
    dev = torch.device("cuda:0")
    pos, mass = W.make("uniform", 500, 206)
    q0, u0 = W.lattice_state(pos, 207)
    plan = Plan(500, order=3, theta=0.7, leaf_size=16, dtype=torch.float64, device=dev)
    q, u = gpu_lattice(plan, q0, u0, mass, 1e-3, 0, +1, torch.float64)
    assert np.array_equal(q, q0) and np.array_equal(u, u0)
    with pytest.raises(FmmError) as e:
        gpu_lattice(plan, q0, u0, mass, 1e-3, 1, 0, torch.float64)
    assert e.value.code == -1
    plan.close()
    one = Plan(1, order=4, dtype=torch.float64, device=dev)
    q1, u1 = gpu_lattice(one, q0[:1], u0[:1], mass[:1], 0.37, 3, +1, torch.float64)
    qr, ur, _ = orc.lattice_steps(q0[:1], u0[:1], mass[:1], W.LATTICE_DX, W.LATTICE_DV, 0.37, 3, +1)
    assert np.array_equal(q1, qr) and np.array_equal(u1, ur) and np.array_equal(u1, u0[:1])
    one.close()


def test_lattice_overflow_reported():
    """An increment beyond 2^62 (here a huge time step) is an error, not a wrap."""
    torch = _torch()
    from multipole_body_gravity_amd import FmmError, Plan
    pos, mass = W.make("plummer", 2000, 204)
    q0, u0 = W.lattice_state(pos, 205)
    plan = Plan(2000, order=3, theta=0.7, leaf_size=16, dtype=torch.float64,
                device=torch.device("cuda:0"))
    with pytest.raises(FmmError) as e:
        gpu_lattice(plan, q0, u0, mass, 1e12, 1, +1, torch.float64)
    assert e.value.code == -5
    plan.close()


def test_streams_and_timing(orc):
    """Build on one stream and evaluate (and VJP) on another, with no ordering
    between the caller's streams: the library orders each call of a plan after
    the previous one itself.  Steps alternate between two particle sets, so a
    build that overtook the previous eval would change the lists and tasks that
    eval reads; every step's outputs are checked.  With timing on, every stage
    and kernel is counted once per step and the means are positive."""
    torch = _torch()
    from multipole_body_gravity_amd import Plan
    dev = torch.device("cuda:0")
    sets = []
    for seed in (71, 73):
        pos, mass = W.make("plummer", 30000, seed)
        pb, ab = sensitivities(30000, seed + 1, "f64")
        ref = orc.fmm(pos, mass, 4, 0.7, 16)
        rx, rm = orc.fmm_vjp(pos, mass, pb, ab, 4, 0.7, 16)
        sets.append(dict(pos=pos, mass=mass, pb=pb, ab=ab, ref=ref, rx=rx, rm=rm,
                         tp=torch.from_numpy(pos).to(dev), tm=torch.from_numpy(mass).to(dev),
                         tpb=torch.from_numpy(pb).to(dev), tab=torch.from_numpy(ab).to(dev)))
    plan = Plan(30000, order=4, theta=0.7, leaf_size=16, dtype=torch.float64, device=dev)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())  # the inputs were copied on the default stream
    s2.wait_stream(torch.cuda.current_stream())
    plan.set_timing(True)
    steps = 4
    outs = []
    for k in range(steps):
        d = sets[k % 2]
        with torch.cuda.stream(s1):
            plan.build(d["tp"], d["tm"], stream=s1)
        with torch.cuda.stream(s2):
            phi = torch.empty(30000, dtype=torch.float64, device=dev)
            acc = torch.empty(30000, 3, dtype=torch.float64, device=dev)
            xb = torch.empty(30000, 3, dtype=torch.float64, device=dev)
            mb = torch.empty(30000, dtype=torch.float64, device=dev)
            plan.eval(phi, acc, stream=s2)
            plan.vjp(d["tpb"], d["tab"], xb, mb, stream=s2)
        outs.append((phi, acc, xb, mb))
    torch.cuda.synchronize()
    st = plan.stats()
    assert st["timed_builds"] == steps and st["timed_evals"] == steps, st
    assert st["timed_vjps"] == steps, st
    for k, v in st["stage_ms"].items():
        assert v >= 0.0, (k, st["stage_ms"])
    for k in ("keys", "sort", "tree", "walk", "up", "m2l", "down", "p2p", "vjp"):
        assert st["stage_ms"][k] > 0.0, (k, st["stage_ms"])
    for k in ("m2l_sib", "m2l_tail", "p2p", "vjp_m2l_sib", "vjp_p2p"):
        assert st["kernel_ms"][k] > 0.0, (k, st["kernel_ms"])
    for k, (phi, acc, xb, mb) in enumerate(outs):
        d = sets[k % 2]
        say(f"    step {k}")
        check_values(phi.cpu().numpy(), acc.cpu().numpy(), d["ref"], "f64")
        check_vjp(xb.cpu().numpy(), mb.cpu().numpy(), d["rx"], d["rm"], "f64",
                  inputs=(d["pos"], d["mass"], d["pb"], d["ab"]))
    # timing mode 2: the kernels and the VJP call only, no other stage events
    plan.set_timing(2)
    for k in range(2):
        d = sets[k % 2]
        plan.build(d["tp"], d["tm"])
        phi, acc = plan.eval()
        plan.vjp(d["tpb"], d["tab"], xb, mb)
    torch.cuda.synchronize()
    st = plan.stats()
    assert st["timed_builds"] == 2 and st["timed_evals"] == 2 and st["timed_vjps"] == 2, st
    for k, v in st["stage_ms"].items():
        assert (v > 0.0) if k == "vjp" else (v == 0.0), (k, st["stage_ms"])
    for k in ("m2l_sib", "m2l_tail", "p2p", "vjp_m2l_sib", "vjp_p2p"):
        assert st["kernel_ms"][k] > 0.0, (k, st["kernel_ms"])
    check_values(phi.double().cpu().numpy(), acc.double().cpu().numpy(), sets[1]["ref"], "f64")
    # timing mode 3: the near-field kernels and the VJP call only
    plan.set_timing(3)
    for k in range(2):
        d = sets[k % 2]
        plan.build(d["tp"], d["tm"])
        phi, acc = plan.eval()
        plan.vjp(d["tpb"], d["tab"], xb, mb)
    torch.cuda.synchronize()
    st = plan.stats()
    assert st["timed_builds"] == 2 and st["timed_evals"] == 2 and st["timed_vjps"] == 2, st
    for k, v in st["stage_ms"].items():
        assert (v > 0.0) if k == "vjp" else (v == 0.0), (k, st["stage_ms"])
    for k, v in st["kernel_ms"].items():
        assert (v > 0.0) if k in ("p2p", "vjp_p2p") else (k == "p2p_combine" or v == 0.0), \
            (k, st["kernel_ms"])
    check_values(phi.double().cpu().numpy(), acc.double().cpu().numpy(), sets[1]["ref"], "f64")
    with pytest.raises(RuntimeError):
        plan.set_timing(4)
    plan.close()
