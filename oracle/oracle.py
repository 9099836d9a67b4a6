"""ctypes wrapper of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark.  It never imports the product package and the
product package never imports it.  Everything here is argument marshalling; the
arithmetic lives in oracle.c (fp64, G = 1, no softening).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

ERR_ARG = -1
ERR_OOM = -3
ERR_NONFINITE = -5


SAN_LIB = os.path.join(HERE, "liboracle_san.so")
# ORACLE_SANITIZE=1: build and load the oracle with AddressSanitizer and
# UndefinedBehaviorSanitizer (CPU code only; python itself is not
# instrumented, so the run needs the ASan runtime preloaded:
#   ORACLE_SANITIZE=1 LD_PRELOAD=$(gcc -print-file-name=libasan.so) \
#   ASAN_OPTIONS=detect_leaks=0 python -m pytest tests/test_oracle.py)
SANITIZE = os.environ.get("ORACLE_SANITIZE", "0") == "1"


def build_library(sanitize: bool = False) -> str:
    """Compile oracle.c with gcc (no fused multiply-add, OpenMP over targets);
    sanitize: with -fsanitize=address,undefined (aborting on the first report)."""
    out = SAN_LIB if sanitize else LIB
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"] if sanitize else ["-O2"]
    cmd = ["gcc", *flags, "-std=c11", "-D_POSIX_C_SOURCE=200809L", "-fopenmp",
           "-ffp-contract=off", "-fPIC", "-shared", "-Wall", "-o", out + ".tmp", SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = SAN_LIB if SANITIZE else LIB
    if not os.path.exists(path) or os.path.getmtime(path) < os.path.getmtime(SRC):
        build_library(sanitize=SANITIZE)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.oracle_ncoef.argtypes = [i32]
    lib.oracle_set_threads.argtypes = [i32]
    lib.oracle_set_threads.restype = None
    lib.oracle_direct.argtypes = [i64, P, P, i64, P, P, P]
    lib.oracle_fmm.argtypes = [i64, P, P, i32, dbl, i32, i64, P, i32, ctypes.POINTER(P)]
    lib.oracle_free.argtypes = [P]
    lib.oracle_free.restype = None
    for name, nargs in [("oracle_sizes", 1), ("oracle_times", 1), ("oracle_copy_mark", 1)]:
        getattr(lib, name).argtypes = [P] * (nargs + 1)
        getattr(lib, name).restype = None
    lib.oracle_root.argtypes = [P, P, P]
    lib.oracle_root.restype = None
    lib.oracle_copy_keys.argtypes = [P, P, P]
    lib.oracle_copy_keys.restype = None
    lib.oracle_copy_tree.argtypes = [P] * 8
    lib.oracle_copy_tree.restype = None
    lib.oracle_copy_lists.argtypes = [P] * 5
    lib.oracle_copy_lists.restype = None
    lib.oracle_copy_digests.argtypes = [P] * 5
    lib.oracle_copy_expansions.argtypes = [P, P, P]
    lib.oracle_copy_expansions.restype = None
    lib.oracle_copy_result.argtypes = [P, P, P]
    lib.oracle_copy_result.restype = None
    lib.oracle_p2m.argtypes = [i32, i64, P, P, P, P]
    lib.oracle_m2m.argtypes = [i32, P, P, P]
    lib.oracle_dtensor.argtypes = [i32, P, P]
    lib.oracle_m2l.argtypes = [i32, P, P, P]
    lib.oracle_l2l.argtypes = [i32, P, P, P]
    lib.oracle_l2p.argtypes = [i32, P, P, P, P]
    lib.oracle_morton.argtypes = [i64, P, P, P, P]
    lib.oracle_direct_vjp.argtypes = [i64, P, P, P, P, P, P]
    lib.oracle_fmm_vjp.argtypes = [i64, P, P, i32, dbl, i32, i64, P, P, P, P, P]
    lib.oracle_p2m_dipole.argtypes = [i32, i64, P, P, P, P, P]
    lib.oracle_l2p_hessian.argtypes = [i32, P, P, P]
    lib.oracle_lattice_steps.argtypes = [i64, P, P, P, dbl, dbl, dbl, i32, i32, i32, dbl, i32, P]
    _lib = lib
    return lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _f64(a, shape=None) -> np.ndarray:
    a = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
    if shape is not None:
        a = a.reshape(shape)
    return a


class OracleError(RuntimeError):
    def __init__(self, code: int):
        super().__init__(f"oracle error {code}")
        self.code = code


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def ncoef(order: int) -> int:
    return int(_load().oracle_ncoef(order))


def multi_indices(order: int):
    """The coefficient layout of the copy-out calls: degree, then a, b descending."""
    out = []
    for d in range(order + 1):
        for a in range(d, -1, -1):
            for b in range(d - a, -1, -1):
                out.append((a, b, d - a - b))
    return out


def direct(pos, mass, targets=None):
    """O(N^2) direct sum (fp64).  Returns (phi[nt], acc[nt,3])."""
    lib = _load()
    pos = _f64(pos, (-1, 3))
    mass = _f64(mass)
    n = pos.shape[0]
    tg = np.arange(n, dtype=np.int64) if targets is None else np.ascontiguousarray(targets, dtype=np.int64)
    phi = np.zeros(tg.shape[0])
    acc = np.zeros((tg.shape[0], 3))
    rc = lib.oracle_direct(n, _p(pos), _p(mass), tg.shape[0], _p(tg), _p(phi), _p(acc))
    if rc:
        raise OracleError(rc)
    return phi, acc


@dataclass
class OracleResult:
    n: int
    order: int
    K: int
    lo: np.ndarray
    side: float
    keys: np.ndarray
    perm: np.ndarray
    level: np.ndarray
    prefix: np.ndarray
    begin: np.ndarray
    count: np.ndarray
    parent: np.ndarray
    first_child: np.ndarray
    n_child: np.ndarray
    mark: np.ndarray
    m2l_off: np.ndarray
    m2l_src: np.ndarray
    p2p_off: np.ndarray
    p2p_src: np.ndarray
    depth: int
    n_leaves: int
    times: np.ndarray
    mpole: np.ndarray | None = None
    local: np.ndarray | None = None
    phi: np.ndarray | None = None
    acc: np.ndarray | None = None
    # per target node: entry counts and order-independent source hashes of the
    # M2L and P2P lists (oracle_copy_digests)
    digests: dict | None = None
    n_m2l: int = 0
    n_p2p: int = 0


def fmm(pos, mass, order=4, theta=0.7, leaf_size=32, sample=None, numeric=True,
        expansions=False, digests=None) -> OracleResult:
    """Run the oracle FMM.  `sample` (particle indices) restricts the targets.

    digests: None, "lists" (also form every target's list digests from the
    stored lists) or "walk" (digest mode: the walk stores no lists, only the
    digests; no numeric passes, empty list arrays)."""
    lib = _load()
    pos = _f64(pos, (-1, 3))
    mass = _f64(mass)
    n = pos.shape[0]
    smp = np.zeros(0, dtype=np.int64) if sample is None else np.ascontiguousarray(sample, dtype=np.int64)
    if digests not in (None, "lists", "walk"):
        raise ValueError(digests)
    walk_digests = digests == "walk"
    if walk_digests:
        numeric = False
    h = ctypes.c_void_p()
    rc = lib.oracle_fmm(n, _p(pos), _p(mass), int(order), float(theta), int(leaf_size),
                        smp.shape[0], _p(smp) if smp.shape[0] else None,
                        (1 if numeric else 0) | (2 if walk_digests else 0), ctypes.byref(h))
    if rc:
        raise OracleError(rc)
    try:
        sizes = np.zeros(7, dtype=np.int64)
        lib.oracle_sizes(h, _p(sizes))
        nn, nl, depth, nm2l, np2p, _, K = (int(v) for v in sizes)
        lo = np.zeros(3)
        side = np.zeros(1)
        lib.oracle_root(h, _p(lo), _p(side))
        keys = np.zeros(n, dtype=np.uint64)
        perm = np.zeros(n, dtype=np.int32)
        lib.oracle_copy_keys(h, _p(keys), _p(perm))
        level = np.zeros(nn, dtype=np.uint8)
        prefix = np.zeros(nn, dtype=np.uint64)
        begin = np.zeros(nn, dtype=np.int32)
        count = np.zeros(nn, dtype=np.int32)
        parent = np.zeros(nn, dtype=np.int32)
        first_child = np.zeros(nn, dtype=np.int32)
        n_child = np.zeros(nn, dtype=np.uint8)
        lib.oracle_copy_tree(h, _p(level), _p(prefix), _p(begin), _p(count), _p(parent),
                             _p(first_child), _p(n_child))
        mark = np.zeros(nn, dtype=np.uint8)
        lib.oracle_copy_mark(h, _p(mark))
        if walk_digests:
            m2l_off = p2p_off = np.zeros(0, dtype=np.int64)
            m2l_src = p2p_src = np.zeros(0, dtype=np.int32)
        else:
            m2l_off = np.zeros(nn + 1, dtype=np.int64)
            p2p_off = np.zeros(nn + 1, dtype=np.int64)
            m2l_src = np.zeros(max(nm2l, 1), dtype=np.int32)
            p2p_src = np.zeros(max(np2p, 1), dtype=np.int32)
            lib.oracle_copy_lists(h, _p(m2l_off), _p(m2l_src), _p(p2p_off), _p(p2p_src))
        times = np.zeros(8)
        lib.oracle_times(h, _p(times))
        res = OracleResult(n, order, K, lo, float(side[0]), keys, perm, level, prefix, begin,
                           count, parent, first_child, n_child, mark.astype(bool), m2l_off,
                           m2l_src[:nm2l], p2p_off, p2p_src[:np2p], depth, nl, times,
                           n_m2l=nm2l, n_p2p=np2p)
        if digests is not None:
            d = {k: np.zeros(nn, dtype=np.uint64)
                 for k in ("m2l_cnt", "m2l_hash", "p2p_cnt", "p2p_hash")}
            rc = lib.oracle_copy_digests(h, _p(d["m2l_cnt"]), _p(d["m2l_hash"]),
                                         _p(d["p2p_cnt"]), _p(d["p2p_hash"]))
            if rc:
                raise OracleError(rc)
            res.digests = d
        if numeric:
            res.phi = np.zeros(n)
            res.acc = np.zeros((n, 3))
            lib.oracle_copy_result(h, _p(res.phi), _p(res.acc))
            if expansions:
                res.mpole = np.zeros((nn, K))
                res.local = np.zeros((nn, K))
                lib.oracle_copy_expansions(h, _p(res.mpole), _p(res.local))
        return res
    finally:
        lib.oracle_free(h)


# ---- single operators (for pinning each step) ----------------------------

def morton(pos):
    lib = _load()
    pos = _f64(pos, (-1, 3))
    lo = np.zeros(3)
    side = np.zeros(1)
    keys = np.zeros(pos.shape[0], dtype=np.uint64)
    rc = lib.oracle_morton(pos.shape[0], _p(pos), _p(lo), _p(side), _p(keys))
    if rc:
        raise OracleError(rc)
    return lo, float(side[0]), keys


def p2m(order, pos, mass, centre):
    lib = _load()
    pos = _f64(pos, (-1, 3))
    mass = _f64(mass)
    c = _f64(centre)
    out = np.zeros(ncoef(order))
    rc = lib.oracle_p2m(order, pos.shape[0], _p(pos), _p(mass), _p(c), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def m2m(order, mpole_child, d, accum=None):
    lib = _load()
    out = np.zeros(ncoef(order)) if accum is None else _f64(accum).copy()
    rc = lib.oracle_m2m(order, _p(_f64(mpole_child)), _p(_f64(d)), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def dtensor(order, r):
    lib = _load()
    out = np.zeros(ncoef(order))
    rc = lib.oracle_dtensor(order, _p(_f64(r)), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def m2l(order, mpole, r, accum=None):
    lib = _load()
    out = np.zeros(ncoef(order)) if accum is None else _f64(accum).copy()
    rc = lib.oracle_m2l(order, _p(_f64(mpole)), _p(_f64(r)), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def l2l(order, local_parent, d, accum=None):
    lib = _load()
    out = np.zeros(ncoef(order)) if accum is None else _f64(accum).copy()
    rc = lib.oracle_l2l(order, _p(_f64(local_parent)), _p(_f64(d)), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def l2p(order, local, delta):
    lib = _load()
    phi = np.zeros(1)
    acc = np.zeros(3)
    rc = lib.oracle_l2p(order, _p(_f64(local)), _p(_f64(delta)), _p(phi), _p(acc))
    if rc:
        raise OracleError(rc)
    return float(phi[0]), acc


# ---- vector-Jacobian products ----------------------------------------------

def direct_vjp(pos, mass, phi_bar, acc_bar):
    """Exact gradient of S = sum pb.phi + ab.a of the direct sum: (xbar[n,3], mbar[n])."""
    lib = _load()
    pos = _f64(pos, (-1, 3))
    mass = _f64(mass)
    pb = _f64(phi_bar)
    ab = _f64(acc_bar, (-1, 3))
    n = pos.shape[0]
    xbar = np.zeros((n, 3))
    mbar = np.zeros(n)
    rc = lib.oracle_direct_vjp(n, _p(pos), _p(mass), _p(pb), _p(ab), _p(xbar), _p(mbar))
    if rc:
        raise OracleError(rc)
    return xbar, mbar


def fmm_vjp(pos, mass, phi_bar, acc_bar, order=4, theta=0.7, leaf_size=32, sample=None):
    """Fast multipole VJP on the oracle's own tree and lists: (xbar[n,3], mbar[n]).
    `sample` restricts the targets to the leaves holding those particles (NaN elsewhere)."""
    lib = _load()
    pos = _f64(pos, (-1, 3))
    mass = _f64(mass)
    pb = _f64(phi_bar)
    ab = _f64(acc_bar, (-1, 3))
    n = pos.shape[0]
    xbar = np.zeros((n, 3))
    mbar = np.zeros(n)
    smp = np.zeros(0, dtype=np.int64) if sample is None else np.ascontiguousarray(sample, dtype=np.int64)
    rc = lib.oracle_fmm_vjp(n, _p(pos), _p(mass), int(order), float(theta), int(leaf_size),
                            smp.shape[0], _p(smp) if smp.shape[0] else None,
                            _p(pb), _p(ab), _p(xbar), _p(mbar))
    if rc:
        raise OracleError(rc)
    return xbar, mbar


def p2m_dipole(order, pos, q, dip, centre):
    lib = _load()
    pos = _f64(pos, (-1, 3))
    out = np.zeros(ncoef(order))
    rc = lib.oracle_p2m_dipole(order, pos.shape[0], _p(pos), _p(_f64(q)), _p(_f64(dip, (-1, 3))),
                               _p(_f64(centre)), _p(out))
    if rc:
        raise OracleError(rc)
    return out


def l2p_hessian(order, local, delta):
    """Second derivatives of the local polynomial at delta, as a symmetric 3x3 matrix."""
    lib = _load()
    h = np.zeros(6)
    rc = lib.oracle_l2p_hessian(order, _p(_f64(local)), _p(_f64(delta)), _p(h))
    if rc:
        raise OracleError(rc)
    return np.array([[h[0], h[3], h[4]], [h[3], h[1], h[5]], [h[4], h[5], h[2]]])


# ---- reversible lattice integrator -------------------------------------------

def lattice_steps(q, u, mass, dx, dv, dt, n_steps, direction=1, order=4, theta=0.7, leaf_size=32):
    """Kick-drift-kick steps on the integer lattice: returns (q, u, min_margin)."""
    lib = _load()
    q = np.ascontiguousarray(q, dtype=np.int64).reshape(-1, 3).copy()
    u = np.ascontiguousarray(u, dtype=np.int64).reshape(-1, 3).copy()
    mass = _f64(mass)
    mm = np.zeros(1)
    rc = lib.oracle_lattice_steps(q.shape[0], _p(q), _p(u), _p(mass), float(dx), float(dv),
                                  float(dt), int(n_steps), int(direction), int(order),
                                  float(theta), int(leaf_size), _p(mm))
    if rc:
        raise OracleError(rc)
    return q, u, float(mm[0])
