"""Thin ctypes binding of libmbg_fmm.so (include/fmm.h).

Argument marshalling only: torch tensors supply device memory and the HIP
stream, every step of the computation runs in the library's HIP kernels.  There
is no CPU fallback: if the library or a GPU is missing, constructing a Plan
raises.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmbg_fmm.so")

FMM_F32, FMM_F64 = 0, 1
MAX_ORDER = 10
STAGES = ["keys", "sort", "tree", "walk", "up", "m2l", "down", "p2p", "tail", "vjp"]  # stage_ms order
KERNELS = ["m2l_sib", "m2l_tail", "p2p", "p2p_combine", "vjp_m2l_sib", "vjp_p2p", "p2m",
           "l2p"]  # kernel_ms order
_ERR = {0: "ok", -1: "invalid argument", -2: "plan not built", -3: "device out of memory",
        -4: "HIP runtime error", -5: "non-finite position or mass", -6: "no HIP device"}


class FmmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        super().__init__(f"{what}: {_ERR.get(code, 'unknown')} ({code})")
        self.code = code


class _Stats(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int64), ("n_nodes", ctypes.c_int64), ("n_leaves", ctypes.c_int64),
                ("n_m2l", ctypes.c_int64), ("n_p2p", ctypes.c_int64), ("depth", ctypes.c_int32),
                ("order", ctypes.c_int32), ("leaf_size", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("theta", ctypes.c_double), ("lo", ctypes.c_double * 3), ("side", ctypes.c_double),
                ("stage_ms", ctypes.c_float * len(STAGES)), ("walk_retries", ctypes.c_int32),
                ("kernel_ms", ctypes.c_float * len(KERNELS)), ("timed_builds", ctypes.c_int32),
                ("timed_evals", ctypes.c_int32), ("timed_vjps", ctypes.c_int32),
                ("walk_one_block", ctypes.c_int32)]


_lib = None


def load_library():
    """Load libmbg_fmm.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FmmError(-6, f"{LIB_PATH} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, dbl = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.fmm_plan.argtypes = [ctypes.POINTER(P), i64, i32, dbl, i32, i32]
    lib.fmm_build.argtypes = [P, P, P, P]
    lib.fmm_eval.argtypes = [P, P, P, P]
    lib.fmm_vjp.argtypes = [P, P, P, P, P, P]
    lib.fmm_lattice_steps.argtypes = [P, P, P, P, dbl, dbl, dbl, i32, i32, P]
    lib.fmm_destroy.argtypes = [P]
    lib.fmm_strerror.argtypes = [i32]
    lib.fmm_strerror.restype = ctypes.c_char_p
    lib.fmm_set_timing.argtypes = [P, i32]
    lib.fmm_set_walk_pool_hint.argtypes = [P, i64]
    lib.fmm_set_mutual_near_field.argtypes = [P, i32]
    lib.fmm_stats.argtypes = [P, ctypes.POINTER(_Stats)]
    lib.fmm_copy_keys.argtypes = [P, P, P]
    lib.fmm_copy_tree.argtypes = [P] * 8
    lib.fmm_copy_lists.argtypes = [P] * 5
    lib.fmm_copy_expansions.argtypes = [P, P, P]
    lib.fmm_direct.argtypes = [P, P, i64, P, i64, i32, P, P, P]
    lib.fmm_measure_peaks.argtypes = [P, P, P]
    lib.fmm_direct_noalloc.argtypes = [P, P, i64, P, i64, i32, P, P, P]
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _stream_handle(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


class Plan:
    """FMM plan for N particles: ``build(pos, mass)`` then ``eval() -> (phi, acc)``.

    pos: [N, 3] and mass: [N] device tensors of the plan's dtype (float32 or
    float64).  G = 1, no softening; outputs are in the input particle order.
    """

    def __init__(self, n: int, order: int = 4, theta: float = 0.7, leaf_size: int = 32,
                 dtype: torch.dtype = torch.float64, device=None):
        if dtype not in (torch.float32, torch.float64):
            raise FmmError(-1, "dtype must be float32 or float64")
        self.lib = load_library()
        self.n, self.order, self.theta, self.leaf_size = int(n), int(order), float(theta), int(leaf_size)
        self.dtype = dtype
        self.device = torch.device("cuda", torch.cuda.current_device() if device is None
                                   else torch.device(device).index or 0)
        self._h = ctypes.c_void_p()
        with torch.cuda.device(self.device):
            rc = self.lib.fmm_plan(ctypes.byref(self._h), self.n, self.order, self.theta,
                                   self.leaf_size, FMM_F64 if dtype == torch.float64 else FMM_F32)
        if rc:
            self._h = ctypes.c_void_p()
            raise FmmError(rc, "fmm_plan")
        self._keep = None

    def _check(self, rc, what):
        if rc:
            raise FmmError(rc, what)

    def build(self, pos: torch.Tensor, mass: torch.Tensor, stream=None) -> "Plan":
        if pos.shape != (self.n, 3) or mass.shape != (self.n,):
            raise FmmError(-1, "fmm_build: pos must be [N,3] and mass [N]")
        if pos.dtype != self.dtype or mass.dtype != self.dtype or not pos.is_cuda or not mass.is_cuda:
            raise FmmError(-1, "fmm_build: inputs must be device tensors of the plan dtype")
        pos = pos.contiguous()
        mass = mass.contiguous()
        with torch.cuda.device(self.device):
            rc = self.lib.fmm_build(self._h, ctypes.c_void_p(pos.data_ptr()),
                                    ctypes.c_void_p(mass.data_ptr()), _stream_handle(stream))
        self._check(rc, "fmm_build")
        return self

    def eval(self, phi: torch.Tensor | None = None, acc: torch.Tensor | None = None, stream=None):
        if phi is None:
            phi = torch.empty(self.n, dtype=self.dtype, device=self.device)
        if acc is None:
            acc = torch.empty(self.n, 3, dtype=self.dtype, device=self.device)
        if phi.shape != (self.n,) or acc.shape != (self.n, 3) or not phi.is_contiguous() \
                or not acc.is_contiguous() or phi.dtype != self.dtype or acc.dtype != self.dtype:
            raise FmmError(-1, "fmm_eval: phi [N] and acc [N,3] contiguous, plan dtype")
        with torch.cuda.device(self.device):
            rc = self.lib.fmm_eval(self._h, ctypes.c_void_p(phi.data_ptr()),
                                   ctypes.c_void_p(acc.data_ptr()), _stream_handle(stream))
        self._check(rc, "fmm_eval")
        return phi, acc

    def vjp(self, phi_bar: torch.Tensor, acc_bar: torch.Tensor, pos_bar: torch.Tensor | None = None,
            mass_bar: torch.Tensor | None = None, stream=None):
        """Sensitivities of S back to the built positions and masses, given
        phi_bar = dS/dphi [N] and acc_bar = dS/da [N,3] (fmm_vjp).  Returns
        (pos_bar [N,3], mass_bar [N])."""
        for t, shp in ((phi_bar, (self.n,)), (acc_bar, (self.n, 3))):
            if t.shape != shp or t.dtype != self.dtype or not t.is_cuda:
                raise FmmError(-1, "fmm_vjp: phi_bar [N] and acc_bar [N,3] device tensors, plan dtype")
        phi_bar, acc_bar = phi_bar.contiguous(), acc_bar.contiguous()
        if pos_bar is None:
            pos_bar = torch.empty(self.n, 3, dtype=self.dtype, device=self.device)
        if mass_bar is None:
            mass_bar = torch.empty(self.n, dtype=self.dtype, device=self.device)
        if pos_bar.shape != (self.n, 3) or mass_bar.shape != (self.n,) or not pos_bar.is_contiguous() \
                or not mass_bar.is_contiguous() or pos_bar.dtype != self.dtype or mass_bar.dtype != self.dtype:
            raise FmmError(-1, "fmm_vjp: pos_bar [N,3] and mass_bar [N] contiguous, plan dtype")
        with torch.cuda.device(self.device):
            rc = self.lib.fmm_vjp(self._h, ctypes.c_void_p(phi_bar.data_ptr()),
                                  ctypes.c_void_p(acc_bar.data_ptr()), ctypes.c_void_p(pos_bar.data_ptr()),
                                  ctypes.c_void_p(mass_bar.data_ptr()), _stream_handle(stream))
        self._check(rc, "fmm_vjp")
        return pos_bar, mass_bar

    def lattice_steps(self, q: torch.Tensor, u: torch.Tensor, mass: torch.Tensor, dx: float,
                      dv: float, dt: float, n_steps: int = 1, direction: int = 1, stream=None):
        """Reversible kick-drift-kick steps on the integer lattice x = q dx,
        v = u dv (fmm_lattice_steps); q and u are int64 [N,3] device tensors,
        updated in place.  direction -1 undoes direction +1 exactly."""
        for t in (q, u):
            if t.shape != (self.n, 3) or t.dtype != torch.int64 or not t.is_cuda or not t.is_contiguous():
                raise FmmError(-1, "fmm_lattice_steps: q and u contiguous int64 [N,3] device tensors")
        if mass.shape != (self.n,) or mass.dtype != self.dtype or not mass.is_cuda:
            raise FmmError(-1, "fmm_lattice_steps: mass [N] device tensor of the plan dtype")
        mass = mass.contiguous()
        with torch.cuda.device(self.device):
            rc = self.lib.fmm_lattice_steps(self._h, ctypes.c_void_p(q.data_ptr()),
                                            ctypes.c_void_p(u.data_ptr()),
                                            ctypes.c_void_p(mass.data_ptr()), float(dx), float(dv),
                                            float(dt), int(n_steps), int(direction),
                                            _stream_handle(stream))
        self._check(rc, "fmm_lattice_steps")
        return q, u

    def set_mutual_near_field(self, enable: bool = True) -> None:
        """Sum the sibling leaves' near field mutually (fmm_set_mutual_near_field);
        takes effect at the next build."""
        self._check(self.lib.fmm_set_mutual_near_field(self._h, 1 if enable else 0),
                    "fmm_set_mutual_near_field")

    def set_walk_pool_hint(self, entries_per_node: int = -1) -> None:
        """Walk pool size at each build's start, entries per node (-1: automatic;
        fmm_set_walk_pool_hint)."""
        self._check(self.lib.fmm_set_walk_pool_hint(self._h, int(entries_per_node)),
                    "fmm_set_walk_pool_hint")

    def set_timing(self, enable=True) -> None:
        """HIP events read at the next synchronization a call makes anyway.

        True or 1: stage and kernel events; 2: the main kernels' events only;
        3: the near-field kernels' events (and the fmm_vjp stage) only;
        False or 0: off.  Each event is a marker on the stream that costs a
        little by itself, so fewer events disturb the timed work less.
        """
        mode = 1 if enable is True else (0 if enable is False else int(enable))
        self._check(self.lib.fmm_set_timing(self._h, mode), "fmm_set_timing")

    def stats(self) -> dict:
        s = _Stats()
        self._check(self.lib.fmm_stats(self._h, ctypes.byref(s)), "fmm_stats")
        return {"n": s.n, "n_nodes": s.n_nodes, "n_leaves": s.n_leaves, "n_m2l": s.n_m2l,
                "n_p2p": s.n_p2p, "depth": s.depth, "order": s.order, "leaf_size": s.leaf_size,
                "theta": s.theta, "lo": list(s.lo), "side": s.side, "walk_retries": s.walk_retries,
                "stage_ms": {k: float(v) for k, v in zip(STAGES, s.stage_ms)},
                "kernel_ms": {k: float(v) for k, v in zip(KERNELS, s.kernel_ms)},
                "timed_builds": s.timed_builds, "timed_evals": s.timed_evals,
                "timed_vjps": s.timed_vjps, "walk_one_block": bool(s.walk_one_block)}

    def copy_keys(self):
        keys = np.zeros(self.n, dtype=np.uint64)
        perm = np.zeros(self.n, dtype=np.int32)
        self._check(self.lib.fmm_copy_keys(self._h, _ptr(keys), _ptr(perm)), "fmm_copy_keys")
        return keys, perm

    def copy_tree(self) -> dict:
        m = self.stats()["n_nodes"]
        out = {"level": np.zeros(m, np.uint8), "prefix": np.zeros(m, np.uint64),
               "begin": np.zeros(m, np.int32), "count": np.zeros(m, np.int32),
               "parent": np.zeros(m, np.int32), "first_child": np.zeros(m, np.int32),
               "n_child": np.zeros(m, np.uint8)}
        self._check(self.lib.fmm_copy_tree(self._h, *[_ptr(out[k]) for k in
                                                      ("level", "prefix", "begin", "count", "parent",
                                                       "first_child", "n_child")]), "fmm_copy_tree")
        return out

    def copy_lists(self) -> dict:
        st = self.stats()
        m = st["n_nodes"]
        out = {"m2l_off": np.zeros(m + 1, np.int64), "m2l_src": np.zeros(max(st["n_m2l"], 1), np.int32),
               "p2p_off": np.zeros(m + 1, np.int64), "p2p_src": np.zeros(max(st["n_p2p"], 1), np.int32)}
        self._check(self.lib.fmm_copy_lists(self._h, _ptr(out["m2l_off"]), _ptr(out["m2l_src"]),
                                            _ptr(out["p2p_off"]), _ptr(out["p2p_src"])), "fmm_copy_lists")
        out["m2l_src"] = out["m2l_src"][:st["n_m2l"]]
        out["p2p_src"] = out["p2p_src"][:st["n_p2p"]]
        return out

    def copy_expansions(self):
        st = self.stats()
        K = (self.order + 1) * (self.order + 2) * (self.order + 3) // 6
        mp = np.zeros((st["n_nodes"], K))
        lc = np.zeros((st["n_nodes"], K))
        self._check(self.lib.fmm_copy_expansions(self._h, _ptr(mp), _ptr(lc)), "fmm_copy_expansions")
        return mp, lc

    def close(self) -> None:
        if getattr(self, "_h", None) and self._h.value:
            self.lib.fmm_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _direct_call(name, pos, mass, targets, phi, acc, stream):
    if pos.dim() != 2 or pos.shape[1] != 3 or mass.shape != (pos.shape[0],):
        raise FmmError(-1, f"{name}: pos must be [N,3] and mass [N]")
    if pos.dtype not in (torch.float32, torch.float64) or mass.dtype != pos.dtype:
        raise FmmError(-1, f"{name}: pos and mass of one float dtype")
    if targets.dtype != torch.int64 or not (pos.is_cuda and mass.is_cuda and targets.is_cuda):
        raise FmmError(-1, f"{name}: device tensors, int64 targets")
    pos, mass, targets = pos.contiguous(), mass.contiguous(), targets.contiguous()
    nt = targets.shape[0]
    if phi is None:
        phi = torch.empty(nt, dtype=pos.dtype, device=pos.device)
    if acc is None:
        acc = torch.empty(nt, 3, dtype=pos.dtype, device=pos.device)
    if phi.shape != (nt,) or acc.shape != (nt, 3) or phi.dtype != pos.dtype \
            or acc.dtype != pos.dtype or not phi.is_contiguous() or not acc.is_contiguous():
        raise FmmError(-1, f"{name}: phi [T] and acc [T,3] contiguous, the inputs' dtype")
    lib = load_library()
    with torch.cuda.device(pos.device):
        rc = getattr(lib, name)(ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(mass.data_ptr()),
                                pos.shape[0], ctypes.c_void_p(targets.data_ptr()), nt,
                                FMM_F64 if pos.dtype == torch.float64 else FMM_F32,
                                ctypes.c_void_p(phi.data_ptr()), ctypes.c_void_p(acc.data_ptr()),
                                _stream_handle(stream))
    if rc:
        raise FmmError(rc, name)
    return phi, acc


def direct(pos: torch.Tensor, mass: torch.Tensor, targets: torch.Tensor, stream=None):
    """Direct-sum potential and acceleration of particles `targets` (int64 device
    tensor of indices) from all particles (fp64 sums; fmm_direct)."""
    return _direct_call("fmm_direct", pos, mass, targets, None, None, stream)


DIRECT_NOALLOC_MAX_TARGETS = 4096


def direct_noalloc(pos: torch.Tensor, mass: torch.Tensor, targets: torch.Tensor,
                   phi: torch.Tensor | None = None, acc: torch.Tensor | None = None, stream=None):
    """fmm_direct_noalloc: the same sums with the library's static workspace (at
    most DIRECT_NOALLOC_MAX_TARGETS targets; asynchronous on the stream).  Pass
    phi [T] and acc [T,3] to keep the call free of any allocation."""
    return _direct_call("fmm_direct_noalloc", pos, mass, targets, phi, acc, stream)


def measure_peaks(stream=None):
    """Measured fp64 and fp32 (unpacked) vector multiply-add rates of the
    current device in TFLOP/s (fmm_measure_peaks)."""
    lib = load_library()
    f64, f32 = ctypes.c_double(), ctypes.c_double()
    rc = lib.fmm_measure_peaks(ctypes.byref(f64), ctypes.byref(f32), _stream_handle(stream))
    if rc:
        raise FmmError(rc, "fmm_measure_peaks")
    return f64.value, f32.value
