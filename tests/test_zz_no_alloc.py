"""The allocation-free direct sum (fmm_direct_noalloc) against fmm_direct,
through the C-ABI: two calls in a row, the second with a smaller input, each
equal bit for bit to the allocating entry point's result (same kernels, same
summation order), in fp64 and fp32; and its argument checks."""
import ctypes

import numpy as np
import pytest

from multipole_body_gravity_amd import workloads as W

pytestmark = pytest.mark.gpu


def _call(lib, name, pos, mass, tg, phi, acc):
    import torch
    dt = 1 if pos.dtype == torch.float64 else 0
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return getattr(lib, name)(ctypes.c_void_p(pos.data_ptr()), ctypes.c_void_p(mass.data_ptr()),
                              pos.shape[0], ctypes.c_void_p(tg.data_ptr()), tg.shape[0], dt,
                              ctypes.c_void_p(phi.data_ptr()), ctypes.c_void_p(acc.data_ptr()), s)


@pytest.mark.parametrize("dt", ["f64", "f32"])
def test_direct_noalloc_matches_direct(dt):
    import torch

    from multipole_body_gravity_amd import fmm
    lib = fmm.load_library()
    dev = torch.device("cuda:0")
    tdt = torch.float64 if dt == "f64" else torch.float32
    cases = [("plummer", 30000, 401, 4096), ("clustered", 7001, 402, 333)]  # second smaller
    for dist, n, seed, nt in cases:
        print(f"  noalloc {dt} {dist} n={n} targets={nt}", flush=True)
        pos, mass = W.make(dist, n, seed)
        tp = torch.from_numpy(pos).to(dev, tdt)
        tm = torch.from_numpy(mass).to(dev, tdt)
        tg = torch.from_numpy(np.random.default_rng(seed).choice(n, nt, replace=False)).to(dev)
        ref_phi = torch.empty(nt, dtype=tdt, device=dev)
        ref_acc = torch.empty(nt, 3, dtype=tdt, device=dev)
        assert _call(lib, "fmm_direct", tp, tm, tg, ref_phi, ref_acc) == 0
        phi = torch.full((nt,), float("nan"), dtype=tdt, device=dev)
        acc = torch.full((nt, 3), float("nan"), dtype=tdt, device=dev)
        assert _call(lib, "fmm_direct_noalloc", tp, tm, tg, phi, acc) == 0
        torch.cuda.synchronize()
        assert torch.equal(phi, ref_phi) and torch.equal(acc, ref_acc)
        assert torch.isfinite(acc).all()


def test_direct_noalloc_arguments():
    import torch

    from multipole_body_gravity_amd import fmm
    lib = fmm.load_library()
    dev = torch.device("cuda:0")
    tp = torch.rand(100, 3, dtype=torch.float64, device=dev)
    tm = torch.ones(100, dtype=torch.float64, device=dev)
    too_many = torch.zeros(fmm.DIRECT_NOALLOC_MAX_TARGETS + 1, dtype=torch.int64, device=dev)
    phi = torch.empty(too_many.shape[0], dtype=torch.float64, device=dev)
    acc = torch.empty(too_many.shape[0], 3, dtype=torch.float64, device=dev)
    assert _call(lib, "fmm_direct_noalloc", tp, tm, too_many, phi, acc) == -1
    # the Python binding with caller-supplied outputs
    tg = torch.arange(0, 100, 7, dtype=torch.int64, device=dev)
    p1, a1 = fmm.direct(tp, tm, tg)
    p2, a2 = fmm.direct_noalloc(tp, tm, tg)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(a1, a2)
