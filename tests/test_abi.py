"""C-ABI checks that need no GPU: the library loads, exports every function that
include/fmm.h declares, and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fmm.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(fmm_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    from multipole_body_gravity_amd import fmm
    return fmm.load_library()


def test_header_declares_entry_points():
    names = declared_functions()
    for want in ["fmm_plan", "fmm_build", "fmm_eval", "fmm_destroy", "fmm_strerror",
                 "fmm_set_timing", "fmm_stats", "fmm_copy_keys", "fmm_copy_tree",
                 "fmm_copy_lists", "fmm_copy_expansions", "fmm_direct", "fmm_vjp", "fmm_lattice_steps",
                 "fmm_node_id_bits", "fmm_direct_noalloc", "fmm_set_walk_pool_hint",
                 "fmm_measure_peaks", "fmm_set_mutual_near_field"]:
        assert want in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror(lib):
    for code in [0, -1, -2, -3, -4, -5, -6]:
        s = lib.fmm_strerror(code)
        assert s and s != b"unknown status"
    assert lib.fmm_strerror(12345) == b"unknown status"


@pytest.mark.parametrize("args", [
    (0, 4, 0.7, 32, 1), (-5, 4, 0.7, 32, 1), (2 ** 31, 4, 0.7, 32, 1),
    (10, -1, 0.7, 32, 1), (10, 11, 0.7, 32, 1),
    (10, 4, 0.0, 32, 1), (10, 4, 1.0, 32, 1), (10, 4, float("nan"), 32, 1),
    (10, 4, 0.7, 0, 1), (10, 4, 0.7, 32, 2), (10, 4, 0.7, 32, -1)])
def test_plan_rejects_bad_arguments(lib, args):
    """Orders 0..10 are accepted (FMM_MAX_ORDER = 10); everything outside the
    documented ranges is refused before any device call."""
    h = ctypes.c_void_p()
    assert lib.fmm_plan(ctypes.byref(h), *args) == -1
    assert not h.value


def test_null_plan_calls(lib):
    P = ctypes.c_void_p
    assert lib.fmm_build(None, P(1), P(1), None) == -1
    assert lib.fmm_eval(None, P(1), P(1), None) == -1
    assert lib.fmm_vjp(None, P(1), P(1), P(1), P(1), None) == -1
    D = ctypes.c_double
    assert lib.fmm_lattice_steps(None, P(1), P(1), P(1), D(1.0), D(1.0), D(0.1), 1, 1, None) == -1
    assert lib.fmm_destroy(None) == -1
    # the direct-sum reference checks its arguments before any device call
    assert lib.fmm_direct(None, P(1), 10, P(1), 1, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct(P(1), P(1), 0, P(1), 1, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct(P(1), P(1), 10, P(1), -1, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct(P(1), P(1), 10, P(1), 1, 7, P(1), P(1), None) == -1
    assert lib.fmm_direct(P(1), P(1), 10, P(1), 0, 1, P(1), P(1), None) == 0
    # the allocation-free variant: the same checks, and at most 4096 targets
    assert lib.fmm_direct_noalloc(None, P(1), 10, P(1), 1, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct_noalloc(P(1), P(1), 0, P(1), 1, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct_noalloc(P(1), P(1), 10, P(1), 4097, 1, P(1), P(1), None) == -1
    assert lib.fmm_direct_noalloc(P(1), P(1), 10, P(1), 1, 7, P(1), P(1), None) == -1
    assert lib.fmm_direct_noalloc(P(1), P(1), 10, P(1), 0, 1, P(1), P(1), None) == 0
    assert lib.fmm_set_timing(None, 1) == -1
    lib.fmm_set_walk_pool_hint.argtypes = [P, ctypes.c_int64]
    assert lib.fmm_set_walk_pool_hint(None, 4) == -1
    assert lib.fmm_set_mutual_near_field(None, 1) == -1
    assert lib.fmm_copy_keys(None, None, None) == -1
    assert lib.fmm_plan(None, 10, 4, 0.7, 32, 1) == -1


def test_node_id_bits(lib):
    """The walk packs (kind, target, source) node ids into 2 b + 1 bits, b the
    bits that hold every id of the tree; the largest tree a build accepts
    (FMM_MAX_NODES = 2^31 - 1 cells) still fits 64 bits, one more cell does
    not, and is refused."""
    lib.fmm_node_id_bits.argtypes = [ctypes.c_int64, ctypes.POINTER(ctypes.c_int)]
    b = ctypes.c_int()
    max_nodes = 2 ** 31 - 1
    text = open(HEADER).read()
    assert re.search(r"#define FMM_MAX_NODES 2147483647LL", text)
    for nn, want in [(1, 1), (2, 2), (3, 2), (4, 3), (125390, 17), (2 ** 30, 31),
                     (2 ** 31 - 1, 31)]:
        assert lib.fmm_node_id_bits(nn, ctypes.byref(b)) == 0
        assert b.value == want, (nn, b.value)
        assert (1 << b.value) > nn >= (1 << (b.value - 1)) or nn == 1
    assert lib.fmm_node_id_bits(max_nodes, ctypes.byref(b)) == 0
    assert 2 * b.value + 1 <= 64
    for bad in (0, -1, max_nodes + 1, 2 ** 40):
        assert lib.fmm_node_id_bits(bad, ctypes.byref(b)) == -1
    assert lib.fmm_node_id_bits(10, None) == -1
