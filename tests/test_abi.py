"""CPU-only checks of the C ABI: the library loads, exports every entry point
that include/spec_verify.h declares, and its host-side validation rejects bad
arguments before anything reaches the GPU (no compute call is made)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "rejection_sampling_verify_13_amd", "libspecverify.so")


def declared_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(spec_verify\w*)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libspecverify.so is not built; run __graft_entry__.build()")
    import rejection_sampling_verify_13_amd as sv  # imports torch first, then binds
    return sv.lib


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("spec_verify", "spec_verify_diag", "spec_verify_workspace_size", "spec_verify_status_string",
              "spec_verify_version", "spec_verify_flat", "spec_verify_flat_timed", "spec_verify_rollback",
              "spec_verify_flat_synthetic", "spec_verify_flat_ex", "spec_verify_device_errors",
              "spec_verify_static", "spec_verify_static_scratch_bytes"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_version_and_status_strings(lib):
    assert lib.spec_verify_version() == 1
    for code in range(7):
        assert lib.spec_verify_status_string(code)


def test_static_entry_point_host_validation(lib):
    # sizes are checked before any device state is touched
    P = ctypes.c_void_p(0x1000)
    call = lambda N, G, V: lib.spec_verify_static(N, G, V, P, P, P, 1, None, None, None, P, P, P, P, None)
    assert lib.spec_verify_static_scratch_bytes() == 16 << 20
    assert call(-1, 4, 100) == 2
    assert call(4, 65, 100) == 2
    assert call(0, 4, 100) == 0
    assert lib.spec_verify_workspace_size(8192, 8, 151936) > lib.spec_verify_static_scratch_bytes()
    assert call(8192, 8, 151936) == 6
    assert lib.spec_verify_workspace_size(1024, 8, 128256) <= lib.spec_verify_static_scratch_bytes()


def _call(lib, N=2, G=3, V=16, ids=1, q=0, logits=1, dtype=1, ua=1, us=1, out=1, num=1, ws=None, wsb=0):
    P = lambda flag: ctypes.c_void_p(0x1000) if flag else None
    return lib.spec_verify(N, G, V, P(ids), P(q), P(logits), dtype, None, None, None, P(ua), P(us), P(out),
                           P(num), ws, wsb, None)


def test_host_validation(lib):
    # every rejected call returns before touching device memory or launching
    assert _call(lib, N=-1) == 2
    assert _call(lib, G=65) == 2
    assert _call(lib, G=-1) == 2
    assert _call(lib, V=0) == 2
    assert _call(lib, dtype=7) == 3
    assert _call(lib, logits=0) == 1
    assert _call(lib, us=0) == 1
    assert _call(lib, out=0) == 1
    assert _call(lib, num=0) == 1
    assert _call(lib, ids=0) == 1
    assert _call(lib, ua=0) == 1
    assert _call(lib, N=0) == 0  # empty batch: nothing to do
    # grids whose size in work-items (256 per workgroup) needs more than 32 bits
    assert _call(lib, N=(1 << 24) // 65 + 1, G=64) == 2     # row pass: N * (gmax + 2) workgroups
    # padded layout, gmax a multiple of 8: one more row-pass workgroup per request
    assert _call(lib, N=(1 << 32) // 2560 + 1, G=8) == 2     # N * 10 * 256 reaches 2^32
    assert _call(lib, N=(1 << 32) // 2560, G=8, logits=0) == 1  # just inside: the next check fires
    assert _call(lib, N=(1 << 32) // 2560 + 1, G=7, logits=0) == 1  # gmax = 7: N * 8 workgroups
    assert _call(lib, N=(1 << 24) // 2, G=0, V=16384) == 2   # draw pass: N * 2 workgroups at 8192 < V <= 16384
    assert _call(lib, N=(1 << 24) // 2 - 1, G=0, V=16384, logits=0) == 1  # just inside: the next check fires
    assert _call(lib, N=(1 << 24), G=0, V=16) == 2           # row pass: N workgroups
    small = ctypes.c_void_p(0x1000)
    assert _call(lib, ws=small, wsb=16) == 4
    # the workspace is the caller's: a NULL one is refused, nothing is allocated
    assert _call(lib) == 1
    assert _call(lib, N=0) == 0


def test_device_errors_host_validation(lib):
    n = ctypes.c_int32(7)
    ws = ctypes.c_void_p(0x1000)
    assert lib.spec_verify_device_errors(None, 4096, None, ctypes.byref(n)) == 1
    assert lib.spec_verify_device_errors(ws, 4096, None, None) == 1
    assert lib.spec_verify_device_errors(ws, 255, None, ctypes.byref(n)) == 4
    assert n.value == 7  # untouched when refused
    assert lib.spec_verify_workspace_size(0, 0, 1) >= 256


def _flat(lib, N=2, G=3, V=16, T=4, cu=1, ids=1, logits=1, ua=1, us=1, out=1, num=1):
    P = lambda flag: ctypes.c_void_p(0x1000) if flag else None
    return lib.spec_verify_flat(N, G, V, T, P(cu), P(ids), None, None, P(logits), 1, None, None, None, P(ua), P(us),
                                P(out), P(num), None, 0, None)


def test_flat_host_validation(lib):
    assert _flat(lib, cu=0) == 1
    assert _flat(lib, T=-1) == 2
    assert _flat(lib, T=7) == 2          # more drafts than N * gmax
    assert _flat(lib, ids=0) == 1
    assert _flat(lib, ua=0) == 1
    assert _flat(lib, T=0, ids=0, ua=0, logits=0) == 1   # ids may be NULL without drafts; logits may not
    assert _flat(lib, N=0, cu=0) == 0    # empty batch
    assert _flat(lib, G=65) == 2


def _ex(lib, N=2, G=3, V=16, T=4, R=6, tidx=0, bidx=0, boff=0, bids=0, pen=(0, 0, 0, 0, 0, 0)):
    P = lambda flag: ctypes.c_void_p(0x1000) if flag else None
    # a 16-byte workspace: every accepted argument set stops at the workspace check
    return lib.spec_verify_flat_ex(N, G, V, T, P(1), P(1), None, None, P(1), R, P(tidx), P(bidx), 1, None, None, None,
                                   P(boff), P(bids), *[P(x) for x in pen], P(1), P(1), P(1), P(1), None, None, None,
                                   None, P(1), 16, None, None, None, None)


def test_flat_ex_host_validation(lib):
    assert _ex(lib) == 4
    assert _ex(lib, tidx=1) == 1               # draft-row indices without bonus-row indices
    assert _ex(lib, bidx=1) == 1               # bonus-row indices without draft-row indices, with drafts
    assert _ex(lib, T=0, R=1, bidx=1) == 4     # no drafts: the draft-row indices may be NULL
    assert _ex(lib, R=5) == 2                  # fewer rows than num_drafts + N without indices
    assert _ex(lib, R=0, tidx=1, bidx=1) == 2
    assert _ex(lib, R=1, tidx=1, bidx=1) == 4  # any row count with indices
    assert _ex(lib, bids=1) == 1               # banned ids without offsets
    assert _ex(lib, boff=1) == 4               # offsets alone: every list empty
    assert _ex(lib, N=0, T=0, R=0, tidx=1) == 0  # empty batch
    # penalties: the offsets select the option; ids and counts go together
    assert _ex(lib, pen=(1, 0, 0, 0, 0, 0)) == 4
    assert _ex(lib, pen=(1, 1, 1, 1, 1, 1)) == 4
    assert _ex(lib, pen=(1, 1, 0, 0, 0, 0)) == 1
    assert _ex(lib, pen=(1, 0, 1, 0, 0, 0)) == 1
    for k in range(1, 6):
        assert _ex(lib, pen=tuple(int(t == k) for t in range(6))) == 1   # a penalty argument without offsets


def test_synthetic_host_validation(lib):
    P = lambda: ctypes.c_void_p(0x1000)
    call = lambda N, G, rates: lib.spec_verify_flat_synthetic(N, G, 16, N * G, P(), P(), None, None, P(), 1, None,
                                                               None, None, rates, P(), P(), P(), P(), None, None,
                                                               0, None, None, None, None)
    assert call(2, 3, None) == 1          # rates required with drafts
    assert call(0, 3, None) == 0          # empty batch
    assert call(2, 65, P()) == 2


def test_rollback_host_validation(lib):
    P = ctypes.c_void_p(0x1000)
    assert lib.spec_verify_rollback(-1, 4, P, None, P, None, None, None, None) == 2
    assert lib.spec_verify_rollback(3, 65, P, None, P, None, None, None, None) == 2
    assert lib.spec_verify_rollback(3, 4, P, None, None, None, None, None, None) == 1   # num_accepted
    assert lib.spec_verify_rollback(3, 4, None, None, P, None, None, None, None) == 1   # no counts
    assert lib.spec_verify_rollback(3, 4, P, P, P, None, None, None, None) == 1        # both layouts
    assert lib.spec_verify_rollback(0, 4, None, None, None, None, None, None, None) == 0


def test_workspace_size_grows_with_rows(lib):
    a = lib.spec_verify_workspace_size(10, 4, 1000)
    b = lib.spec_verify_workspace_size(20, 4, 1000)
    c = lib.spec_verify_workspace_size(10, 8, 1000)
    assert 0 < a < b and a < c
