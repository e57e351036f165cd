"""The C-ABI library on the host: it loads, exports every function that
include/spconv_mi355x.h declares, and its argument checks return the
documented status codes before anything is enqueued (no GPU needed)."""
import ctypes
import os
import re

import pytest

import submanifold_sparse_convolution_spconv_amd as sp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spconv_mi355x.h")
FAKE = 0x7f0000000000           # aligned, never dereferenced: every call below fails a check first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spconv_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return sp.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version_and_strings(lib):
    assert lib.spconv_abi_version() == 1
    for code, name in sp.STATUS.items():
        s = lib.spconv_status_string(code).decode()
        assert s and s != "unknown status", name
    assert lib.spconv_status_string(99).decode() == "unknown status"


def sizes(lib, N, K):
    a, w = ctypes.c_size_t(), ctypes.c_size_t()
    rc = lib.spconv_nmap_sizes(N, K, ctypes.byref(a), ctypes.byref(w))
    return rc, a.value, w.value


def test_sizes(lib):
    rc, a, w = sizes(lib, 1006716, 27)
    assert rc == 0
    npad = (1006716 + 255) // 256 * 256
    # map + row order, one 16-bit block mask per (tile, offset), one 64-bit
    # pair count per tile, and per half tile (128 rows) the distinct-row
    # count, up to 3 x 315 listed rows (one list per staging pass) and a
    # 16-bit slot code per (row, offset), plus alignment and a small header
    ntiles = npad // 256
    need = (4 * 27 * npad + 4 * npad + 2 * 27 * ntiles + 8 * ntiles + 4 * 2 * ntiles
            + 4 * 945 * 2 * ntiles + 2 * 27 * 256 * ntiles)
    assert need <= a < need + 4096
    assert w >= 24 * 1006716 + 16 * (1 << 21)
    # maps of more than 27 offsets keep no distinct-row lists
    rc, a125, _ = sizes(lib, 1006716, 125)
    need125 = 4 * 125 * npad + 4 * npad + 2 * 125 * ntiles + 8 * ntiles + 4 * 2 * ntiles
    assert rc == 0 and need125 <= a125 < need125 + 4096
    assert sizes(lib, -1, 27)[0] == -1
    assert sizes(lib, 10, 0)[0] == -1
    assert sizes(lib, 1 << 31, 27)[0] == -2
    rc, a0, w0 = sizes(lib, 0, 27)
    assert rc == 0 and a0 > 0


def build(lib, coords, N, K, d, arena, ab, ws, wb, out=True):
    h = ctypes.c_void_p()
    rc = lib.spconv_build_nmap(ctypes.c_void_p(coords), N, K, d, ctypes.c_void_p(arena), ab,
                               ctypes.c_void_p(ws), wb, None, ctypes.byref(h) if out else None)
    return rc, h


def test_build_argument_checks(lib):
    _, a, w = sizes(lib, 1000, 27)
    assert build(lib, FAKE, 1000, 26, 1, FAKE, a, FAKE, w)[0] == -1        # K not an odd cube
    assert build(lib, FAKE, 1000, 8, 1, FAKE, a, FAKE, w)[0] == -1         # even cube
    assert build(lib, FAKE, 1000, 27, 0, FAKE, a, FAKE, w)[0] == -1        # dilation < 1
    assert build(lib, FAKE, 1000, 27, 1, 0, a, FAKE, w)[0] == -1           # NULL arena
    assert build(lib, FAKE, 1000, 27, 1, FAKE + 4, a, FAKE, w)[0] == -1    # misaligned arena
    assert build(lib, FAKE, 1000, 27, 1, FAKE, a - 1, FAKE, w)[0] == -5    # arena too small
    assert build(lib, FAKE, 1000, 27, 1, FAKE, a, FAKE, w - 1)[0] == -5    # workspace too small
    assert build(lib, 0, 1000, 27, 1, FAKE, a, FAKE, w)[0] == -1           # NULL coords
    assert build(lib, FAKE, 1000, 27, 1, FAKE, a, 0, w)[0] == -1           # NULL workspace
    assert build(lib, FAKE, 1000, 27, 1, FAKE, a, FAKE, w, out=False)[0] == -1
    assert build(lib, FAKE, -5, 27, 1, FAKE, a, FAKE, w)[0] == -1
    rc, _ = build(lib, FAKE, 1000, 26, 1, FAKE, a, FAKE, w)
    assert b"odd cube" in lib.spconv_last_error()
    lib.spconv_last_hip_error.restype = ctypes.c_char_p
    assert lib.spconv_last_hip_error() == lib.spconv_last_error()


def test_empty_map_is_a_noop(lib):
    _, a, _ = sizes(lib, 0, 27)
    rc, h = build(lib, 0, 0, 27, 1, FAKE, a, 0, 0)
    assert rc == 0 and h.value
    N, K, d, vp = ctypes.c_int64(), ctypes.c_int(), ctypes.c_int(), ctypes.c_int64()
    assert lib.spconv_nmap_info(h, ctypes.byref(N), ctypes.byref(K), ctypes.byref(d), ctypes.byref(vp),
                                None) == 0
    assert (N.value, K.value, d.value, vp.value) == (0, 27, 1, 0)
    assert lib.spconv_nmap_export(h, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == 0
    # forward over no voxels enqueues nothing
    assert lib.spconv_forward(ctypes.c_void_p(FAKE), h, ctypes.c_void_p(FAKE), None,
                              ctypes.c_void_p(FAKE), 128, 128, 1, None) == 0
    lib.spconv_nmap_destroy(h)


def test_forward_argument_checks(lib):
    _, a, _ = sizes(lib, 0, 27)
    rc, h = build(lib, 0, 0, 27, 1, FAKE, a, 0, 0)
    assert rc == 0
    F = lambda h_, ci, co, dt: lib.spconv_forward(ctypes.c_void_p(FAKE), h_, ctypes.c_void_p(FAKE), None,
                                                  ctypes.c_void_p(FAKE), ci, co, dt, None)
    assert F(None, 32, 32, 0) == -1                 # no handle
    assert F(h, 32, 32, 2) == -1                    # bad dtype
    assert F(h, 48, 32, 0) == -2                    # Ci without a kernel
    assert F(h, 32, 40, 1) == -2                    # Co not a multiple of 32
    assert F(h, 32, 8192, 1) == -2
    assert F(h, 0, 32, 1) == -1
    assert F(h, 256, 4096, 0) == 0                  # supported, N = 0
    lib.spconv_nmap_destroy(h)


def test_forward_mixed_argument_checks(lib):
    _, a, _ = sizes(lib, 0, 27)
    rc, h = build(lib, 0, 0, 27, 1, FAKE, a, 0, 0)
    assert rc == 0
    M = lambda h_, fdt, ci, co, dt, ws=None, wsb=0: lib.spconv_forward_mixed(
        ctypes.c_void_p(FAKE), fdt, h_, ctypes.c_void_p(FAKE), None, None, ctypes.c_void_p(FAKE), ci, co, dt,
        None if ws is None else ctypes.c_void_p(ws), ctypes.c_size_t(wsb), None)
    assert M(None, 0, 32, 32, 1) == -1              # no handle
    assert M(h, 2, 32, 32, 1) == -1                 # bad feats dtype
    assert M(h, -1, 32, 32, 0) == -1
    assert M(h, 0, 32, 32, 3) == -1                 # bad w dtype
    assert M(h, 0, 48, 32, 1) == -2                 # Ci without a kernel
    for fdt in (0, 1):
        for dt in (0, 1):
            assert M(h, fdt, 128, 128, dt) == 0     # every pairing, N = 0
            assert M(h, fdt, 128, 128, dt, FAKE, 0) == 0
    lib.spconv_nmap_destroy(h)
    # the cast pass's workspace: N*Ci bf16 values for fp32 feats into bf16 w, else none
    n = ctypes.c_size_t(7)
    S = lambda N, ci, fdt, dt: lib.spconv_forward_mixed_workspace_size(N, ci, fdt, dt, ctypes.byref(n))
    assert S(1000, 128, 0, 1) == 0 and n.value == 256000
    assert S(1001, 32, 0, 1) == 0 and n.value == 64256              # 64064 rounded up to 256
    for fdt, dt in ((1, 0), (0, 0), (1, 1)):
        assert S(1000, 128, fdt, dt) == 0 and n.value == 0
    assert S(-1, 128, 0, 1) == -1 and S(10, 128, 2, 1) == -1 and S(10, 0, 0, 1) == -1
    assert lib.spconv_forward_mixed_workspace_size(10, 128, 0, 1, None) == -1


def test_wrap_argument_checks(lib):
    _, a, _ = sizes(lib, 100, 27)
    h = ctypes.c_void_p()
    W = lambda nbr, N, K, arena, ab: lib.spconv_nmap_wrap(ctypes.c_void_p(nbr), N, K, ctypes.c_void_p(arena),
                                                          ab, None, ctypes.byref(h))
    assert W(FAKE, 100, 0, FAKE, a) == -1
    assert W(0, 100, 27, FAKE, a) == -1
    assert W(FAKE, 100, 27, FAKE, a - 1) == -5
    assert W(FAKE, 100, 27, 0, a) == -1
    _, a0, _ = sizes(lib, 0, 27)
    assert W(0, 0, 27, FAKE, a0) == 0 and h.value
    lib.spconv_nmap_destroy(h)


def test_pack_weights_sizes(lib):
    """The packed copy has w's own size wherever a packed form exists (bf16,
    Ci in {128, 256}, any output-channel tile), and none elsewhere."""
    pk = ctypes.c_size_t()
    for K, ci, co in [(27, 128, 128), (27, 128, 64), (3, 128, 96), (2, 256, 64), (2, 256, 96), (2, 128, 32),
                      (1, 256, 256), (125, 128, 160)]:
        assert lib.spconv_pack_weights_size(K, ci, co, 1, ctypes.byref(pk)) == 0
        assert pk.value == K * ci * co * 2, (K, ci, co)
    for K, ci, co, dt in [(27, 128, 128, 0), (27, 64, 64, 1), (27, 32, 96, 1)]:
        assert lib.spconv_pack_weights_size(K, ci, co, dt, ctypes.byref(pk)) == 0
        assert pk.value == 0, (K, ci, co, dt)


def test_dgrad_argument_checks(lib):
    sz = ctypes.c_size_t()
    WS = lambda K, ci, co, dt: lib.spconv_dgrad_workspace_size(K, ci, co, dt, ctypes.byref(sz))
    assert WS(27, 128, 128, 1) == 0
    # mirrored weights (27*128*128 bf16) plus their packed form (the exchanged forward's)
    pk = ctypes.c_size_t()
    assert lib.spconv_pack_weights_size(27, 128, 128, 1, ctypes.byref(pk)) == 0
    assert sz.value == 27 * 128 * 128 * 2 + pk.value
    assert WS(27, 96, 64, 0) == 0 and sz.value == (27 * 96 * 64 * 4 + 255) // 256 * 256
    assert WS(27, 64, 48, 0) == -2                  # Co has no kernel as the exchanged Ci
    assert WS(27, 40, 64, 1) == -2                  # Ci not a multiple of 32
    assert WS(0, 64, 64, 1) == -1
    assert WS(27, 64, 64, 3) == -1
    assert lib.spconv_dgrad_workspace_size(27, 64, 64, 1, None) == -1
    D = lambda h_, ws, wb, ci, co, dt: lib.spconv_dgrad(ctypes.c_void_p(FAKE), h_, ctypes.c_void_p(FAKE),
                                                        ctypes.c_void_p(ws), wb, ctypes.c_void_p(FAKE),
                                                        ci, co, dt, None)
    assert D(None, FAKE, 1 << 30, 64, 64, 1) == -1  # no handle
    _, a, _ = sizes(lib, 0, 27)
    rc, h = build(lib, 0, 0, 27, 1, FAKE, a, 0, 0)
    assert rc == 0
    assert D(h, FAKE, 1 << 30, 64, 48, 1) == -2     # no kernel
    assert D(h, FAKE, 1 << 30, 64, 64, 1) == 0      # supported, N = 0: nothing enqueued
    lib.spconv_nmap_destroy(h)
    # a caller-made map need not be its own mirror
    hw = ctypes.c_void_p()
    assert lib.spconv_nmap_wrap(None, 0, 27, ctypes.c_void_p(FAKE), a, None, ctypes.byref(hw)) == 0
    assert D(hw, FAKE, 1 << 30, 64, 64, 1) == -2
    lib.spconv_nmap_destroy(hw)


def test_wgrad_argument_checks(lib):
    sz = ctypes.c_size_t()
    WS = lambda N, K, ci, co, dt: lib.spconv_wgrad_workspace_size(N, K, ci, co, dt, ctypes.byref(sz))
    assert WS(1006716, 27, 128, 128, 1) == 0
    assert sz.value > 0 and sz.value % (27 * 128 * 128 * 4) == 0   # whole fp32 partial tiles
    assert WS(1000, 27, 96, 64, 0) == 0
    assert WS(1000, 27, 48, 64, 1) == -2                # not a multiple of 32
    assert WS(1000, 27, 64, 8192, 1) == -2
    assert WS(1000, 0, 64, 64, 1) == -1
    assert WS(-1, 27, 64, 64, 1) == -1
    assert WS(1000, 27, 64, 64, 5) == -1
    G = lambda h_, ws, wb, dw, ci, co: lib.spconv_wgrad(ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), h_,
                                                        ctypes.c_void_p(ws), wb, ctypes.c_void_p(dw), ci, co, 1, None)
    assert G(None, FAKE, 1 << 30, FAKE, 64, 64) == -1  # no handle
    _, a, _ = sizes(lib, 0, 27)
    rc, h = build(lib, 0, 0, 27, 1, FAKE, a, 0, 0)
    assert rc == 0
    assert G(h, FAKE, 1 << 30, 0, 64, 64) == -1        # no dw
    assert G(h, FAKE, 1 << 30, FAKE + 4, 64, 64) == -1 # misaligned dw
    assert G(h, FAKE, 1 << 30, FAKE, 64, 40) == -2
    lib.spconv_nmap_destroy(h)


def test_build_batched_argument_checks(lib):
    _, a, w = sizes(lib, 1000, 27)
    h = ctypes.c_void_p()
    B = lambda coords, N, nb, K, d, arena, ab, ws, wb: lib.spconv_build_nmap_batched(
        ctypes.c_void_p(coords), N, nb, K, d, ctypes.c_void_p(arena), ab, ctypes.c_void_p(ws), wb, None,
        ctypes.byref(h))
    assert B(FAKE, 1000, 0, 27, 1, FAKE, a, FAKE, w) == -1          # no batches
    assert B(FAKE, 1000, -3, 27, 1, FAKE, a, FAKE, w) == -1
    assert B(FAKE, 1000, (1 << 20) + 1, 27, 1, FAKE, a, FAKE, w) == -2
    # 2^20 batches leave x-slabs of 2 values: too narrow for a 3x3x3 stencil
    assert B(FAKE, 1000, 1 << 20, 27, 1, FAKE, a, FAKE, w) == -2
    assert B(FAKE, 1000, 8, 26, 1, FAKE, a, FAKE, w) == -1          # K not an odd cube
    assert B(FAKE, 1000, 8, 27, 1, FAKE, a - 1, FAKE, w) == -5
    assert B(0, 1000, 8, 27, 1, FAKE, a, FAKE, w) == -1
    _, a0, _ = sizes(lib, 0, 27)
    assert B(0, 0, 8, 27, 1, FAKE, a0, 0, 0) == 0 and h.value      # empty set
    lib.spconv_nmap_destroy(h)
