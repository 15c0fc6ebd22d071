"""C ABI checks that need no GPU: the library loads, exports every symbol that
include/bakron.h declares, and rejects invalid arguments on the host before
enqueueing any work."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bakron.h")


@pytest.fixture(scope="module")
def lib():
    import kronecker_hessian_rounding_amd as bk
    return bk.LIB


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bakron_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_entry_points():
    names = declared_functions()
    for n in ("bakron_hessian_accum", "bakron_ldl", "bakron_solve"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    import kronecker_hessian_rounding_amd as bk
    names = declared_functions()
    assert set(names) == set(bk.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None
    # and through the dynamic symbol table
    out = os.popen("nm -D --defined-only %s" % bk.LIB_PATH).read()
    for n in names:
        assert re.search(r"\bT %s\b" % n, out), n


def test_version_and_status_strings(lib):
    assert lib.bakron_abi_version() == 1
    for s in range(5):
        assert lib.bakron_status_str(s)
    assert lib.bakron_status_str(99) == b"unknown status"


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first


def test_hessian_accum_rejects_bad_arguments(lib):
    f = lib.bakron_hessian_accum
    assert f(FAKE, 10, 0, 4, 1.0, 0.0, FAKE, 4, None, 0, None) == 1     # d <= 0
    assert f(FAKE, -1, 4, 4, 1.0, 0.0, FAKE, 4, None, 0, None) == 1     # T < 0
    assert f(None, 10, 4, 4, 1.0, 0.0, FAKE, 4, None, 0, None) == 1     # X NULL
    assert f(FAKE, 10, 4, 3, 1.0, 0.0, FAKE, 4, None, 0, None) == 1     # ldx < d
    assert f(FAKE, 10, 4, 4, 1.0, 0.0, FAKE, 3, None, 0, None) == 1     # ldh < d
    assert f(FAKE, 10, 4, 4, 1.0, 0.0, None, 4, None, 0, None) == 1     # H NULL
    assert lib.bakron_hessian_accum_workspace_bytes(10, 4) >= 0
    assert lib.bakron_hessian_accum_workspace_bytes(10, 0) == 0


def test_ldl_rejects_bad_arguments(lib):
    f = lib.bakron_ldl
    bad = ctypes.c_int64(7)
    ws_need = lib.bakron_ldl_workspace_bytes(100)
    assert ws_need >= 100 * 100 * 8
    assert f(None, 100, 100, 0.01, None, ctypes.byref(bad), FAKE, ws_need, None) == 1
    assert bad.value == -1
    assert f(FAKE, 0, 100, 0.01, None, None, FAKE, ws_need, None) == 1
    assert f(FAKE, 100, 99, 0.01, None, None, FAKE, ws_need, None) == 1
    assert f(FAKE, 100, 100, -0.5, None, None, FAKE, ws_need, None) == 1
    assert f(FAKE, 100, 100, float("nan"), None, None, FAKE, ws_need, None) == 1
    assert f(FAKE, 100, 100, 0.01, None, None, None, ws_need, None) == 3
    assert f(FAKE, 100, 100, 0.01, None, None, FAKE, ws_need - 1, None) == 3


def test_ldl_async_rejects_bad_arguments(lib):
    f = lib.bakron_ldl_async
    ws_need = lib.bakron_ldl_workspace_bytes(100)
    assert f(FAKE, 100, 100, 0.01, None, None, FAKE, ws_need, None) == 1   # status pointer NULL
    assert f(None, 100, 100, 0.01, None, FAKE, FAKE, ws_need, None) == 1   # H NULL
    assert f(FAKE, 0, 100, 0.01, None, FAKE, FAKE, ws_need, None) == 1     # d <= 0
    assert f(FAKE, 100, 99, 0.01, None, FAKE, FAKE, ws_need, None) == 1    # ldh < d
    assert f(FAKE, 100, 100, -0.5, None, FAKE, FAKE, ws_need, None) == 1   # damping < 0
    assert f(FAKE, 100, 100, 0.01, None, FAKE, None, ws_need, None) == 3   # no workspace
    assert f(FAKE, 100, 100, 0.01, None, FAKE, FAKE, ws_need - 1, None) == 3


def test_ldl_pair_async_rejects_bad_arguments(lib):
    f = lib.bakron_ldl_pair_async
    na, nb = lib.bakron_ldl_workspace_bytes(100), lib.bakron_ldl_workspace_bytes(60)
    ok = (FAKE, 100, 100, None, FAKE, FAKE, na, FAKE, 60, 60, None, FAKE, FAKE, nb, 0.01, None, None)

    def call(**kw):
        a = list(ok)
        names = ["HA", "dA", "ldha", "DA", "badA", "wsA", "wsA_bytes", "HB", "dB", "ldhb", "DB", "badB", "wsB",
                 "wsB_bytes", "damp", "sa", "sb"]
        for k, v in kw.items():
            a[names.index(k)] = v
        return f(*a)

    assert call(badA=None) == 1          # status pointers are required
    assert call(badB=None) == 1
    assert call(HA=None) == 1
    assert call(HB=None) == 1
    assert call(dA=0) == 1
    assert call(dB=-3) == 1
    assert call(ldha=99) == 1            # ldh < d
    assert call(ldhb=59) == 1
    assert call(damp=-0.5) == 1
    assert call(damp=float("inf")) == 1
    assert call(wsA=None) == 3           # workspace missing or short
    assert call(wsB_bytes=nb - 1) == 3


def test_solve_rejects_bad_arguments(lib):
    import kronecker_hessian_rounding_amd._binding as b
    f = lib.bakron_solve
    q = b._Quantizer(2, 0, 0, None)
    m, n = 70, 50
    need = lib.bakron_solve_workspace_bytes(m, n)
    assert need >= 2 * m * n * 4

    def call(W=FAKE, m=m, n=n, ldw=n, LO=FAKE, ldlo=m, LI=FAKE, ldli=n, qq=q, codes=FAKE, ldc=n,
             scales=FAKE, delta=None, ldd=n, DO=None, DI=None, loss=None, ws=FAKE, nb=need):
        return f(W, m, n, ldw, LO, ldlo, LI, ldli, ctypes.byref(qq) if qq is not None else None,
                 codes, ldc, scales, delta, ldd, DO, DI, loss, None, None, ws, nb, None)

    assert call(W=None) == 1
    assert call(m=0) == 1
    assert call(n=-3) == 1
    assert call(ldw=n - 1) == 1
    assert call(ldc=n - 1) == 1
    assert call(ldlo=m - 1) == 1
    assert call(ldli=n - 1) == 1
    assert call(codes=None) == 1
    assert call(scales=None) == 1
    assert call(qq=None) == 1
    assert call(delta=FAKE, ldd=n - 1) == 1
    assert call(qq=b._Quantizer(0, 0, 0, None)) == 1
    assert call(qq=b._Quantizer(9, 0, 0, None)) == 1
    assert call(qq=b._Quantizer(2, 2, 0, None)) == 1
    assert call(loss=FAKE) == 1                       # D_I missing
    assert call(loss=FAKE, DI=FAKE) == 1              # D_O missing with L_O given
    assert call(ws=None) == 3
    assert call(nb=need - 1) == 3
    assert lib.bakron_solve_workspace_bytes(0, 5) == 0


def test_rht_rejects_invalid_arguments(lib):
    # host-side checks only: every call below returns before any launch
    f = lib.bakron_rht
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_uint64, ctypes.c_int, ctypes.c_void_p]
    f.restype = ctypes.c_int
    INVALID = 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the arguments fail first
    assert f(None, 4, 4, 4, 0, 1, 0, None) == INVALID
    assert f(fake, 0, 4, 4, 0, 1, 0, None) == INVALID
    assert f(fake, 4, 0, 4, 1, 1, 0, None) == INVALID
    assert f(fake, 4, 8, 7, 0, 1, 0, None) == INVALID  # lda < cols
    assert f(fake, 4, 8, 8, 2, 1, 0, None) == INVALID  # no such axis
    assert f(fake, 4, 32768, 32768, 1, 1, 0, None) == INVALID  # row blocks above 16384


def test_hessian_accum_t_rejects_invalid_arguments(lib):
    f = lib.bakron_hessian_accum_t
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_float,
                  ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    INVALID, WORKSPACE = 1, 3
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the arguments fail first
    assert f(fake, 16, 8, 15, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # ldx < T
    assert f(fake, 16, 0, 16, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # d <= 0
    assert f(None, 16, 8, 16, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # X missing
    assert f(fake, 16, 8, 16, 1.0, 0.0, fake, 8, None, 0, None) == WORKSPACE      # no workspace


def test_layer_report_rejects_invalid_arguments(lib):
    f = lib.bakron_layer_report
    f.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                  ctypes.c_void_p]
    f.restype = ctypes.c_int
    INVALID = 1
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the arguments fail first
    assert f(0, 4, fake, fake, fake, None, 0, None, 0, fake, None) == INVALID
    assert f(4, 4, fake, None, fake, None, 0, None, 0, fake, None) == INVALID   # no D_I
    assert f(4, 4, fake, fake, None, None, 0, None, 0, fake, None) == INVALID   # no scales
    assert f(4, 4, fake, fake, fake, None, 0, None, 0, None, None) == INVALID   # no out
    assert f(4, 8, fake, fake, fake, fake, 7, None, 0, fake, None) == INVALID   # ld(H_I) < n


def test_sketch_a_entry_points_reject_invalid_arguments(lib):
    fw = lib.bakron_token_weights
    fw.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    fw.restype = ctypes.c_int
    fa = lib.bakron_hessian_accum_w
    fa.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                   ctypes.c_size_t, ctypes.c_void_p]
    fa.restype = ctypes.c_int
    INVALID, WORKSPACE = 1, 3
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the arguments fail first
    assert fw(fake, 10, 0, 4, None, 0, fake, None, 0, None) == INVALID       # d <= 0
    assert fw(fake, 10, 4, 3, None, 0, fake, None, 0, None) == INVALID       # ldy < d
    assert fw(fake, 10, 4, 4, fake, 3, fake, None, 0, None) == INVALID       # ldh < d
    assert fw(fake, 10, 4, 4, fake, 4, fake, None, 0, None) == WORKSPACE     # H given, no workspace
    assert fa(fake, 10, 4, 4, None, 1.0, 0.0, fake, 4, fake, 1 << 30, None) == INVALID  # no weights
    assert fa(fake, 10, 4, 4, fake, 1.0, 0.0, fake, 4, None, 0, None) == WORKSPACE
    assert lib.bakron_token_weights_workspace_bytes(10, 0) == 0


def test_hessian_accum_tb_rejects_invalid_arguments(lib):
    f = lib.bakron_hessian_accum_tb
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_float, ctypes.c_float, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    f.restype = ctypes.c_int
    INVALID, WORKSPACE = 1, 3
    fake = ctypes.c_void_p(0x1000)  # never dereferenced: the arguments fail first
    assert f(fake, 2, 8, 16, 15, 128, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # ldx < tin
    assert f(fake, 2, 8, 16, 16, 127, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # batches overlap
    assert f(fake, 2, 0, 16, 16, 128, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # d <= 0
    assert f(fake, -1, 8, 16, 16, 128, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # S < 0
    assert f(None, 2, 8, 16, 16, 128, 1.0, 0.0, fake, 8, fake, 1 << 30, None) == INVALID  # X missing
    assert f(fake, 2, 8, 16, 16, 128, 1.0, 0.0, fake, 7, fake, 1 << 30, None) == INVALID  # ldh < d
    assert f(fake, 2, 8, 16, 16, 128, 1.0, 0.0, fake, 8, None, 0, None) == WORKSPACE      # no workspace


def test_sketch_b_checks_arguments_before_any_launch(monkeypatch):
    # invalid gradients (host tensors here) are rejected before the library is called
    import torch

    import kronecker_hessian_rounding_amd as bk

    calls = []

    class Spy:
        def __getattr__(self, name):
            calls.append(name)
            raise AssertionError("library called: " + name)

    monkeypatch.setattr(bk._binding, "LIB", Spy())
    with pytest.raises(ValueError):
        bk.sketch_b(torch.zeros((2, 8, 16)))
    with pytest.raises(ValueError):
        bk.sketch_b([])
    assert calls == []


def test_solve_noalloc_rejects_bad_arguments_and_oversize_shapes(lib):
    # validated on the host before the library's scratch array is touched: the same
    # argument errors as bakron_solve, and BAKRON_E_WORKSPACE for shapes whose
    # workspace exceeds the scratch array
    import kronecker_hessian_rounding_amd as bk

    q = bk._binding._Quantizer(2, 0, 0, None)
    f = lib.bakron_solve_noalloc
    args = lambda m, n, qq: (FAKE, m, n, n, FAKE, m, FAKE, n, qq, FAKE, n, FAKE, None, n, None, None, None,
                             None, None, None)
    assert f(*args(0, 64, ctypes.byref(q))) == 1
    assert f(*args(64, 64, None)) == 1
    bad = bk._binding._Quantizer(9, 0, 0, None)
    assert f(*args(64, 64, ctypes.byref(bad))) == 1
    assert lib.bakron_solve_workspace_bytes(4096, 4096) > bk.NOALLOC_SCRATCH_BYTES
    assert f(*args(4096, 4096, ctypes.byref(q))) == 3
    assert lib.bakron_solve_workspace_bytes(2048, 2048) <= bk.NOALLOC_SCRATCH_BYTES
    assert lib.bakron_solve_workspace_bytes(1024, 3072) <= bk.NOALLOC_SCRATCH_BYTES
    assert lib.bakron_solve_workspace_bytes(1024, 4096) > bk.NOALLOC_SCRATCH_BYTES
