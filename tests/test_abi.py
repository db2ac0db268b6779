"""The C ABI without a GPU: the library loads, exports every declared symbol,
and the host-side argument checks return their codes before any launch."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "pg.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    return pg


def test_exports_every_declared_symbol(pg):
    names = declared_functions()
    assert {"gemv_q8", "gemv_f16", "prefill_gemm_q8", "add_rmsnorm", "moe_grouped",
            "pg_strerror", "pg_version", "prefill_gemm_q8_workspace_bytes",
            "moe_grouped_workspace_bytes", "gemv_q8_addnorm", "prefill_gemm_q8_addnorm"} <= set(names)
    L = pg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_version(pg):
    assert pg.version().startswith("0.")
    for code in (0, -1, -2, -3, -4, -5):
        assert pg.strerror(code)
    assert pg.strerror(7) == "unknown status"


def test_workspace_queries(pg):
    n, rows, cols = 64, 6144, 4096
    ws = pg.prefill_gemm_q8_workspace_bytes(rows, cols, n)
    assert ws >= (n + 1) * cols * 4
    assert pg.prefill_gemm_q8_workspace_bytes(rows, 100, n) == 0
    assert pg.moe_grouped_workspace_bytes(64, 2688, 1856, 128, 6) >= 64 * 6 * (2688 + 1856) * 4
    assert pg.moe_grouped_workspace_bytes(64, 2688, 1850, 128, 6) == 0


FAKE = ctypes.c_void_p(0x100000)      # aligned, never dereferenced: every call below returns early
ODD = ctypes.c_void_p(0x100004)


def test_argument_checks_return_before_launch(pg):
    L = pg.lib()
    # null pointer / bad sizes
    assert L.gemv_q8(None, FAKE, FAKE, 8, 64, FAKE, FAKE, 0, None) == pg.PG_EINVAL
    assert L.gemv_q8(FAKE, FAKE, FAKE, 0, 64, FAKE, FAKE, 0, None) == pg.PG_EINVAL
    assert L.gemv_q8(FAKE, FAKE, FAKE, 8, 64, FAKE, FAKE, 2, None) == pg.PG_EINVAL
    assert L.gemv_q8(ODD, FAKE, FAKE, 8, 64, FAKE, FAKE, 0, None) == pg.PG_EINVAL
    # y overlapping x (workgroups write y while others still read x)
    assert L.gemv_q8(FAKE, FAKE, FAKE, 64, 64, FAKE, FAKE, 0, None) == pg.PG_EINVAL
    assert L.gemv_f16(FAKE, 64, 64, FAKE, ctypes.c_void_p(0x100000 + 128), 0, None) == pg.PG_EINVAL
    assert L.decode_frame_q8_status(None, 4096, None) == pg.PG_EWORKSPACE
    # the allocation-free prefill product: argument checks and its scratch limit
    assert L.prefill_gemm_q8_noalloc(None, FAKE, FAKE, 8, 64, FAKE, 4, FAKE, 0, None) == pg.PG_EINVAL
    assert L.prefill_gemm_q8_noalloc(FAKE, FAKE, FAKE, 8, 64, FAKE, 65, FAKE, 0, None) == pg.PG_EUNSUPPORTED
    assert L.prefill_gemm_q8_noalloc(FAKE, FAKE, FAKE, 4096, 65536, FAKE, 64, FAKE, 0, None) == pg.PG_EUNSUPPORTED
    assert L.gemv_q8(FAKE, FAKE, FAKE, 8, 48, FAKE, FAKE, 0, None) == pg.PG_EUNSUPPORTED
    assert L.gemv_q8(FAKE, FAKE, FAKE, 8, 65536, FAKE, FAKE, 0, None) == pg.PG_EUNSUPPORTED
    assert L.gemv_f16(FAKE, 8, 12, FAKE, FAKE, 0, None) == pg.PG_EUNSUPPORTED
    assert L.gemv_f16(None, 8, 16, FAKE, FAKE, 0, None) == pg.PG_EINVAL
    # prefill: n range, width, workspace
    assert L.prefill_gemm_q8(FAKE, FAKE, FAKE, 8, 64, FAKE, 65, FAKE, 0, FAKE, 1 << 30, None) == pg.PG_EUNSUPPORTED
    assert L.prefill_gemm_q8(FAKE, FAKE, FAKE, 8, 40, FAKE, 4, FAKE, 0, FAKE, 1 << 30, None) == pg.PG_EUNSUPPORTED
    assert L.prefill_gemm_q8(FAKE, FAKE, FAKE, 8, 64, FAKE, 0, FAKE, 0, FAKE, 1 << 30, None) == pg.PG_EINVAL
    assert L.prefill_gemm_q8(FAKE, FAKE, FAKE, 8, 64, FAKE, 4, FAKE, 0, FAKE, 16, None) == pg.PG_EWORKSPACE
    assert L.prefill_gemm_q8(FAKE, FAKE, FAKE, 8, 64, FAKE, 4, FAKE, 0, None, 1 << 30, None) == pg.PG_EWORKSPACE
    # add_rmsnorm: hidden limits, stride, aliasing
    assert L.add_rmsnorm(FAKE, None, 0, FAKE, 1e-6, 18, 1, ctypes.c_void_p(0x200000), None) == pg.PG_EUNSUPPORTED
    assert L.add_rmsnorm(FAKE, None, 0, FAKE, 1e-6, 32768, 1, ctypes.c_void_p(0x900000), None) == pg.PG_EUNSUPPORTED
    assert L.add_rmsnorm(FAKE, FAKE, 8, FAKE, 1e-6, 16, 1, ctypes.c_void_p(0x200000), None) == pg.PG_EINVAL
    assert L.add_rmsnorm(FAKE, None, 0, FAKE, 1e-6, 16, 4, ctypes.c_void_p(0x100010), None) == pg.PG_EINVAL
    # moe: limits
    args = lambda n, H, E, k, I: (FAKE, n, H, FAKE, E, k, 0, FAKE, FAKE, FAKE, I, FAKE, FAKE, FAKE,
                                  FAKE, FAKE, ctypes.c_float(1e-6), ctypes.c_void_p(0x300000), FAKE, FAKE,
                                  FAKE, FAKE, FAKE, FAKE, ctypes.c_size_t(1 << 40), None)
    assert L.moe_grouped(*args(65, 64, 8, 2, 64)) == pg.PG_EUNSUPPORTED
    assert L.moe_grouped(*args(4, 48, 8, 2, 64)) == pg.PG_EUNSUPPORTED
    assert L.moe_grouped(*args(4, 64, 8, 9, 64)) == pg.PG_EUNSUPPORTED
    assert L.moe_grouped(*args(4, 64, 2000, 2, 64)) == pg.PG_EUNSUPPORTED
    assert L.moe_grouped(*args(4, 64, 8, 17, 64)) == pg.PG_EUNSUPPORTED
    assert L.moe_grouped(*args(4, 64, 8, 0, 64)) == pg.PG_EINVAL


def test_fused_norm_argument_checks(pg):
    L = pg.lib()
    f = ctypes.c_float
    A, B, C, D, E = (ctypes.c_void_p(a) for a in (0x100000, 0x200000, 0x300000, 0x400000, 0x500000))
    # gemv_q8_addnorm(q, scale, bias, rows, cols, h, delta, w, eps, h_out, x_out, y, act, stream)
    g = lambda h, d, w, eps, ho, xo, y, rows=8, cols=64, act=0: L.gemv_q8_addnorm(
        FAKE, FAKE, FAKE, rows, cols, h, d, w, f(eps), ho, xo, y, act, None)
    assert g(None, None, B, 1e-6, None, None, C) == pg.PG_EINVAL
    assert g(A, None, B, -1.0, None, None, C) == pg.PG_EINVAL
    assert g(A, None, B, float("nan"), None, None, C) == pg.PG_EINVAL
    assert g(A, ODD, B, 1e-6, None, None, C) == pg.PG_EINVAL
    assert g(A, None, B, 1e-6, None, None, C, cols=48) == pg.PG_EUNSUPPORTED
    assert g(A, None, B, 1e-6, A, None, C) == pg.PG_EINVAL          # h_out aliases h
    assert g(A, D, B, 1e-6, ctypes.c_void_p(0x400010), None, C) == pg.PG_EINVAL   # h_out overlaps delta
    assert g(A, None, B, 1e-6, None, B, C) == pg.PG_EINVAL          # x_out aliases w
    assert g(A, None, B, 1e-6, D, D, C) == pg.PG_EINVAL             # h_out aliases x_out
    assert g(A, None, B, 1e-6, None, None, A) == pg.PG_EINVAL       # y aliases h
    assert g(A, None, B, 1e-6, None, None, C, act=3) == pg.PG_EINVAL
    # prefill_gemm_q8_addnorm(q, scale, bias, rows, cols, H, delta, stride, w, eps, n, H_out, X_out, Y, act, ws, wsb, s)
    big = ctypes.c_size_t(1 << 30)
    WS = ctypes.c_void_p(0x10000000)
    p = lambda H, d, st, w, n, Ho, Xo, Y, cols=64, wsb=big, ws=WS: L.prefill_gemm_q8_addnorm(
        FAKE, FAKE, FAKE, 8, cols, H, d, st, w, f(1e-6), n, Ho, Xo, Y, 0, ws, wsb, None)
    assert p(A, None, 0, B, 65, None, None, C) == pg.PG_EUNSUPPORTED
    assert p(A, None, 0, B, 4, None, None, C, cols=32768) == pg.PG_EUNSUPPORTED
    assert p(A, D, 32, B, 4, None, None, C) == pg.PG_EINVAL          # stride < cols
    assert p(A, D, 66, B, 4, None, None, C) == pg.PG_EINVAL          # stride % 4
    assert p(A, None, 0, B, 4, None, None, C, wsb=ctypes.c_size_t(16)) == pg.PG_EWORKSPACE
    assert p(A, None, 0, B, 4, ctypes.c_void_p(0x100100), None, C) == pg.PG_EINVAL   # H_out overlaps H, not equal
    assert p(A, None, 0, B, 4, None, A, C) == pg.PG_EINVAL           # X_out aliases H
    assert p(A, None, 0, B, 4, D, D, C) == pg.PG_EINVAL              # H_out aliases X_out
    assert p(A, None, 0, B, 4, None, None, WS) == pg.PG_EINVAL       # Y inside the workspace


def test_residual_pair_argument_checks(pg):
    L = pg.lib()
    f = ctypes.c_float
    X, Y, H, Wn, HO, XW, PT = (ctypes.c_void_p(a) for a in
                               (0x100000, 0x200000, 0x300000, 0x400000, 0x500000, 0x600000, 0x700000))
    r = lambda rows=16, cols=64, hidden=8, x=X, y=Y, h=H, ho=HO, xw=XW, pt=PT, act=0: L.gemv_q8_residual(
        FAKE, FAKE, FAKE, rows, cols, x, y, act, h, Wn, hidden, ho, xw, pt, None)
    assert r(hidden=17) == pg.PG_EINVAL                 # hidden > rows
    assert r(xw=None) == pg.PG_EINVAL
    assert r(cols=48) == pg.PG_EUNSUPPORTED
    assert r(y=X) == pg.PG_EINVAL                       # y aliases x
    assert r(ho=ctypes.c_void_p(0x300010)) == pg.PG_EINVAL   # h_out overlaps h without being h
    assert r(xw=PT) == pg.PG_EINVAL                     # xw aliases parts
    assert r(pt=ctypes.c_void_p(0x200004)) == pg.PG_EINVAL   # parts overlaps y
    n = lambda cols=64, xw=XW, pt=PT, y=Y, eps=1e-6: L.gemv_q8_normed(FAKE, FAKE, FAKE, 16, cols, xw, pt, f(eps), y, 0,
                                                                      None)
    assert n(eps=-1.0) == pg.PG_EINVAL
    assert n(y=XW) == pg.PG_EINVAL
    assert n(y=PT) == pg.PG_EINVAL
    assert n(cols=40) == pg.PG_EUNSUPPORTED
