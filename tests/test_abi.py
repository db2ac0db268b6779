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
            "moe_grouped_workspace_bytes"} <= set(names)
    L = pg.lib()
    for n in names:
        assert hasattr(L, n), n


def test_strerror_and_version(pg):
    assert pg.version().startswith("0.")
    for code in (0, -1, -2, -3, -4):
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
