"""gemv_q82 (the q8_2f format: int8 body, f16 row scales, f16 column field)
against the CPU oracle, through the C ABI: shapes that span several
workgroups and a ragged last one, columns that end inside a 1024-column step,
the four decode-frame shapes, the exact-integer case bit for bit, relu^2, and
the argument errors."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import TOL_Q8, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _dev_q82(pg, m):
    return pg.Q82Weight(to_dev(m.q, torch), torch.as_tensor(m.rs).cuda(), torch.as_tensor(m.cf).cuda())


@pytest.mark.parametrize("rows,cols", [(1024, 1024), (1000, 96), (37, 1040), (6144, 4096), (14336, 4096),
                                       (4096, 14336), (32000, 4096)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q82_parity(pg, oracle, rows, cols, act):
    _case(f"gemv_q82 {rows}x{cols} act={act}")
    rng = np.random.default_rng(rows + cols + act)
    m = synth.q82(rng, rows, cols)
    x = synth.normal(rng, cols)
    y = pg.gemv_q82(_dev_q82(pg, m), to_dev(x, torch), act=act)
    torch.cuda.synchronize()
    ref = oracle.gemm_q82(m.q, m.rs, m.cf, x, act=act)
    err = oracle.rel_err(y.cpu().numpy(), ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_Q8


def test_gemv_q82_exact_integer_case(pg, oracle):
    """Power-of-two row scales and column field, integer x: every f32 step is exact, so the
    device must equal the oracle bit for bit."""
    _case("gemv_q82 exact")
    rng = np.random.default_rng(5)
    rows, cols = 300, 2048
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    rs = (2.0 ** -rng.integers(2, 6, rows)).astype(np.float16)
    cf = (2.0 ** rng.integers(-1, 2, cols)).astype(np.float16)
    x = rng.integers(-8, 9, size=cols).astype(np.float32)
    y = pg.gemv_q82(_dev_q82(pg, synth.Q82(q, rs, cf)), to_dev(x, torch))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.gemm_q82(q, rs, cf, x))


def test_gemv_q82_errors(pg):
    _case("gemv_q82 errors")
    L = pg.lib()
    q = torch.zeros(64 * 1024, dtype=torch.int8, device="cuda")
    rs = torch.zeros(64, dtype=torch.float16, device="cuda")
    cf = torch.zeros(1024, dtype=torch.float16, device="cuda")
    x = torch.zeros(1024, device="cuda")
    y = torch.zeros(64, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(rows=64, cols=1024, qp=None, xp=None, cfp=None, act=0):
        return L.gemv_q82(qp or P(q), P(rs), cfp or P(cf), rows, cols, xp or P(x), P(y), act, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(cols=1000) == pg.PG_EUNSUPPORTED          # not a multiple of 16
    assert call(rows=0) == pg.PG_EINVAL
    assert call(act=2) == pg.PG_EINVAL
    assert call(qp=P(q, 4)) == pg.PG_EINVAL               # misaligned weights
    assert call(xp=P(x, 4)) == pg.PG_EINVAL               # misaligned x
    assert call(cfp=P(cf, 2)) == pg.PG_EINVAL             # column field not 8-byte aligned
    assert L.gemv_q82(None, P(rs), P(cf), 64, 1024, P(x), P(y), 0, s) == pg.PG_EINVAL
