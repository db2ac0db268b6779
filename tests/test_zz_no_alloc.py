"""prefill_gemm_q8_noalloc: the prefill product with the library's fixed device
scratch array instead of a workspace, through the C ABI, against the
workspace-taking prefill_gemm_q8 (same kernels, so bit for bit) and the
oracle: two calls in a row, the second on a smaller input, then the largest
product of the hidden-4096 layer frame (4096 x 14336 at 64 positions)."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import TOL_Q8, q8_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _noalloc(pg, W, X, act):
    """Call the entry point through the C ABI with a caller-allocated output."""
    n = X.shape[0]
    Y = torch.empty(n, W.rows, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = pg.lib().prefill_gemm_q8_noalloc(ctypes.c_void_p(W.q.data_ptr()), ctypes.c_void_p(W.scale.data_ptr()),
                                          ctypes.c_void_p(W.bias.data_ptr()), W.rows, W.cols,
                                          ctypes.c_void_p(X.data_ptr()), n, ctypes.c_void_p(Y.data_ptr()), act, s)
    assert rc == pg.PG_OK, pg.strerror(rc)
    return Y


@pytest.mark.parametrize("shapes", [[(640, 4096, 64, 1), (300, 2048, 5, 0)],
                                    [(4096, 14336, 64, 0), (1000, 1024, 1, 1)]])
def test_noalloc_matches_workspace_call(pg, oracle, shapes):
    for i, (rows, cols, n, act) in enumerate(shapes):
        _case(f"prefill_gemm_q8_noalloc call {i}: {rows}x{cols} n={n} act={act}")
        rng = np.random.default_rng(rows + n)
        m = synth.q8(rng, rows, cols)
        X = synth.normal(rng, (n, cols))
        W, Xd = q8_dev(m, torch), to_dev(X, torch)
        Y = _noalloc(pg, W, Xd, act)
        Y_ws = pg.prefill_gemm_q8(W, Xd, act=act)
        torch.cuda.synchronize()
        assert torch.equal(Y, Y_ws)
        idx = np.unique(rng.choice(rows, min(rows, 256), replace=False))
        ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, X, act=act)
        assert oracle.rel_err(Y.cpu().numpy()[:, idx], ref) <= TOL_Q8


def test_noalloc_rejects_beyond_scratch(pg):
    """A product whose workspace would exceed the fixed array is refused before launch."""
    _case("prefill_gemm_q8_noalloc size limit")
    rows, cols, n = 4096, 65536, 64
    assert pg.prefill_gemm_q8_workspace_bytes(rows, cols, n) > 16 << 20
    fake = ctypes.c_void_p(0x100000)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert pg.lib().prefill_gemm_q8_noalloc(fake, fake, fake, rows, cols, fake, n, fake, 0, s) == pg.PG_EUNSUPPORTED
