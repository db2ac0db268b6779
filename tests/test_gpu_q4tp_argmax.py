"""gemv_q4tp (the pages' 4-bit format) and argmax_rows against the CPU oracle,
through the C ABI: several workgroups and a ragged last one, columns that end
inside a 64-group step, the decode frame's shapes, bit-exact cases that check
every code field (including those straddling two code bytes), relu^2; argmax
with planted ties, NaN, -inf and floor rows, the vector and the scalar path,
and the argument errors."""
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


def _dev_q4(pg, m):
    return pg.Q4TPWeight(to_dev(m.nib, torch), to_dev(m.params.view(np.int32), torch), to_dev(m.codes, torch))


@pytest.mark.parametrize("rows,cols", [(1024, 1024), (1000, 96), (37, 2080), (6144, 4096), (14336, 4096),
                                       (4096, 14336), (32000, 4096), (8, 32768)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q4tp_parity(pg, oracle, rows, cols, act):
    _case(f"gemv_q4tp {rows}x{cols} act={act}")
    rng = np.random.default_rng(rows + 3 * cols + act)
    m = synth.q4tp(rng, rows, cols)
    x = synth.normal(rng, cols)
    y = pg.gemv_q4tp(_dev_q4(pg, m), to_dev(x, torch), act=act)
    torch.cuda.synchronize()
    ref = oracle.gemm_q4tp(m.nib, m.params, m.codes, x, act=act)
    err = oracle.rel_err(y.cpu().numpy(), ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_Q8


@pytest.mark.parametrize("cols,group", [(32, 0), (64, 1), (256, 3), (256, 7), (2080, 64)])
def test_gemv_q4tp_exact_one_group(pg, oracle, cols, group):
    """Integer base and step 1 with integer x that is zero outside one group: the result is
    2^(base + code) times an integer, exact in f32, so the device must equal the oracle bit for
    bit; over 3000 rows this checks the chosen group's code field for every code value (groups
    1 and 3 straddle two code bytes; group 64 is the last of a ragged step and its code sits in
    the row's last code byte)."""
    _case(f"gemv_q4tp exact cols={cols} group={group}")
    rng = np.random.default_rng(cols + group)
    rows = 3000
    m = synth.q4tp(rng, rows, cols)
    base = rng.integers(-24, -8, rows).astype(np.float16)
    step = np.ones(rows, np.float16)
    m.params = (base.view(np.uint16).astype(np.uint32) | (step.view(np.uint16).astype(np.uint32) << 16))
    x = np.zeros(cols, np.float32)
    x[32 * group:32 * group + 32] = rng.integers(-8, 9, 32)
    y = pg.gemv_q4tp(_dev_q4(pg, m), to_dev(x, torch))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.gemm_q4tp(m.nib, m.params, m.codes, x))


def test_gemv_q4tp_errors(pg):
    _case("gemv_q4tp errors")
    L = pg.lib()
    rows, cols = 64, 1024
    nib = torch.zeros(rows * cols // 2, dtype=torch.uint8, device="cuda")
    params = torch.zeros(rows + 1, dtype=torch.int32, device="cuda")
    codes = torch.zeros(rows * 20, dtype=torch.uint8, device="cuda")
    x = torch.zeros(cols + 4, device="cuda")
    y = torch.zeros(rows, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(rows=rows, cols=cols, np_=None, pp=None, xp=None, act=0):
        return L.gemv_q4tp(np_ or P(nib), pp or P(params), P(codes), rows, cols, xp or P(x), P(y), act, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(cols=1008) == pg.PG_EUNSUPPORTED          # not a multiple of 32
    assert call(cols=32800) == pg.PG_EUNSUPPORTED
    assert call(rows=0) == pg.PG_EINVAL
    assert call(act=2) == pg.PG_EINVAL
    assert call(np_=P(nib, 8)) == pg.PG_EINVAL            # nibbles not 16-byte aligned
    assert call(pp=P(params, 2)) == pg.PG_EINVAL          # params not 4-byte aligned
    assert call(xp=P(x, 4)) == pg.PG_EINVAL
    assert L.gemv_q4tp(P(nib), P(params), None, rows, cols, P(x), P(y), 0, s) == pg.PG_EINVAL


# ------------------------------------------------------------------ argmax

def _plant(rng, L):
    """Ties, NaN, -inf and floor rows on a logits matrix (in place)."""
    n, V = L.shape
    for b in range(0, n, 2):                      # the row maximum repeated at later indices
        L[b, rng.choice(V, min(3, V), replace=False)] = L[b].max()
    if n > 3:
        L[1, ::7] = np.nan
        L[3, :] = -np.inf
    if n > 5:
        L[5, :] = np.float32(-3.0e38)
        L[5, V - 1] = np.float32(-2.9e38)
    return L


@pytest.mark.parametrize("n,vocab", [(1, 32000), (64, 32000), (7, 262144), (9, 50257), (4, 1), (6, 5),
                                     (64, 4096)])
def test_argmax_parity(pg, oracle, n, vocab):
    _case(f"argmax n={n} vocab={vocab}")
    rng = np.random.default_rng(n * 31 + vocab)
    L = _plant(rng, synth.logits(rng, n, vocab))
    ids = pg.argmax_rows(to_dev(L, torch))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy().astype(np.uint32), oracle.argmax_rows(L))


def test_argmax_scalar_path_misaligned(pg, oracle):
    """A row base 4 bytes off a 16-byte boundary takes the scalar path and chooses the same."""
    _case("argmax misaligned")
    rng = np.random.default_rng(77)
    n, vocab = 5, 4000
    L = _plant(rng, synth.logits(rng, n, vocab))
    buf = torch.empty(n * vocab + 1, device="cuda")
    buf[1:] = to_dev(L.reshape(-1), torch)
    ids = torch.empty(n, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = pg.lib().argmax_rows(ctypes.c_void_p(buf.data_ptr() + 4), n, vocab, ctypes.c_void_p(ids.data_ptr()), s)
    assert rc == pg.PG_OK
    torch.cuda.synchronize()
    np.testing.assert_array_equal(ids.cpu().numpy().astype(np.uint32), oracle.argmax_rows(L))


def test_argmax_errors(pg):
    _case("argmax errors")
    L = pg.lib()
    logits = torch.zeros(4 * 100, device="cuda")
    ids = torch.zeros(4, dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)
    assert L.argmax_rows(P(logits), 4, 100, P(ids), s) == pg.PG_OK
    torch.cuda.synchronize()
    assert L.argmax_rows(P(logits), 0, 100, P(ids), s) == pg.PG_EINVAL
    assert L.argmax_rows(P(logits), 4, 0, P(ids), s) == pg.PG_EINVAL
    assert L.argmax_rows(P(logits, 2), 4, 100, P(ids), s) == pg.PG_EINVAL
    assert L.argmax_rows(P(logits), 4, 100, P(logits, 16), s) == pg.PG_EINVAL   # ids inside the logits
    assert L.argmax_rows(None, 4, 100, P(ids), s) == pg.PG_EINVAL
