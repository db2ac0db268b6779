"""prefill_gemm_q4tp (the pages' 4-bit format on the matrix cores) against the
CPU oracle through the C ABI: position counts 1..64 and ragged shapes, K
splits, the decode frame's four shapes sampled, relu^2, bit-exact cases (every
5-bit code value, codes straddling two code bytes, and a whole product with
small power-of-two scales), agreement with gemv_q4tp, and argument errors."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import TOL_Q8, int_acts, to_dev

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


def _pack_codes(codes5):
    """5-bit group codes [rows][groups] -> code bytes [rows][ceil(5 groups / 8)], code g at
    bits 5 g .. 5 g + 4 of the row, least significant bit first."""
    rows, groups = codes5.shape
    out = np.zeros((rows, (5 * groups + 7) // 8), np.uint8)
    for g in range(groups):
        for b in range(5):
            bit = 5 * g + b
            out[:, bit // 8] |= (((codes5[:, g] >> b) & 1) << (bit % 8)).astype(np.uint8)
    return out


def _params(base, step):
    return (base.astype(np.float16).view(np.uint16).astype(np.uint32)
            | (step.astype(np.float16).view(np.uint16).astype(np.uint32) << 16))


@pytest.mark.parametrize("rows,cols,n", [(1024, 1024, 1), (1000, 96, 33), (37, 2080, 64), (300, 14336, 7),
                                         (640, 4096, 64), (4096, 1024, 17)])
@pytest.mark.parametrize("act", [0, 1])
def test_prefill_q4tp_parity(pg, oracle, rows, cols, n, act):
    _case(f"prefill_gemm_q4tp {rows}x{cols} n={n} act={act}")
    rng = np.random.default_rng(rows + cols + n + act)
    m = synth.q4tp(rng, rows, cols)
    X = synth.normal(rng, (n, cols))
    Y = pg.prefill_gemm_q4tp(_dev_q4(pg, m), to_dev(X, torch), act=act)
    torch.cuda.synchronize()
    err = oracle.rel_err(Y.cpu().numpy(), oracle.gemm_q4tp(m.nib, m.params, m.codes, X, act=act))
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_Q8


@pytest.mark.parametrize("rows,cols", [(6144, 4096), (14336, 4096), (4096, 14336), (32000, 4096)])
def test_prefill_q4tp_frame_shapes_sampled(pg, oracle, rows, cols):
    """The decode frame's four shapes at 64 positions; 300 sampled rows against the oracle."""
    _case(f"prefill_gemm_q4tp frame shape {rows}x{cols}")
    rng = np.random.default_rng(rows * 7 + cols)
    m = synth.q4tp(rng, rows, cols)
    X = synth.normal(rng, (64, cols))
    Y = pg.prefill_gemm_q4tp(_dev_q4(pg, m), to_dev(X, torch)).cpu().numpy()
    idx = np.unique(rng.choice(rows, 300, replace=False))
    ref = oracle.gemm_q4tp(m.nib[idx], m.params[idx], m.codes[idx], X)
    err = oracle.rel_err(Y[:, idx], ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_Q8


@pytest.mark.parametrize("cols,group,n", [(32, 0, 64), (256, 1, 40), (256, 3, 64), (2080, 64, 9), (4096, 101, 64)])
def test_prefill_q4tp_exact_one_group(pg, oracle, cols, group, n):
    """Integer base, step 1 and integer x that is zero outside one group: each output is 2^(base
    + code) times an integer, exact in f32 on both sides, so they must agree bit for bit; over
    3000 rows every code value of the group's field is met (groups 1 and 3 straddle two code
    bytes; group 64 is in a row's last code byte)."""
    _case(f"prefill_gemm_q4tp exact one group cols={cols} group={group} n={n}")
    rng = np.random.default_rng(cols + group + n)
    rows = 3000
    m = synth.q4tp(rng, rows, cols)
    m.params = _params(rng.integers(-24, -8, rows), np.ones(rows))
    X = np.zeros((n, cols), np.float32)
    X[:, 32 * group:32 * group + 32] = rng.integers(-8, 9, (n, 32))
    Y = pg.prefill_gemm_q4tp(_dev_q4(pg, m), to_dev(X, torch))
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), oracle.gemm_q4tp(m.nib, m.params, m.codes, X))


@pytest.mark.parametrize("rows,cols,n", [(500, 4096, 64), (256, 14336, 20)])
def test_prefill_q4tp_exact_whole_product(pg, oracle, rows, cols, n):
    """Codes 0..3 with base -6 and step 1 (scales 2^-6 .. 2^-3) and integer x: every partial sum,
    the -8 scale offset term included, is a multiple of 2^-6 below 2^18, so the whole product
    (K splits too) is exact: bit for bit."""
    _case(f"prefill_gemm_q4tp exact {rows}x{cols} n={n}")
    rng = np.random.default_rng(rows + cols)
    m = synth.q4tp(rng, rows, cols)
    m.codes = _pack_codes(rng.integers(0, 4, (rows, cols // 32)))
    m.params = _params(np.full(rows, -6.0), np.ones(rows))
    X = int_acts(rng, (n, cols), lim=8)
    Y = pg.prefill_gemm_q4tp(_dev_q4(pg, m), to_dev(X, torch))
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), oracle.gemm_q4tp(m.nib, m.params, m.codes, X))


def test_prefill_q4tp_rows_match_gemv(pg, oracle):
    """Each position of the pass against gemv_q4tp on that position (same group scales).  The
    two differ by the prefill's operand rounding: x as bf16 hi + lo (2^-17) and the offset term
    -8 scale sum x, about twice a group's own sum, taken with both factors as bf16 hi + lo;
    2e-4 of the output RMS bounds that with room."""
    _case("prefill_gemm_q4tp vs gemv_q4tp")
    rng = np.random.default_rng(41)
    m = synth.q4tp(rng, 700, 2048)
    W = _dev_q4(pg, m)
    X = to_dev(synth.normal(rng, (12, 2048)), torch)
    Y = pg.prefill_gemm_q4tp(W, X)
    for b in range(12):
        y = pg.gemv_q4tp(W, X[b].contiguous())
        torch.cuda.synchronize()
        err = oracle.rel_err(Y[b].cpu().numpy(), y.cpu().numpy())
        print(f"[info] position {b}: prefill vs gemv {err:.2e}", flush=True)
        assert err <= 2e-4


def test_prefill_q4tp_errors(pg):
    _case("prefill_gemm_q4tp errors")
    L = pg.lib()
    rows, cols, n = 64, 1024, 8
    nib = torch.zeros(rows * cols // 2, dtype=torch.uint8, device="cuda")
    params = torch.zeros(rows + 1, dtype=torch.int32, device="cuda")
    codes = torch.zeros(rows * 20 + 4, dtype=torch.uint8, device="cuda")
    X = torch.zeros(n * cols + 4, device="cuda")
    Y = torch.zeros(n * rows, device="cuda")
    ws = torch.empty(pg.prefill_gemm_q8_workspace_bytes(rows, cols, n), dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(rows=rows, cols=cols, nn=n, np_=None, pp=None, cp=None, act=0, wsb=ws.numel()):
        return L.prefill_gemm_q4tp(np_ or P(nib), pp or P(params), cp or P(codes), rows, cols, P(X), nn, P(Y), act,
                                   P(ws), wsb, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(cols=1008) == pg.PG_EUNSUPPORTED
    assert call(nn=65) == pg.PG_EUNSUPPORTED
    assert call(rows=0) == pg.PG_EINVAL
    assert call(act=2) == pg.PG_EINVAL
    assert call(np_=P(nib, 8)) == pg.PG_EINVAL       # nibbles not 16-byte aligned
    assert call(pp=P(params, 2)) == pg.PG_EINVAL     # params not 4-byte aligned
    assert call(cp=P(codes, 2)) == pg.PG_EINVAL      # codes not 4-byte aligned
    assert call(wsb=ws.numel() - 256) == pg.PG_EWORKSPACE
