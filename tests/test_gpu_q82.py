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


def _plant_m128(rng, q):
    """q = -128 (outside the generator's range; the int8 body decodes it as -128) on the
    first row and on 2% of the entries."""
    q[0, :] = -128
    q[rng.random(q.shape) < 0.02] = -128
    return q


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
    q = _plant_m128(rng, rng.integers(-127, 128, size=(rows, cols), dtype=np.int8))
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


# ------------------------------------------------------------------ prefill_gemm_q82

@pytest.mark.parametrize("rows,cols,n", [(128, 512, 1), (300, 1056, 33), (37, 96, 64), (1000, 4096, 64),
                                         (4096, 1024, 17), (2048, 14336, 64)])
@pytest.mark.parametrize("act", [0, 1])
def test_prefill_q82_parity(pg, oracle, rows, cols, n, act):
    _case(f"prefill_gemm_q82 n={n} {rows}x{cols} act={act}")
    rng = np.random.default_rng(rows * 7 + cols + n + act)
    m = synth.q82(rng, rows, cols)
    X = synth.normal(rng, (n, cols))
    Y = pg.prefill_gemm_q82(_dev_q82(pg, m), to_dev(X, torch), act=act)
    torch.cuda.synchronize()
    ref = oracle.gemm_q82(m.q, m.rs, m.cf, X, act=act)
    err = oracle.rel_err(Y.cpu().numpy(), ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_Q8


@pytest.mark.parametrize("rows,cols", [(6144, 4096), (14336, 4096), (4096, 14336), (32000, 4096)])
def test_prefill_q82_frame_shapes_sampled(pg, oracle, rows, cols):
    """The layer frame's shapes at 64 positions, checked on 96 sampled rows of every position."""
    _case(f"prefill_gemm_q82 sampled {rows}x{cols}")
    rng = np.random.default_rng(rows ^ cols)
    m = synth.q82(rng, rows, cols)
    X = synth.normal(rng, (64, cols))
    Y = pg.prefill_gemm_q82(_dev_q82(pg, m), to_dev(X, torch)).cpu().numpy()
    idx = np.unique(np.concatenate([rng.choice(rows, 94, replace=False), [0, rows - 1]]))
    ref = oracle.gemm_q82(m.q[idx], m.rs[idx], m.cf, X)
    assert oracle.rel_err(Y[:, idx], ref) <= TOL_Q8


@pytest.mark.parametrize("rows,cols,n", [(300, 2048, 64), (4096, 4096, 5)])
def test_prefill_q82_exact_bitwise(pg, oracle, rows, cols, n):
    """Power-of-two scales, integer activations: every step is exact, the K splits included."""
    _case(f"prefill_gemm_q82 exact n={n} {rows}x{cols}")
    rng = np.random.default_rng(11 + n)
    q = _plant_m128(rng, rng.integers(-127, 128, size=(rows, cols), dtype=np.int8))
    rs = (2.0 ** -rng.integers(2, 6, rows)).astype(np.float16)
    cf = (2.0 ** rng.integers(-1, 2, cols)).astype(np.float16)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = pg.prefill_gemm_q82(_dev_q82(pg, synth.Q82(q, rs, cf)), to_dev(X, torch))
    torch.cuda.synchronize()
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), oracle.gemm_q82(q, rs, cf, X))


def test_prefill_q82_rows_match_gemv(pg):
    """Each position of the prefill product agrees with the decode product on that row."""
    _case("prefill_gemm_q82 vs gemv_q82")
    rng = np.random.default_rng(3)
    m = synth.q82(rng, 2048, 4096)
    W = _dev_q82(pg, m)
    X = to_dev(synth.normal(rng, (9, 4096)), torch)
    Y = pg.prefill_gemm_q82(W, X)
    for b in range(9):
        g = pg.gemv_q82(W, X[b].contiguous())
        assert float((Y[b] - g).abs().max() / g.pow(2).mean().sqrt()) <= 2 * TOL_Q8


def test_prefill_q82_errors(pg):
    _case("prefill_gemm_q82 errors")
    L = pg.lib()
    rows, cols = 64, 1024
    q = torch.zeros(rows * cols, dtype=torch.int8, device="cuda")
    rs = torch.zeros(rows, dtype=torch.float16, device="cuda")
    cf = torch.zeros(cols, dtype=torch.float16, device="cuda")
    X = torch.zeros(64 * cols, device="cuda")
    Y = torch.zeros(65 * rows, device="cuda")
    need = pg.prefill_gemm_q8_workspace_bytes(rows, cols, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(rows=rows, cols=cols, n=64, qp=None, xp=None, act=0, wsb=need):
        return L.prefill_gemm_q82(qp or P(q), P(rs), P(cf), rows, cols, xp or P(X), n, P(Y), act,
                                  P(ws), wsb, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(n=65) == pg.PG_EUNSUPPORTED
    assert call(cols=1000) == pg.PG_EUNSUPPORTED
    assert call(n=0) == pg.PG_EINVAL
    assert call(act=3) == pg.PG_EINVAL
    assert call(qp=P(q, 4)) == pg.PG_EINVAL
    assert call(xp=P(X, 4)) == pg.PG_EINVAL
    assert call(wsb=need - 1) == pg.PG_EWORKSPACE
    assert L.prefill_gemm_q82(P(q), None, P(cf), rows, cols, P(X), 64, P(Y), 0, P(ws), need, s) == pg.PG_EINVAL


# ------------------------------------------------------------------ expert_bank_q82

def _bank_case(rng, E, rows, cols, n, k):
    """q8_2f experts, n positions each choosing k distinct experts (the grouping from the
    oracle), x [n][cols]."""
    ms = [synth.q82(rng, rows, cols) for _ in range(E)]
    sel = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    return ms, sel, synth.normal(rng, (n, cols))


@pytest.mark.parametrize("E,rows,cols,n,k,act", [(6, 320, 256, 40, 2, 0), (6, 320, 256, 40, 2, 1),
                                                 (3, 100, 96, 64, 3, 1), (1, 33, 32, 1, 1, 0),
                                                 (16, 1856, 2688, 64, 6, 1)])
def test_expert_bank_q82_parity(pg, oracle, E, rows, cols, n, k, act):
    """Each listed entry's row against the oracle's q8_2f product of its expert (x row j / k)."""
    _case(f"expert_bank_q82 E={E} {rows}x{cols} n={n} k={k} act={act}")
    rng = np.random.default_rng(E * rows + cols + n + act)
    ms, sel, X = _bank_case(rng, E, rows, cols, n, k)
    counts, lists = oracle.group(sel, E)
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).cuda()
    out = pg.expert_bank_q82(dev(np.stack([m.q for m in ms])), dev(np.stack([m.rs for m in ms])),
                             dev(np.stack([m.cf for m in ms])), dev(X), dev(counts),
                             dev(np.maximum(lists, 0).astype(np.int32)), src_div=k, act=act, n_out=n * k)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    worst = 0.0
    for e in range(E):
        js = lists[e, :counts[e]]
        if len(js) == 0:
            continue
        ref = oracle.gemm_q82(ms[e].q, ms[e].rs, ms[e].cf, X[js // k], act=act)
        worst = max(worst, oracle.rel_err(out[js], ref))
    print(f"[info] worst rel err {worst:.2e}", flush=True)
    assert worst <= TOL_Q8


def test_expert_bank_q82_exact_bitwise(pg, oracle):
    """Power-of-two scales and column field with integer x: exact on both sides."""
    _case("expert_bank_q82 exact")
    rng = np.random.default_rng(19)
    E, rows, cols, n, k = 5, 200, 512, 24, 2
    ms = []
    for _ in range(E):
        q = _plant_m128(rng, rng.integers(-127, 128, size=(rows, cols), dtype=np.int8))
        rs = (2.0 ** -rng.integers(2, 6, rows)).astype(np.float16)
        cf = (2.0 ** rng.integers(-1, 2, cols)).astype(np.float16)
        ms.append(synth.Q82(q, rs, cf))
    sel = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    counts, lists = oracle.group(sel, E)
    dev = lambda a: torch.as_tensor(np.ascontiguousarray(a)).cuda()
    out = pg.expert_bank_q82(dev(np.stack([m.q for m in ms])), dev(np.stack([m.rs for m in ms])),
                             dev(np.stack([m.cf for m in ms])), dev(X), dev(counts),
                             dev(np.maximum(lists, 0).astype(np.int32)), src_div=k, n_out=n * k)
    torch.cuda.synchronize()
    out = out.cpu().numpy().astype(np.float64)
    for e in range(E):
        js = lists[e, :counts[e]]
        assert np.array_equal(out[js], oracle.gemm_q82(ms[e].q, ms[e].rs, ms[e].cf, X[js // k])), e
