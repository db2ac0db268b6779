"""expert_bank_q4tp (the grouped expert product on the pages' 4-bit format)
against the CPU oracle through the C ABI: each listed entry's row against the
oracle's q4tp product of its expert, at small shapes, a ragged block count,
one entry and one expert, and the MoE pass's up and down shapes; bit-exact
cases (every code value of one group, and whole products with small
power-of-two scales); argument errors."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import TOL_Q8

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _dev(a):
    return torch.as_tensor(np.ascontiguousarray(a)).cuda()


def _pack_codes(codes5):
    """5-bit group codes [rows][groups] -> code bytes, code g at bits 5 g .. (LSB first)."""
    rows, groups = codes5.shape
    bits = ((codes5[:, :, None] >> np.arange(5)) & 1).astype(np.uint8).reshape(rows, -1)
    out = np.packbits(bits, axis=1, bitorder="little")
    return out[:, :(5 * groups + 7) // 8]


def _params(base, step):
    return (np.asarray(base, np.float16).view(np.uint16).astype(np.uint32)
            | (np.asarray(step, np.float16).view(np.uint16).astype(np.uint32) << 16))


def _run(pg, oracle, ms, sel, X, k, act=0):
    E = len(ms)
    n = sel.shape[0]
    counts, lists = oracle.group(sel, E)
    out = pg.expert_bank_q4tp(_dev(np.stack([m.nib for m in ms])),
                              _dev(np.stack([m.params for m in ms]).view(np.int32)),
                              _dev(np.stack([m.codes for m in ms])), _dev(X), _dev(counts),
                              _dev(np.maximum(lists, 0).astype(np.int32)), src_div=k, act=act, n_out=n * k)
    torch.cuda.synchronize()
    return out.cpu().numpy(), counts, lists


@pytest.mark.parametrize("E,rows,cols,n,k,act", [(6, 320, 256, 40, 2, 0), (6, 320, 256, 40, 2, 1),
                                                 (3, 100, 96, 64, 3, 1), (1, 33, 32, 1, 1, 0),
                                                 (5, 64, 2080, 24, 2, 0),
                                                 (16, 1856, 2688, 64, 6, 1), (16, 2688, 1856, 64, 6, 0)])
def test_expert_bank_q4tp_parity(pg, oracle, E, rows, cols, n, k, act):
    """Each listed entry's row against the oracle's q4tp product of its expert (x row j / k)."""
    _case(f"expert_bank_q4tp E={E} {rows}x{cols} n={n} k={k} act={act}")
    rng = np.random.default_rng(E * rows + cols + n + act)
    ms = [synth.q4tp(rng, rows, cols) for _ in range(E)]
    sel = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    X = synth.normal(rng, (n, cols))
    out, counts, lists = _run(pg, oracle, ms, sel, X, k, act)
    worst = 0.0
    for e in range(E):
        js = lists[e, :counts[e]]
        if len(js) == 0:
            continue
        ref = oracle.gemm_q4tp(ms[e].nib, ms[e].params, ms[e].codes, X[js // k], act=act)
        worst = max(worst, oracle.rel_err(out[js], ref))
    print(f"[info] worst rel err {worst:.2e}", flush=True)
    assert worst <= TOL_Q8


@pytest.mark.parametrize("cols,group", [(256, 1), (256, 3), (2080, 64)])
def test_expert_bank_q4tp_exact_one_group(pg, oracle, cols, group):
    """Integer base, step 1 and integer x that is zero outside one group: every output is 2^(base
    + code) times an integer, exact on both sides, bit for bit; 1000 rows an expert meet every
    code value of the group's field (groups 1 and 3 straddle two code bytes)."""
    _case(f"expert_bank_q4tp exact one group cols={cols} group={group}")
    rng = np.random.default_rng(cols + group)
    E, rows, n, k = 3, 1000, 24, 2
    ms = []
    for _ in range(E):
        m = synth.q4tp(rng, rows, cols)
        m.params = _params(rng.integers(-24, -8, rows), np.ones(rows))
        ms.append(m)
    sel = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    X = np.zeros((n, cols), np.float32)
    X[:, 32 * group:32 * group + 32] = rng.integers(-8, 9, (n, 32))
    out, counts, lists = _run(pg, oracle, ms, sel, X, k)
    for e in range(E):
        js = lists[e, :counts[e]]
        ref = oracle.gemm_q4tp(ms[e].nib, ms[e].params, ms[e].codes, X[js // k])
        assert np.array_equal(out[js].astype(np.float64), ref), e


@pytest.mark.parametrize("rows,cols", [(200, 512), (300, 2688)])
def test_expert_bank_q4tp_exact_whole(pg, oracle, rows, cols):
    """Codes 0..3 with base -6 and step 1 and integer x: every partial sum (the -8 scale term
    too) is a multiple of 2^-6 below 2^18, so the whole product is exact: bit for bit."""
    _case(f"expert_bank_q4tp exact {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    E, n, k = 4, 30, 2
    ms = []
    for _ in range(E):
        m = synth.q4tp(rng, rows, cols)
        m.codes = _pack_codes(rng.integers(0, 4, (rows, cols // 32)))
        m.params = _params(np.full(rows, -6.0), np.ones(rows))
        ms.append(m)
    sel = np.stack([rng.choice(E, k, replace=False) for _ in range(n)]).astype(np.int32)
    X = rng.integers(-8, 9, (n, cols)).astype(np.float32)
    out, counts, lists = _run(pg, oracle, ms, sel, X, k)
    for e in range(E):
        js = lists[e, :counts[e]]
        ref = oracle.gemm_q4tp(ms[e].nib, ms[e].params, ms[e].codes, X[js // k])
        assert np.array_equal(out[js].astype(np.float64), ref), e


def test_expert_bank_q4tp_errors(pg):
    _case("expert_bank_q4tp errors")
    L = pg.lib()
    E, rows, cols, cap = 2, 64, 256, 8
    nib = torch.zeros(E * rows * cols // 2, dtype=torch.uint8, device="cuda")
    params = torch.zeros(E * rows + 1, dtype=torch.int32, device="cuda")
    codes = torch.zeros(E * rows * 5, dtype=torch.uint8, device="cuda")
    x = torch.zeros(cap * cols + 4, device="cuda")
    counts = torch.zeros(E, dtype=torch.int32, device="cuda")
    lists = torch.zeros(E * cap, dtype=torch.int32, device="cuda")
    out = torch.zeros(cap * rows, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(cols=cols, cap=cap, np_=None, pp=None, xp=None, act=0, ldx=cols, rows=rows):
        return L.expert_bank_q4tp(np_ or P(nib), pp or P(params), P(codes), E, rows, cols, xp or P(x), ldx, 1,
                                  P(counts), P(lists), cap, P(out), rows, act, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(cols=240) == pg.PG_EUNSUPPORTED
    assert call(cap=65) == pg.PG_EUNSUPPORTED
    # a code buffer under 8 bytes (one row of one group: one code byte) cannot hold a code window
    assert call(rows=1, cols=32, ldx=32) == pg.PG_EUNSUPPORTED
    assert call(act=2) == pg.PG_EINVAL
    assert call(np_=P(nib, 8)) == pg.PG_EINVAL
    assert call(pp=P(params, 2)) == pg.PG_EINVAL
    assert call(xp=P(x, 4)) == pg.PG_EINVAL
    assert call(ldx=cols - 4) == pg.PG_EINVAL
