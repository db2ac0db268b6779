"""Pins of the CPU oracle to things other than itself (runs without a GPU).

Each oracle function is checked against what mathematics fixes independently of
its code: exact rational arithmetic on tiny inputs, exact-integer special
cases, closed forms, invariants, and textbook numpy/scipy routines.  The cases
are chosen so that a plausible mistake (a dropped term, a wrong block index, a
transposed operand, a wrong sign, a wrong tie rule) fails at least one of them;
``test_planted_*`` show that on purpose-broken oracle calls.
"""
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import synth

BLOCK = 32


def _rand_q8(rng, rows, cols):
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    s = rng.uniform(1e-3, 1e-2, size=(rows, cols // BLOCK)).astype(np.float32)
    b = rng.normal(0, 1e-3, size=(rows, cols // BLOCK)).astype(np.float32)
    return q, s, b


# ------------------------------------------------------------------ binary16

def test_f16_decode_all_patterns(oracle):
    """Every binary16 pattern decodes to numpy's float16 -> float64 value."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([oracle.f16_to_f64(int(v)) for v in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_decode_closed_forms(oracle):
    assert oracle.f16_to_f64(0x3C00) == 1.0
    assert oracle.f16_to_f64(0xC000) == -2.0
    assert oracle.f16_to_f64(0x7BFF) == 65504.0
    assert oracle.f16_to_f64(0x0001) == 2.0 ** -24
    assert oracle.f16_to_f64(0x0400) == 2.0 ** -14
    assert oracle.f16_to_f64(0x3555) == 1365 / 4096


# ------------------------------------------------------------------ dequant

def test_dequant_special_cases(oracle):
    rng = np.random.default_rng(1)
    q, s, b = _rand_q8(rng, 3, 96)
    w0 = oracle.dequant_q8(q, np.zeros_like(s), b)
    assert np.array_equal(w0, np.repeat(b.astype(np.float64), BLOCK, axis=1))
    w1 = oracle.dequant_q8(q, s, np.zeros_like(b))
    # s*q with s f32 and |q| < 2^7 is exact in double
    exact = np.array([[float(Fraction(float(s[r, c // BLOCK])) * int(q[r, c]))
                       for c in range(96)] for r in range(3)])
    assert np.array_equal(w1, exact)


def test_dequant_block_index(oracle):
    """Scale 2^-(r+blk), bias (r+1)*2^-(10+blk), q = column-dependent: catches a swapped
    or misplaced block index (c % 32 instead of c // 32, rows for columns)."""
    rows, cols = 4, 128
    q = np.array([[(c % 7) - 3 for c in range(cols)] for _ in range(rows)], np.int8)
    s = np.array([[2.0 ** -(r + k) for k in range(cols // BLOCK)] for r in range(rows)], np.float32)
    b = np.array([[(r + 1) * 2.0 ** -(10 + k) for k in range(cols // BLOCK)] for r in range(rows)],
                 np.float32)
    w = oracle.dequant_q8(q, s, b)
    for r in range(rows):
        for c in range(cols):
            k = c // BLOCK
            assert w[r, c] == ((c % 7) - 3) * 2.0 ** -(r + k) + (r + 1) * 2.0 ** -(10 + k)


def _affine_quant(w):
    """Test-only affine quantizer of one 32-block: b = (max+min)/2, s = (max-min)/254,
    q = clamp(round_half_even((w - b)/s), -127, 127)."""
    lo, hi = float(np.min(w)), float(np.max(w))
    b = np.float32((hi + lo) / 2)
    s = np.float32((hi - lo) / 254) if hi > lo else np.float32(1.0)
    q = np.clip(np.rint((w.astype(np.float64) - b) / s), -127, 127).astype(np.int8)
    return q, s, b


def test_dequant_round_trip(oracle):
    rng = np.random.default_rng(2)
    for trial in range(20):
        rows, cols = 2, 64
        w = rng.normal(0, 10.0 ** rng.uniform(-3, 2), size=(rows, cols))
        q = np.empty((rows, cols), np.int8)
        s = np.empty((rows, cols // BLOCK), np.float32)
        b = np.empty((rows, cols // BLOCK), np.float32)
        for r in range(rows):
            for k in range(cols // BLOCK):
                q[r, k * BLOCK:(k + 1) * BLOCK], s[r, k], b[r, k] = _affine_quant(
                    w[r, k * BLOCK:(k + 1) * BLOCK])
        deq = oracle.dequant_q8(q, s, b)
        bound = np.repeat(s.astype(np.float64), BLOCK, axis=1) * (0.5 + 1e-5) + 1e-7 * np.abs(w)
        assert np.all(np.abs(deq - w) <= bound), trial


# ------------------------------------------------------------------ q8 products

def test_gemm_q8_brute_force_fractions(oracle):
    """Exact rational evaluation of the definition on a tiny 3x64 matrix, two positions."""
    rng = np.random.default_rng(3)
    q, s, b = _rand_q8(rng, 3, 64)
    X = rng.standard_normal((2, 64)).astype(np.float32)
    Y = oracle.gemm_q8(q, s, b, X)
    for p in range(2):
        for r in range(3):
            acc = Fraction(0)
            for c in range(64):
                w = Fraction(float(s[r, c // BLOCK])) * int(q[r, c]) + Fraction(float(b[r, c // BLOCK]))
                acc += w * Fraction(float(X[p, c]))
            assert abs(Y[p, r] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc)))


def test_gemm_q8_exact_integer_case(oracle):
    """s = 2^-3, b = 0, integer x: every partial sum is an exact dyadic, so the f64 result
    equals the integer product exactly (also the case a device must match bit for bit)."""
    rng = np.random.default_rng(4)
    rows, cols, n = 37, 320, 5
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    s = np.full((rows, cols // BLOCK), 0.125, np.float32)
    b = np.zeros((rows, cols // BLOCK), np.float32)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = oracle.gemm_q8(q, s, b, X)
    exact = (X.astype(np.int64) @ q.astype(np.int64).T) / 8
    assert np.array_equal(Y, exact)


def test_gemm_q8_two_term_identity(oracle):
    """y_r = sum_blk s_rb (sum_{c in blk} q_rc x_c) + sum_blk b_rb X_blk with X_blk the block
    sum of x: a dropped bias term, a misplaced scale or a transposed operand breaks it."""
    rng = np.random.default_rng(5)
    rows, cols, n = 50, 256, 3
    q, s, b = _rand_q8(rng, rows, cols)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    Y = oracle.gemm_q8(q, s, b, X)
    nb = cols // BLOCK
    qb = q.astype(np.float64).reshape(rows, nb, BLOCK)
    Xb = X.astype(np.float64).reshape(n, nb, BLOCK)
    T = np.einsum("rkc,pkc->prk", qb, Xb)           # per-block integer-weight dots
    two = np.einsum("prk,rk->pr", T, s.astype(np.float64)) + Xb.sum(-1) @ b.astype(np.float64).T
    np.testing.assert_allclose(Y, two, rtol=1e-12, atol=1e-12)


def test_gemm_q8_textbook_numpy(oracle):
    rng = np.random.default_rng(6)
    rows, cols, n = 70, 192, 4
    q, s, b = _rand_q8(rng, rows, cols)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    W = np.repeat(s.astype(np.float64), BLOCK, 1) * q + np.repeat(b.astype(np.float64), BLOCK, 1)
    np.testing.assert_allclose(oracle.gemm_q8(q, s, b, X), X.astype(np.float64) @ W.T,
                               rtol=1e-12, atol=1e-12)


def test_gemm_q8_act_and_rows(oracle):
    rng = np.random.default_rng(7)
    q, s, b = _rand_q8(rng, 40, 128)
    X = rng.standard_normal((3, 128)).astype(np.float32)
    Y0 = oracle.gemm_q8(q, s, b, X, act=0)
    Y1 = oracle.gemm_q8(q, s, b, X, act=1)
    assert np.array_equal(Y1, np.where(Y0 > 0, Y0 * Y0, 0.0))
    idx = np.array([39, 0, 17, 17])
    assert np.array_equal(oracle.gemm_q8_rows(q, s, b, idx, X, act=1), Y1[:, idx])
    for p in range(3):
        assert np.array_equal(oracle.gemm_q8(q, s, b, X[p]), Y0[p])


# ------------------------------------------------------------------ q8_2f products

def _rand_q82(rng, rows, cols):
    """q8_2f inputs (synthetic recipe): q U[-127,127], row scales U(1e-3,1e-2) and column
    field U(0.5,1.5), both rounded to binary16."""
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    rs = rng.uniform(1e-3, 1e-2, rows).astype(np.float16)
    cf = rng.uniform(0.5, 1.5, cols).astype(np.float16)
    return q, rs, cf


def test_gemm_q82_brute_force_fractions(oracle):
    """Exact rational evaluation of w = rs[r] cf[c] q[r][c] on a tiny 3x40 matrix (binary16
    values are exact in binary64, so Fraction(float(.)) is their exact value)."""
    rng = np.random.default_rng(31)
    q, rs, cf = _rand_q82(rng, 3, 40)
    X = rng.standard_normal((2, 40)).astype(np.float32)
    Y = oracle.gemm_q82(q, rs, cf, X)
    for p in range(2):
        for r in range(3):
            acc = sum(Fraction(float(rs[r])) * Fraction(float(cf[c])) * int(q[r, c]) * Fraction(float(X[p, c]))
                      for c in range(40))
            assert abs(Y[p, r] - float(acc)) <= 1e-13 * max(1.0, abs(float(acc)))


def test_gemm_q82_exact_integer_case(oracle):
    """Power-of-two row scales and column field with integer x: the f64 result equals the
    integer product exactly (the case a device must match bit for bit)."""
    rng = np.random.default_rng(32)
    rows, cols, n = 29, 160, 4
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    rs = (2.0 ** -rng.integers(2, 6, rows)).astype(np.float16)
    cf = (2.0 ** rng.integers(-1, 2, cols)).astype(np.float16)
    X = rng.integers(-8, 9, size=(n, cols)).astype(np.float32)
    Y = oracle.gemm_q82(q, rs, cf, X)
    num = (X.astype(np.int64) * (cf.astype(np.float64) * 2).astype(np.int64)) @ q.astype(np.int64).T
    exact = num * rs.astype(np.float64)[None, :] / 2
    assert np.array_equal(Y, exact)


def test_gemm_q82_equals_block_format_without_column_field(oracle):
    """cf = 1 and rs[r] = s_r make q8_2f the block format with scale s_r on every block and
    zero bias: the two oracles agree (a swapped row / column role would not)."""
    rng = np.random.default_rng(33)
    rows, cols, n = 24, 96, 3
    q, rs, _ = _rand_q82(rng, rows, cols)
    cf = np.ones(cols, np.float16)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    s = np.repeat(rs.astype(np.float32)[:, None], cols // BLOCK, 1)
    b = np.zeros_like(s)
    np.testing.assert_allclose(oracle.gemm_q82(q, rs, cf, X), oracle.gemm_q8(q, s, b, X),
                               rtol=1e-12, atol=1e-14)


def test_gemm_q82_column_field_folds_into_x(oracle):
    """The column field can be moved onto the activation (the pages fold it into the staged
    x): with power-of-two cf the folded x is exact in f32 and the results are equal."""
    rng = np.random.default_rng(34)
    rows, cols, n = 17, 128, 2
    q, rs, _ = _rand_q82(rng, rows, cols)
    cf = (2.0 ** rng.integers(-2, 3, cols)).astype(np.float16)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    folded = (X * cf.astype(np.float32)).astype(np.float32)
    np.testing.assert_array_equal(oracle.gemm_q82(q, rs, cf, X),
                                  oracle.gemm_q82(q, rs, np.ones(cols, np.float16), folded))


def test_gemm_q82_textbook_numpy_and_act(oracle):
    rng = np.random.default_rng(35)
    rows, cols, n = 45, 224, 3
    q, rs, cf = _rand_q82(rng, rows, cols)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    W = rs.astype(np.float64)[:, None] * cf.astype(np.float64)[None, :] * q
    ref = X.astype(np.float64) @ W.T
    np.testing.assert_allclose(oracle.dequant_q82(q, rs, cf), W, rtol=0, atol=0)
    np.testing.assert_allclose(oracle.gemm_q82(q, rs, cf, X), ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(oracle.gemm_q82(q, rs, cf, X, act=1), np.maximum(ref, 0) ** 2,
                               rtol=1e-12, atol=1e-13)


def test_relu2_closed_form(oracle):
    """relu^2 on outputs with known values: 3 -> 9, -2 -> 0, 0 -> 0."""
    q = np.zeros((3, 32), np.int8)
    q[0, 0], q[1, 0], q[2, 0] = 3, -2, 0
    s = np.ones((3, 1), np.float32)
    b = np.zeros((3, 1), np.float32)
    x = np.zeros(32, np.float32)
    x[0] = 1.0
    assert list(oracle.gemm_q8(q, s, b, x, act=1)) == [9.0, 0.0, 0.0]


# ------------------------------------------------------------------ f16 products

def test_gemm_f16_textbook_and_exact(oracle):
    rng = np.random.default_rng(8)
    W = synth.f16(rng, 33, 96)
    X = rng.standard_normal((2, 96)).astype(np.float32)
    np.testing.assert_allclose(oracle.gemm_f16(W, X), X.astype(np.float64) @ W.astype(np.float64).T,
                               rtol=1e-12, atol=1e-13)
    Wi = (rng.integers(-64, 65, size=(9, 64)) / 16).astype(np.float16)   # exact dyadics
    Xi = rng.integers(-5, 6, size=(3, 64)).astype(np.float32)
    exact = (Xi.astype(np.int64) @ (Wi.astype(np.float64) * 16).astype(np.int64).T) / 16
    assert np.array_equal(oracle.gemm_f16(Wi, Xi), exact)


# ------------------------------------------------------------------ add + RMSNorm

def test_rmsnorm_unit_weight_rms(oracle):
    """w = 1: RMS(out) = sqrt(m / (m + eps)) with m = mean(h'^2)."""
    rng = np.random.default_rng(9)
    for H, eps in [(1024, 1e-6), (2688, 1e-6), (64, 0.5)]:
        h = rng.standard_normal((3, H)).astype(np.float32)
        d = rng.standard_normal((3, H)).astype(np.float32)
        hp, out = oracle.add_rmsnorm(h, d, np.ones(H, np.float32), eps)
        m = np.mean(hp * hp, axis=1)
        np.testing.assert_allclose(np.sqrt(np.mean(out * out, axis=1)), np.sqrt(m / (m + eps)),
                                   rtol=1e-13)


def test_rmsnorm_add_and_stride(oracle):
    rng = np.random.default_rng(10)
    n, H, stride = 4, 256, 384
    h = rng.standard_normal((n, H)).astype(np.float32)
    wide = rng.standard_normal((n, stride)).astype(np.float32)
    w = synth.norm_weight(rng, H)
    hp, out = oracle.add_rmsnorm(h, wide, w, 1e-6, delta_stride=stride)
    assert np.array_equal(hp, h.astype(np.float64) + wide[:, :H])     # exact in f64
    hp0, out0 = oracle.add_rmsnorm(h, None, w, 1e-6)
    assert np.array_equal(hp0, h.astype(np.float64))
    ref = w * hp / np.sqrt(np.mean(hp * hp, axis=1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(out, ref, rtol=1e-13)


def test_rmsnorm_special_cases(oracle):
    H = 128
    w = np.linspace(0.5, 1.5, H).astype(np.float32)
    zero = np.zeros(H, np.float32)
    hp, out = oracle.add_rmsnorm(zero, zero, w, 1e-6)
    assert np.all(out == 0.0)
    a, i = 3.0, 17
    h = zero.copy()
    h[i] = a
    _, out = oracle.add_rmsnorm(h, None, w, 1e-6)
    expect = np.zeros(H)
    expect[i] = float(w[i]) * a / np.sqrt(a * a / H + 1e-6)
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=0)


def test_rmsnorm_scale_invariance(oracle):
    rng = np.random.default_rng(11)
    h = rng.standard_normal(512).astype(np.float32)
    w = synth.norm_weight(rng, 512)
    _, o1 = oracle.add_rmsnorm(h, None, w, 1e-6)
    _, o2 = oracle.add_rmsnorm(h * np.float32(64.0), None, w, 1e-6)
    np.testing.assert_allclose(o1, o2, rtol=1e-6)


# ------------------------------------------------------------------ router

def test_router_logits_f64_textbook(oracle):
    rng = np.random.default_rng(12)
    X = rng.standard_normal((5, 2688)).astype(np.float32)
    Wr = synth.router_weight(rng, 128, 2688)
    np.testing.assert_allclose(oracle.router_logits_f64(X, Wr),
                               X.astype(np.float64) @ Wr.astype(np.float64).T, rtol=1e-12, atol=1e-13)


def test_router_logits_f32_exact_integers(oracle):
    """Small integers: every f32 partial sum is exact, so the f32 logit is the integer dot."""
    rng = np.random.default_rng(13)
    X = rng.integers(-9, 10, size=(4, 2688)).astype(np.float32)
    Wr = rng.integers(-9, 10, size=(16, 2688)).astype(np.float32)
    got = oracle.router_logits_f32(X, Wr)
    assert np.array_equal(got.astype(np.float64), (X.astype(np.int64) @ Wr.astype(np.int64).T))


def test_router_logits_f32_error_bound(oracle):
    """|f32 - exact| <= gamma * sum|x w| with gamma for the longest chain plus tree depth."""
    rng = np.random.default_rng(14)
    H = 2688
    X = rng.standard_normal((8, H)).astype(np.float32)
    Wr = synth.router_weight(rng, 32, H)
    f32 = oracle.router_logits_f32(X, Wr).astype(np.float64)
    f64 = oracle.router_logits_f64(X, Wr)
    depth = 4 * -(-(H // 4) // 64) + 6
    u = 2.0 ** -24
    gamma = depth * u / (1 - depth * u)
    bound = gamma * (np.abs(X.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T)
    assert np.all(np.abs(f32 - f64) <= bound)
    assert np.any(f32 != f64)   # it really is an f32 computation


def test_route_textbook_topk_and_softmax(oracle):
    rng = np.random.default_rng(15)
    n, E, k = 64, 128, 6
    logits = (rng.standard_normal((n, E)) * 1.3).astype(np.float32)
    sel, rw, probs = oracle.route(logits, k)
    for b in range(n):
        order = np.lexsort((np.arange(E), -logits[b].astype(np.float64)))
        assert list(sel[b]) == list(order[:k])
    np.testing.assert_allclose(probs, scipy.special.softmax(logits.astype(np.float64), axis=1),
                               rtol=1e-13)
    np.testing.assert_allclose(probs.sum(1), 1.0, rtol=1e-14)
    assert np.array_equal(rw, np.take_along_axis(probs, sel.astype(np.int64), 1))
    _, rwn, _ = oracle.route(logits, k, renorm=1)
    np.testing.assert_allclose(rwn.sum(1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(rwn, rw / rw.sum(1, keepdims=True), rtol=1e-14)


def test_route_tie_lower_index_wins(oracle):
    """Duplicate router rows e1 < e2 give identical logits; e1 must rank first."""
    rng = np.random.default_rng(16)
    H, E = 256, 16
    Wr = synth.router_weight(rng, E, H)
    Wr[11] = Wr[3]
    Wr[9] = Wr[3] * np.float32(4.0)      # strictly larger for positive logits
    X = rng.standard_normal((32, H)).astype(np.float32)
    L = oracle.router_logits_f32(X, Wr)
    assert np.array_equal(L[:, 3], L[:, 11])
    sel, _, _ = oracle.route(L, E)
    for b in range(32):
        pos = {int(e): t for t, e in enumerate(sel[b])}
        assert pos[3] < pos[11]
    # all-equal logits: selection is 0, 1, 2, ...
    sel, rw, _ = oracle.route(np.zeros((2, 10), np.float32), 4)
    assert sel.tolist() == [[0, 1, 2, 3]] * 2
    np.testing.assert_allclose(rw, 0.1, rtol=1e-15)


def test_group_textbook(oracle):
    rng = np.random.default_rng(17)
    n, k, E = 64, 6, 128
    sel = np.stack([rng.permutation(E)[:k] for _ in range(n)]).astype(np.int32)
    counts, lists = oracle.group(sel, E)
    flat = sel.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    order = np.argsort(flat, kind="stable")
    starts = np.concatenate([[0], np.cumsum(counts)[:-1]])
    for e in range(E):
        assert list(lists[e, :counts[e]]) == list(order[starts[e]:starts[e] + counts[e]])
        assert np.all(lists[e, counts[e]:] == -1)
    assert counts.sum() == n * k
    seen = np.concatenate([lists[e, :counts[e]] for e in range(E)])
    assert np.array_equal(np.sort(seen), np.arange(n * k))


# ------------------------------------------------------------------ routed experts

def _small_moe(seed, n=6, H=64, I=96, E=5, k=2):
    rng = np.random.default_rng(seed)
    up = synth.q8(rng, I, H, lead=(E,))
    down = synth.q8(rng, H, I, lead=(E,))
    X = rng.standard_normal((n, H)).astype(np.float32)
    h = rng.standard_normal((n, H)).astype(np.float32)
    Wr = synth.router_weight(rng, E, H)
    w = synth.norm_weight(rng, H)
    return up, down, X, h, Wr, w, k


def test_moe_grouped_equals_ungrouped(oracle):
    up, down, X, h, Wr, w, k = _small_moe(18)
    sel, _, _ = oracle.route(oracle.router_logits_f32(X, Wr), k)
    t_up, t_dn = (up.q, up.scale, up.bias), (down.q, down.scale, down.bias)
    U0, D0 = oracle.moe_experts(X, sel, t_up, t_dn, grouped=False)
    U1, D1 = oracle.moe_experts(X, sel, t_up, t_dn, grouped=True)
    assert np.array_equal(U0, U1) and np.array_equal(D0, D1)


def test_moe_single_expert_is_dense_ffn(oracle):
    """k = 1 and every position routed to one expert: U = relu^2(Up x), D = Down U."""
    up, down, X, h, Wr, w, _ = _small_moe(19, E=3)
    n = X.shape[0]
    sel = np.full((n, 1), 2, np.int32)
    U, D = oracle.moe_experts(X, sel, (up.q, up.scale, up.bias), (down.q, down.scale, down.bias))
    U_ref = oracle.gemm_q8(up.q[2], up.scale[2], up.bias[2], X, act=1)
    assert np.array_equal(U, U_ref)
    Wd = oracle.dequant_q8(down.q[2], down.scale[2], down.bias[2])
    np.testing.assert_allclose(D, U_ref @ Wd.T, rtol=1e-12, atol=1e-12)


def test_moe_combine_textbook(oracle):
    rng = np.random.default_rng(20)
    n, k, H = 5, 3, 96
    h = rng.standard_normal((n, H)).astype(np.float32)
    D = rng.standard_normal((n * k, H))
    rw = rng.uniform(0, 1, (n, k))
    w = synth.norm_weight(rng, H)
    hp, out = oracle.moe_combine(h, D, rw, w, 1e-6)
    m = np.einsum("bt,bti->bi", rw, D.reshape(n, k, H))
    np.testing.assert_allclose(hp, h + m, rtol=1e-14, atol=1e-14)
    ref = w * hp / np.sqrt(np.mean(hp * hp, 1, keepdims=True) + 1e-6)
    np.testing.assert_allclose(out, ref, rtol=1e-13)


def test_moe_pass_stages_consistent(oracle):
    up, down, X, h, Wr, w, k = _small_moe(21, n=8, E=6, k=3)
    res = oracle.moe_pass(X, h, Wr, (up.q, up.scale, up.bias), (down.q, down.scale, down.bias),
                          w, 1e-6, k)
    assert res["counts"].sum() == 8 * 3
    for j in range(8 * 3):
        b, t = divmod(j, 3)
        e = res["sel"][b, t]
        np.testing.assert_allclose(res["U"][j], oracle.gemm_q8(up.q[e], up.scale[e], up.bias[e],
                                                               X[b], act=1), rtol=0, atol=0)


# ------------------------------------------------------------------ planted mistakes

def test_planted_dropped_bias_is_caught(oracle):
    """A mistake planted in the oracle call (the bias term dropped) fails the
    two-term identity pin."""
    rng = np.random.default_rng(22)
    q, s, b = _rand_q8(rng, 20, 128)
    X = rng.standard_normal((2, 128)).astype(np.float32)
    bad = oracle.gemm_q8(q, s, np.zeros_like(b), X)
    nb = 4
    T = np.einsum("rkc,pkc->prk", q.astype(np.float64).reshape(20, nb, BLOCK),
                  X.astype(np.float64).reshape(2, nb, BLOCK))
    two = np.einsum("prk,rk->pr", T, s.astype(np.float64)) + \
        X.astype(np.float64).reshape(2, nb, BLOCK).sum(-1) @ b.astype(np.float64).T
    assert not np.allclose(bad, two, rtol=1e-9, atol=1e-9)


def test_planted_transpose_is_caught(oracle):
    """A transposed weight operand (square matrix, so the shapes still fit) fails the
    exact rational brute force."""
    rng = np.random.default_rng(23)
    q, s, b = _rand_q8(rng, 64, 64)
    x = rng.standard_normal(64).astype(np.float32)
    W = oracle.dequant_q8(q, s, b)
    qt = np.ascontiguousarray(q.T)
    bad = oracle.gemm_q8(qt, s, b, x)
    exact = np.array([float(sum(Fraction(W[r, c]) * Fraction(float(x[c])) for c in range(64)))
                      for r in range(64)])
    assert np.max(np.abs(bad - exact)) > 1e-3


def test_planted_wrong_tie_rule_is_caught(oracle):
    """Reversing the tie rule (higher index wins) fails the duplicate-row tie pin."""
    L = np.zeros((1, 8), np.float32)
    L[0, 2] = L[0, 6] = 1.0
    sel, _, _ = oracle.route(L, 2)
    assert sel.tolist() == [[2, 6]]
    flipped = oracle.route(L[:, ::-1].copy(), 2)[0]
    assert (7 - flipped).tolist() != [[2, 6]]   # the mirrored walk prefers the other copy


# ------------------------------------------------------------------ q4tp

def _pack_q4tp(v, code, base, step):
    """Independent packer (the inverse of the decoding): v int [-8, 7] [rows][cols],
    code int [0, 31] [rows][cols/32], base/step binary16 [rows] -> (nib, params, codes)."""
    rows, cols = v.shape
    u = (v + 8).astype(np.uint8)
    nib = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    bits = ((code[:, :, None] >> np.arange(5)) & 1).astype(np.uint8).reshape(rows, -1)
    codes = np.packbits(bits, axis=1, bitorder="little")
    params = (base.view(np.uint16).astype(np.uint32) | (step.view(np.uint16).astype(np.uint32) << 16))
    return nib, params.astype(np.uint32), codes


def test_q4tp_hand_worked_example(oracle):
    """One row of two groups worked out by hand: base -2, step 0.5; group 0 code 3 (scale
    2^-0.5), group 1 code 21 (scale 2^8.5), whose 5 bits straddle the first two code bytes
    (byte 0 = 3 | 5 << 5 = 163, byte 1 = 21 >> 3 = 2).  Nibble byte 0 = 0x1F holds columns 0
    (low half, 15 - 8 = 7) and 1 (high half, 1 - 8 = -7); byte 16 = 0x80 holds column 32
    (0 - 8 = -8) and 33 (8 - 8 = 0); every other byte is 0x88 (weights 0)."""
    assert oracle.q4tp_code_bytes(64) == 2
    nib = np.full((1, 32), 0x88, np.uint8)
    nib[0, 0] = 0x1F
    nib[0, 16] = 0x80
    params = np.array([0xC000 | (0x3800 << 16)], np.uint32)   # f16 -2.0 low, f16 0.5 high
    codes = np.array([[163, 2]], np.uint8)
    W = oracle.dequant_q4tp(nib, params, codes)
    want = np.zeros((1, 64))
    want[0, 0], want[0, 1], want[0, 32] = 7 * 2 ** -0.5, -7 * 2 ** -0.5, -8 * 2 ** 8.5
    np.testing.assert_array_equal(W, want)


def test_q4tp_packer_round_trip(oracle):
    """Random integers, codes and parameters packed by the test's own packer decode to
    scale * integer, element by element; a swapped nibble half, a code bit order mistake or a
    wrong group index fails."""
    rng = np.random.default_rng(41)
    rows, cols = 7, 160                          # 5 groups: 25 code bits, 4 bytes a row
    v = rng.integers(-8, 8, size=(rows, cols))
    code = rng.integers(0, 32, size=(rows, cols // 32))
    base = rng.uniform(-12, -4, rows).astype(np.float16)
    step = rng.uniform(0.05, 0.4, rows).astype(np.float16)
    W = oracle.dequant_q4tp(*_pack_q4tp(v, code, base, step))
    scale = np.exp2(base.astype(np.float64)[:, None] + code * step.astype(np.float64)[:, None])
    np.testing.assert_allclose(W, np.repeat(scale, 32, axis=1) * v, rtol=1e-15, atol=0)


def test_gemm_q4tp_equals_block_format(oracle):
    """Integer base and step make every group scale a power of two (exact in f32): q4tp is then
    the block format with q = nib - 8, that scale per 32-column block and zero bias, and the two
    oracles agree."""
    rng = np.random.default_rng(42)
    rows, cols, n = 33, 256, 3
    v = rng.integers(-8, 8, size=(rows, cols))
    code = rng.integers(0, 32, size=(rows, cols // 32))
    base = rng.integers(-20, -8, rows).astype(np.float16)
    step = np.ones(rows, np.float16)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    s = np.exp2(base.astype(np.float64)[:, None] + code).astype(np.float32)
    ref = oracle.gemm_q8(v.astype(np.int8), s, np.zeros_like(s), X)
    np.testing.assert_allclose(oracle.gemm_q4tp(*_pack_q4tp(v, code, base, step), X), ref,
                               rtol=1e-12, atol=1e-14)


def test_gemm_q4tp_textbook_numpy_and_act(oracle):
    rng = np.random.default_rng(43)
    rows, cols, n = 21, 96, 4
    v = rng.integers(-8, 8, size=(rows, cols))
    code = rng.integers(0, 32, size=(rows, cols // 32))
    base = rng.uniform(-10, -6, rows).astype(np.float16)
    step = rng.uniform(0.1, 0.3, rows).astype(np.float16)
    X = rng.standard_normal((n, cols)).astype(np.float32)
    W = np.repeat(np.exp2(base.astype(np.float64)[:, None] + code * step.astype(np.float64)[:, None]), 32, 1) * v
    ref = X.astype(np.float64) @ W.T
    packed = _pack_q4tp(v, code, base, step)
    np.testing.assert_allclose(oracle.gemm_q4tp(*packed, X), ref, rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(oracle.gemm_q4tp(*packed, X, act=1), np.maximum(ref, 0) ** 2,
                               rtol=1e-12, atol=1e-20)


# ------------------------------------------------------------------ argmax

def test_argmax_matches_numpy_first_occurrence(oracle):
    """Finite logits: numpy's argmax (first index of the maximum), with ties planted."""
    rng = np.random.default_rng(51)
    L = rng.standard_normal((40, 1000)).astype(np.float32)
    for b in range(0, 40, 3):                    # duplicate each chosen row's maximum later on
        m = L[b].max()
        L[b, rng.choice(1000, 3, replace=False)] = m
    np.testing.assert_array_equal(oracle.argmax_rows(L), np.argmax(L, axis=1))


def test_argmax_nan_and_floor(oracle):
    """NaN never wins (numpy's nanargmax); a logit must exceed -3.0e38 to be chosen, so rows
    of -inf, of values at or below -3.0e38, or of NaN give 0."""
    rng = np.random.default_rng(52)
    L = rng.standard_normal((6, 64)).astype(np.float32)
    L[0, ::5] = np.nan
    L[1, :] = -np.inf
    L[2, :] = np.float32(-3.0e38)
    L[3, :] = np.nan
    L[4, :] = -np.inf
    L[4, 17] = np.float32(-3.05e38)
    L[5, :] = -np.inf
    L[5, 40] = np.float32(-2.9e38)
    ids = oracle.argmax_rows(L)
    assert ids[0] == np.nanargmax(L[0])
    assert list(ids[1:]) == [0, 0, 0, 0, 40]
    row = np.array([-np.inf, 5, np.nan, 5, 4], np.float32)
    assert oracle.argmax_rows(row) == 1


# ------------------------------------------------------------------ sigmoid router

def test_route_sigmoid_hand_worked(oracle):
    """Four experts with equal logits 0 (sigmoid 1/2 each): the bias alone orders them,
    bias [0.1, 0.3, 0.2, 0.0] -> experts 1 then 2; the bias does not enter the weights,
    which are 1/2 * 2.5 = 1.25 without renormalisation, and 1/2 / (1 + 1e-20) * 2.5 = 1.25
    with it (both halves equal)."""
    L = np.zeros((1, 4), np.float32)
    bias = np.array([0.1, 0.3, 0.2, 0.0], np.float32)
    sel, rw, _ = oracle.route_sigmoid(L, bias, 2, norm=0, scale=2.5)
    assert sel.tolist() == [[1, 2]] and rw.tolist() == [[1.25, 1.25]]
    sel, rw, _ = oracle.route_sigmoid(L, bias, 2, norm=1, scale=2.5)
    assert sel.tolist() == [[1, 2]] and rw.tolist() == [[1.25, 1.25]]


def test_route_sigmoid_zero_bias_is_topk_of_logits(oracle):
    """Zero bias: sigmoid is increasing, so the choice is the k largest logits in order
    (numpy's stable argsort of -l), and the renormalised weights are scipy's expit of the
    chosen logits over their sum, times scale."""
    rng = np.random.default_rng(61)
    L = rng.standard_normal((20, 128)).astype(np.float32)
    sel, rw, choice = oracle.route_sigmoid(L, np.zeros(128, np.float32), 6, norm=1, scale=1.5)
    want = np.argsort(-L.astype(np.float64), axis=1, kind="stable")[:, :6]
    np.testing.assert_array_equal(sel, want)
    s = scipy.special.expit(np.take_along_axis(L.astype(np.float64), want, 1))
    np.testing.assert_allclose(rw, s / (s.sum(1, keepdims=True) + 1e-20) * 1.5, rtol=1e-14)
    np.testing.assert_allclose(choice, scipy.special.expit(L.astype(np.float64)), rtol=4 * 2.0 ** -24)


def test_exp_f32_within_one_ulp(oracle):
    """The fixed binary32 exp is within one unit in the last place of the true value over the
    whole clamped range (a wrong Taylor coefficient, a dropped reduction step or a sign slip
    each break this by orders of magnitude)."""
    rng = np.random.default_rng(64)
    x = np.unique(np.concatenate([np.linspace(-80, 80, 320001), rng.uniform(-20, 20, 50000)]).astype(np.float32))
    got = oracle.exp_f32(x).astype(np.float64)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(got - ref) / ulp) <= 1.0
    # clamped outside [-80, 80]: no subnormal, no infinity
    edge = oracle.exp_f32(np.array([-1e4, -80, 80, 1e4], np.float32))
    assert edge[0] == edge[1] and edge[2] == edge[3] and np.all(np.isfinite(edge)) and edge[0] >= 2.0 ** -126


def test_sigmoid_f32_closed_forms(oracle):
    """sigma(0) = 1/2 exactly (e^0 = 1 exactly: k = 0, r = 0, the polynomial's constant term);
    sigma(l) + sigma(-l) = 1 to a few units in the last place; within 3 ulp of scipy's expit on
    a sweep; saturates to 1 for large l and to a normal number near 0 for very negative l."""
    assert oracle.sigmoid_f32([0.0])[0] == np.float32(0.5)
    l = np.linspace(-30, 30, 200001).astype(np.float32)
    s = oracle.sigmoid_f32(l).astype(np.float64)
    ref = scipy.special.expit(l.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    assert np.max(np.abs(s - ref) / ulp) <= 3.0
    np.testing.assert_allclose(s + oracle.sigmoid_f32(-l).astype(np.float64), 1.0, atol=4 * 2.0 ** -24)
    big = oracle.sigmoid_f32([100.0, 1e6, -100.0, -1e6])
    assert big[0] == 1.0 and big[1] == 1.0 and 0 < big[2] < 2e-35 and big[2] == big[3]


def _topk_f64(c, k):
    return np.lexsort((np.arange(c.size), -c))[:k]


def test_route_sigmoid_f32_choice_equals_f64_definition(oracle):
    """The binary32 choice value (the fixed sigmoid plus one add) selects what the f64
    definition sigma(l) + bias selects wherever the f64 values leave every gap among a
    position's top k + 1 wider than the binary32 error (3 ulp of sigma plus the add's
    rounding, both below 2^-22 for values below 2)."""
    rng = np.random.default_rng(65)
    n, E, k = 400, 128, 6
    L = rng.standard_normal((n, E)).astype(np.float32)
    bias = synth.router_bias(rng, E)
    sel, _, _ = oracle.route_sigmoid(L, bias, k)
    c64 = scipy.special.expit(L.astype(np.float64)) + bias.astype(np.float64)
    bound = 2.0 ** -21
    checked = 0
    for b in range(n):
        top = np.sort(c64[b])[::-1][:k + 1]
        if np.min(top[:k] - top[1:]) > bound:
            assert np.array_equal(sel[b], _topk_f64(c64[b], k)), b
            checked += 1
    assert checked >= 0.95 * n


def test_route_f32_logits_select_as_f64_logits(oracle):
    """Top-k on the fixed-order f32 logits equals top-k on the f64 logits wherever the f64
    logits leave every gap among a position's top k + 1 wider than twice the f32 logits'
    error bound (gamma of the chain length plus fold depth, times sum |x w|)."""
    rng = np.random.default_rng(66)
    n, H, E, k = 96, 2688, 128, 6
    X = rng.standard_normal((n, H)).astype(np.float32)
    Wr = synth.router_weight(rng, E, H)
    f32 = oracle.router_logits_f32(X, Wr)
    f64 = oracle.router_logits_f64(X, Wr)
    sel, _, _ = oracle.route(f32, k)
    depth = 4 * -(-(H // 4) // 64) + 6
    u = 2.0 ** -24
    bound = depth * u / (1 - depth * u) * (np.abs(X.astype(np.float64)) @ np.abs(Wr.astype(np.float64)).T)
    checked = 0
    for b in range(n):
        order = _topk_f64(f64[b], k + 1)
        top = f64[b][order]
        if np.all(top[:k] - top[1:] > 2 * np.max(bound[b])):
            assert np.array_equal(sel[b], order[:k]), b
            checked += 1
    assert checked >= 0.9 * n


def test_route_sigmoid_bias_ties_and_unnormalised(oracle):
    """A large bias forces experts in; exact ties go to the lower index; without
    renormalisation the weight is sigmoid(l) * scale."""
    rng = np.random.default_rng(62)
    L = rng.standard_normal((5, 32)).astype(np.float32)
    bias = np.zeros(32, np.float32)
    bias[[30, 7]] = 5.0                       # always chosen first: 7 vs 30 by choice value
    L[:, 3] = L[:, 9] = 10.0                  # equal choice values: 3 before 9
    sel, rw, _ = oracle.route_sigmoid(L, bias, 4, norm=0, scale=0.75)
    for b in range(5):
        first = sorted([7, 30], key=lambda e: -(scipy.special.expit(float(L[b, e])) + 5.0))
        assert sel[b].tolist() == first + [3, 9]
    np.testing.assert_allclose(rw, scipy.special.expit(np.take_along_axis(L.astype(np.float64), sel, 1)) * 0.75,
                               rtol=1e-14)


def test_moe_combine_shared_term(oracle):
    """The shared term adds to the residual with the slots: equals numpy's h + shared +
    sum_t rw D, then the norm; and shared = 0 equals no shared term."""
    rng = np.random.default_rng(63)
    n, k, H = 3, 4, 64
    h = rng.standard_normal((n, H)).astype(np.float32)
    sh = rng.standard_normal((n, H)).astype(np.float32)
    D = rng.standard_normal((n * k, H))
    rw = rng.uniform(0, 1, (n, k))
    w = rng.uniform(0.5, 1.5, H).astype(np.float32)
    hp, out = oracle.moe_combine(h, D, rw, w, 1e-6, shared=sh)
    ref = h.astype(np.float64) + sh + np.einsum("bt,bti->bi", rw, D.reshape(n, k, H))
    np.testing.assert_allclose(hp, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(out, w * ref / np.sqrt((ref ** 2).mean(1, keepdims=True) + 1e-6), rtol=1e-12)
    hp0, _ = oracle.moe_combine(h, D, rw, w, 1e-6, shared=np.zeros_like(sh))
    np.testing.assert_array_equal(hp0, oracle.moe_combine(h, D, rw, w, 1e-6)[0])


# ------------------------------------------------------------------ prefill attention

def _numpy_attention(q, kc, vc, pos0, scale):
    """Textbook: per position and head, scipy's softmax of the masked scores times V."""
    n, nh, hd = q.shape
    nkv = kc.shape[1]
    rep = nh // nkv
    o = np.zeros((n, nh, hd))
    for b in range(n):
        J = pos0 + b + 1
        for h in range(nh):
            s = scale * (kc[:J, h // rep].astype(np.float64) @ q[b, h].astype(np.float64))
            o[b, h] = scipy.special.softmax(s) @ vc[:J, h // rep].astype(np.float64)
    return o


def test_attn_single_key_and_uniform(oracle):
    """Position 0 of the first pass sees one key: o = v_0 exactly.  q = 0 makes every score
    equal: o is the plain mean of the visible V rows."""
    rng = np.random.default_rng(71)
    n, nh, nkv, hd = 5, 4, 2, 16
    kc = rng.standard_normal((n, nkv, hd)).astype(np.float32)
    vc = rng.standard_normal((n, nkv, hd)).astype(np.float32)
    q = rng.standard_normal((n, nh, hd)).astype(np.float32)
    o = oracle.attn_prefill(q, kc, vc, 0, 0.25)
    for h in range(nh):
        np.testing.assert_array_equal(o[0, h], vc[0, h // 2].astype(np.float64))
    o0 = oracle.attn_prefill(np.zeros_like(q), kc, vc, 0, 0.25)
    for b in range(n):
        for h in range(nh):
            np.testing.assert_allclose(o0[b, h], vc[:b + 1, h // 2].astype(np.float64).mean(0), rtol=1e-13, atol=1e-15)


def test_attn_textbook_gqa_mapping_and_causality(oracle):
    """scipy softmax per (position, head) with KV head h // rep over keys j <= pos0 + b; the
    KV heads hold different values, so reading head h % nkv instead fails, and rows past the
    causal limit hold large values that would show if they were read."""
    rng = np.random.default_rng(72)
    n, pos0, nh, nkv, hd = 6, 9, 8, 2, 32
    ctx = pos0 + n + 3
    kc = rng.standard_normal((ctx, nkv, hd)).astype(np.float32)
    vc = rng.standard_normal((ctx, nkv, hd)).astype(np.float32)
    kc[pos0 + n:] = 50.0
    vc[pos0 + n:] = 1e6
    vc[:, 1] += 3.0
    q = rng.standard_normal((n, nh, hd)).astype(np.float32)
    o = oracle.attn_prefill(q, kc, vc, pos0, hd ** -0.5)
    np.testing.assert_allclose(o, _numpy_attention(q, kc, vc, pos0, hd ** -0.5), rtol=1e-11, atol=1e-12)
    assert np.abs(o).max() < 100


def test_kv_append(oracle):
    rng = np.random.default_rng(73)
    kc = np.zeros((10, 2, 4), np.float32)
    vc = np.zeros((10, 2, 4), np.float32)
    k = rng.standard_normal((3, 8)).astype(np.float32)
    v = rng.standard_normal((3, 8)).astype(np.float32)
    kc2, vc2 = oracle.kv_append(kc, vc, k, v, 4)
    assert (kc2[:4] == 0).all() and (kc2[7:] == 0).all() and (kc == 0).all()
    np.testing.assert_array_equal(kc2[4:7].reshape(3, 8), k)
    np.testing.assert_array_equal(vc2[4:7].reshape(3, 8), v)
