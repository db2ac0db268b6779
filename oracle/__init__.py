"""Python face of the plain CPU oracle (``oracle.c``), computed in float64.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module; the product package
never imports it.  Each function states the definition it evaluates; the C
source cites the page passages.

The shared library is built from ``oracle.c`` with gcc (``build()``), with
OpenMP over independent outputs and no fast-math.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", _LIB, "-lm"]

_lib = None


def build() -> str:
    subprocess.run(GCC_CMD, check=True)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


_P = ctypes.c_void_p
_I = ctypes.c_int64
_i = ctypes.c_int
_D = ctypes.c_double


def _declare(L):
    L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    L.oracle_f16_to_f64.restype = _D
    L.oracle_dequant_q8.argtypes = [_P, _P, _P, _I, _I, _P]
    L.oracle_gemm_q8.argtypes = [_P, _P, _P, _I, _I, _P, _I, _i, _P]
    L.oracle_gemm_q8_rows.argtypes = [_P, _P, _P, _I, _I, _P, _I, _P, _I, _i, _P]
    L.oracle_gemm_f16.argtypes = [_P, _I, _I, _P, _I, _i, _P]
    L.oracle_dequant_q82.argtypes = [_P, _P, _P, _I, _I, _P]
    L.oracle_gemm_q82.argtypes = [_P, _P, _P, _I, _I, _P, _I, _i, _P]
    L.oracle_dequant_q4tp.argtypes = [_P, _P, _P, _I, _I, _P]
    L.oracle_gemm_q4tp.argtypes = [_P, _P, _P, _I, _I, _P, _I, _i, _P]
    L.oracle_argmax_rows.argtypes = [_P, _I, _I, _P]
    L.oracle_attn_prefill.argtypes = [_P, _P, _P, _I, _I, _I, _I, _I, _D, _P]
    L.oracle_add_rmsnorm.argtypes = [_P, _P, _I, _P, _D, _I, _I, _P, _P]
    L.oracle_router_logits_f64.argtypes = [_P, _P, _I, _I, _I, _P]
    L.oracle_router_logits_f32.argtypes = [_P, _P, _I, _I, _I, _P]
    L.oracle_route.argtypes = [_P, _I, _I, _I, _i, _P, _P, _P]
    L.oracle_group.argtypes = [_P, _I, _I, _I, _I, _P, _P]
    L.oracle_moe_experts_ungrouped.argtypes = [_P, _I, _I, _I, _P, _I, _P, _P, _P, _P, _P, _P, _P, _P]
    L.oracle_moe_experts_grouped.argtypes = [_P, _I, _I, _I, _I, _I, _P, _P, _I,
                                             _P, _P, _P, _P, _P, _P, _P, _P]
    L.oracle_moe_combine.argtypes = [_P, _P, _P, _P, _I, _I, _I, _P, _D, _P, _P]
    L.oracle_route_sigmoid.argtypes = [_P, _P, _I, _I, _I, _i, _D, _P, _P, _P]
    L.oracle_exp_f32.argtypes = [ctypes.c_float]
    L.oracle_exp_f32.restype = ctypes.c_float
    L.oracle_sigmoid_f32.argtypes = [ctypes.c_float]
    L.oracle_sigmoid_f32.restype = ctypes.c_float
    L.oracle_sigmoid_f32_array.argtypes = [_P, _I, _P]
    L.oracle_threads.restype = _i
    L.oracle_set_threads.argtypes = [_i]


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_P)


def threads() -> int:
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    """OpenMP threads of the oracle's parallel loops (for timing it)."""
    lib().oracle_set_threads(int(n))


def f16_to_f64(bits: int) -> float:
    """Value of one binary16 bit pattern (IEEE 754 definition)."""
    return lib().oracle_f16_to_f64(int(bits) & 0xFFFF)


def dequant_q8(q, scale, bias) -> np.ndarray:
    """w[r][c] = scale[r][c/32] * q[r][c] + bias[r][c/32]  (float64)."""
    q, scale, bias = _c(q, np.int8), _c(scale, np.float32), _c(bias, np.float32)
    rows, cols = q.shape
    w = np.empty((rows, cols), np.float64)
    lib().oracle_dequant_q8(_p(q), _p(scale), _p(bias), rows, cols, _p(w))
    return w


def gemm_q8(q, scale, bias, X, act: int = 0) -> np.ndarray:
    """Y[b][r] = act(sum_c w[r][c] X[b][c]); X [n][cols] (or [cols]); act 1 = relu^2."""
    q, scale, bias = _c(q, np.int8), _c(scale, np.float32), _c(bias, np.float32)
    vec = np.ndim(X) == 1
    X = _c(np.atleast_2d(X), np.float32)
    rows, cols = q.shape
    assert X.shape[1] == cols
    Y = np.empty((X.shape[0], rows), np.float64)
    lib().oracle_gemm_q8(_p(q), _p(scale), _p(bias), rows, cols, _p(X), X.shape[0], act, _p(Y))
    return Y[0] if vec else Y


def gemm_q8_rows(q, scale, bias, rows_idx, X, act: int = 0) -> np.ndarray:
    """The product restricted to the output rows ``rows_idx``: Y [n][len(rows_idx)]."""
    q, scale, bias = _c(q, np.int8), _c(scale, np.float32), _c(bias, np.float32)
    idx = _c(rows_idx, np.int64)
    X = _c(np.atleast_2d(X), np.float32)
    rows, cols = q.shape
    Y = np.empty((X.shape[0], idx.size), np.float64)
    lib().oracle_gemm_q8_rows(_p(q), _p(scale), _p(bias), rows, cols, _p(idx), idx.size,
                              _p(X), X.shape[0], act, _p(Y))
    return Y


def gemm_f16(W, X, act: int = 0) -> np.ndarray:
    """Y[b][r] = act(sum_c f16(W[r][c]) X[b][c]); W given as float16 (its bits are used)."""
    Wb = _c(np.asarray(W, dtype=np.float16).view(np.uint16), np.uint16)
    vec = np.ndim(X) == 1
    X = _c(np.atleast_2d(X), np.float32)
    rows, cols = Wb.shape
    Y = np.empty((X.shape[0], rows), np.float64)
    lib().oracle_gemm_f16(_p(Wb), rows, cols, _p(X), X.shape[0], act, _p(Y))
    return Y[0] if vec else Y


def _f16bits(a) -> np.ndarray:
    return _c(np.asarray(a, dtype=np.float16).view(np.uint16), np.uint16)


def dequant_q82(q, rs, cf) -> np.ndarray:
    """q8_2f: w[r][c] = f16(rs[r]) * f16(cf[c]) * q[r][c] (float64); rs, cf given as float16."""
    q = _c(q, np.int8)
    rows, cols = q.shape
    rb, cb = _f16bits(rs), _f16bits(cf)
    assert rb.size == rows and cb.size == cols
    w = np.empty((rows, cols), np.float64)
    lib().oracle_dequant_q82(_p(q), _p(rb), _p(cb), rows, cols, _p(w))
    return w


def gemm_q82(q, rs, cf, X, act: int = 0) -> np.ndarray:
    """Y[b][r] = act(sum_c rs[r] cf[c] q[r][c] X[b][c]); rs, cf float16; X [n][cols] or [cols]."""
    q = _c(q, np.int8)
    rows, cols = q.shape
    rb, cb = _f16bits(rs), _f16bits(cf)
    assert rb.size == rows and cb.size == cols
    vec = np.ndim(X) == 1
    X = _c(np.atleast_2d(X), np.float32)
    assert X.shape[1] == cols
    Y = np.empty((X.shape[0], rows), np.float64)
    lib().oracle_gemm_q82(_p(q), _p(rb), _p(cb), rows, cols, _p(X), X.shape[0], act, _p(Y))
    return Y[0] if vec else Y


def q4tp_code_bytes(cols: int) -> int:
    """Bytes of 5-bit group codes in one q4tp row (cols / 32 codes, packed)."""
    return (5 * (cols // 32) + 7) // 8


def _q4tp_args(nib, params, codes):
    nib = _c(nib, np.uint8)
    rows, half = nib.shape
    cols = 2 * half
    params = _c(params, np.uint32)
    codes = _c(codes, np.uint8)
    assert cols % 32 == 0 and params.shape == (rows,) and codes.shape == (rows, q4tp_code_bytes(cols))
    return nib, params, codes, rows, cols


def dequant_q4tp(nib, params, codes) -> np.ndarray:
    """w[r][c] = 2**(base_r + code_{r,c/32} step_r) (nib_r(c) - 8); nib uint8 [rows][cols/2]
    (column c in the low half of byte c/2 when c is even), params uint32 [rows] (base f16 low
    half, step f16 high half), codes uint8 [rows][ceil(5 cols/32 / 8)] (5-bit codes, LSB first)."""
    nib, params, codes, rows, cols = _q4tp_args(nib, params, codes)
    W = np.empty((rows, cols), np.float64)
    lib().oracle_dequant_q4tp(_p(nib), _p(params), _p(codes), rows, cols, _p(W))
    return W


def gemm_q4tp(nib, params, codes, X, act: int = 0) -> np.ndarray:
    """Y[b][r] = act(sum_c w[r][c] X[b][c]) with the q4tp weight of ``dequant_q4tp``."""
    nib, params, codes, rows, cols = _q4tp_args(nib, params, codes)
    vec = np.ndim(X) == 1
    X = _c(np.atleast_2d(X), np.float32)
    assert X.shape[1] == cols
    Y = np.empty((X.shape[0], rows), np.float64)
    lib().oracle_gemm_q4tp(_p(nib), _p(params), _p(codes), rows, cols, _p(X), X.shape[0], act, _p(Y))
    return Y[0] if vec else Y


def kv_append(kc, vc, k, v, pos0: int):
    """The caches with the pass's rows written at pos0 .. pos0 + n - 1 (copies; inputs kept)."""
    kc, vc = np.array(kc, np.float32), np.array(vc, np.float32)
    n = k.shape[0]
    kc[pos0:pos0 + n] = np.asarray(k, np.float32).reshape(kc[pos0:pos0 + n].shape)
    vc[pos0:pos0 + n] = np.asarray(v, np.float32).reshape(vc[pos0:pos0 + n].shape)
    return kc, vc


def attn_prefill(q, kc, vc, pos0: int, scale: float) -> np.ndarray:
    """Causal GQA over a pass: q [n][nh][hd], caches [ctx][nkv][hd] (rows up to pos0 + n - 1
    filled); o[b][h] = softmax_j(scale q[b][h] . kc[j][g]) . vc[j][g] over j <= pos0 + b,
    g = h / (nh / nkv); f64."""
    q = _c(q, np.float32)
    kc, vc = _c(kc, np.float32), _c(vc, np.float32)
    n, nh, hd = q.shape
    nkv = kc.shape[1]
    assert nh % nkv == 0 and kc.shape[2] == hd and vc.shape == kc.shape and kc.shape[0] >= pos0 + n
    o = np.empty((n, nh, hd), np.float64)
    lib().oracle_attn_prefill(_p(q), _p(kc), _p(vc), n, pos0, nh, nkv, hd, float(scale), _p(o))
    return o


def argmax_rows(L) -> np.ndarray:
    """ids[b] = smallest i with L[b][i] the row's largest logit above -3.0e38 (0 if none)."""
    vec = np.ndim(L) == 1
    L = _c(np.atleast_2d(L), np.float32)
    ids = np.empty(L.shape[0], np.uint32)
    lib().oracle_argmax_rows(_p(L), L.shape[0], L.shape[1], _p(ids))
    return ids[0] if vec else ids


def add_rmsnorm(h, delta, w, eps: float, delta_stride: int | None = None):
    """(h', out): h' = h + delta (delta may be None), out = w h' / sqrt(mean(h'^2) + eps).

    h is [n][H] (or [H]); delta rows are ``delta_stride`` floats apart (default H)."""
    vec = np.ndim(h) == 1
    h = _c(np.atleast_2d(h), np.float32)
    n, H = h.shape
    w = _c(w, np.float32)
    dptr = None
    if delta is not None:
        delta = _c(delta, np.float32)
        stride = H if delta_stride is None else delta_stride
        dptr = _p(delta)
    else:
        stride = H
    h_out = np.empty((n, H), np.float64)
    out = np.empty((n, H), np.float64)
    lib().oracle_add_rmsnorm(_p(h), dptr, stride, _p(w), eps, H, n, _p(h_out), _p(out))
    return (h_out[0], out[0]) if vec else (h_out, out)


def router_logits_f64(X, Wr) -> np.ndarray:
    X, Wr = _c(np.atleast_2d(X), np.float32), _c(Wr, np.float32)
    n, H = X.shape
    E = Wr.shape[0]
    out = np.empty((n, E), np.float64)
    lib().oracle_router_logits_f64(_p(X), _p(Wr), n, H, E, _p(out))
    return out


def router_logits_f32(X, Wr) -> np.ndarray:
    """f32 logits in the device's fixed summation order (see oracle.c)."""
    X, Wr = _c(np.atleast_2d(X), np.float32), _c(Wr, np.float32)
    n, H = X.shape
    assert H % 4 == 0
    E = Wr.shape[0]
    out = np.empty((n, E), np.float32)
    lib().oracle_router_logits_f32(_p(X), _p(Wr), n, H, E, _p(out))
    return out


def route(logits_f32, k: int, renorm: int = 0):
    """(sel int32 [n][k], rw f64 [n][k], probs f64 [n][E]) from f32 logits."""
    L = _c(np.atleast_2d(logits_f32), np.float32)
    n, E = L.shape
    sel = np.empty((n, k), np.int32)
    rw = np.empty((n, k), np.float64)
    probs = np.empty((n, E), np.float64)
    lib().oracle_route(_p(L), n, E, k, int(renorm), _p(sel), _p(rw), _p(probs))
    return sel, rw, probs


def exp_f32(x) -> np.ndarray:
    """exp in the fixed binary32 sequence the sigmoid router uses (see oracle.c)."""
    x = _c(np.atleast_1d(x), np.float32)
    return np.array([lib().oracle_exp_f32(float(v)) for v in x], np.float32)


def sigmoid_f32(l) -> np.ndarray:
    """sigma(l) = 1 / (1 + exp(-l)) as one fixed sequence of binary32 operations (see oracle.c)."""
    l = _c(np.atleast_1d(l), np.float32)
    out = np.empty(l.shape, np.float32)
    lib().oracle_sigmoid_f32_array(_p(l), l.size, _p(out))
    return out


def route_sigmoid(logits_f32, bias, k: int, norm: int = 1, scale: float = 1.0):
    """(sel int32 [n][k], rw f64 [n][k], choice f32 [n][E]): choice = sigmoid_f32(l) + bias
    (binary32), top k by choice (lower index on a tie), rw = sigmoid(l_sel) / den * scale in
    f64 with den = sum_t sigmoid(l_sel) + 1e-20 when norm, else 1."""
    L = _c(np.atleast_2d(logits_f32), np.float32)
    n, E = L.shape
    bias = _c(bias, np.float32)
    assert bias.shape == (E,) and 1 <= k <= E
    sel = np.empty((n, k), np.int32)
    rw = np.empty((n, k), np.float64)
    choice = np.empty((n, E), np.float32)
    lib().oracle_route_sigmoid(_p(L), _p(bias), n, E, k, int(norm), float(scale), _p(sel), _p(rw), _p(choice))
    return sel, rw, choice


def group(sel, E: int, cap: int | None = None):
    """(counts int32 [E], lists int32 [E][cap]); unused list slots hold -1."""
    sel = _c(np.atleast_2d(sel), np.int32)
    n, k = sel.shape
    cap = n if cap is None else cap
    counts = np.empty(E, np.int32)
    lists = np.full((E, cap), -1, np.int32)
    lib().oracle_group(_p(sel), n, k, E, cap, _p(counts), _p(lists))
    return counts, lists


def moe_experts(X, sel, up, down, grouped: bool = False, E: int | None = None):
    """(U [n*k][I], D [n*k][H]) of the routed expert FFN (relu^2 between up and down).

    ``up``/``down`` are (q, scale, bias) stacks: up q [E][I][H], down q [E][H][I]."""
    X = _c(np.atleast_2d(X), np.float32)
    sel = _c(np.atleast_2d(sel), np.int32)
    n, H = X.shape
    k = sel.shape[1]
    uq, us, ub = (_c(up[0], np.int8), _c(up[1], np.float32), _c(up[2], np.float32))
    dq, ds, db = (_c(down[0], np.int8), _c(down[1], np.float32), _c(down[2], np.float32))
    I = uq.shape[1]
    E = uq.shape[0] if E is None else E
    U = np.zeros((n * k, I), np.float64)
    D = np.zeros((n * k, H), np.float64)
    if grouped:
        counts, lists = group(sel, E)
        lib().oracle_moe_experts_grouped(_p(X), n, H, I, E, k, _p(counts), _p(lists), n,
                                         _p(uq), _p(us), _p(ub), _p(dq), _p(ds), _p(db),
                                         _p(U), _p(D))
    else:
        lib().oracle_moe_experts_ungrouped(_p(X), n, H, I, _p(sel), k, _p(uq), _p(us), _p(ub),
                                           _p(dq), _p(ds), _p(db), _p(U), _p(D))
    return U, D


def moe_combine(h, D, rw, w, eps: float, shared=None):
    """(h', out): h' = h + shared[b] + sum_t rw[b][t] D[b*k+t] (slot order; shared optional),
    out = rmsnorm(h') * w."""
    h = _c(np.atleast_2d(h), np.float32)
    sh = None if shared is None else _c(np.atleast_2d(shared), np.float32)
    D = _c(D, np.float64)
    rw = _c(np.atleast_2d(rw), np.float64)
    n, H = h.shape
    k = rw.shape[1]
    w = _c(w, np.float32)
    h_out = np.empty((n, H), np.float64)
    out = np.empty((n, H), np.float64)
    assert sh is None or sh.shape == (n, H)
    lib().oracle_moe_combine(_p(h), None if sh is None else _p(sh), _p(D), _p(rw), n, k, H, _p(w), eps,
                             _p(h_out), _p(out))
    return h_out, out


def moe_pass(X, h, Wr, up, down, w, eps: float, k: int, renorm: int = 0, sigmoid=None, shared=None):
    """The whole routed-MoE pass; returns a dict of every stage.  ``sigmoid`` = (bias, norm,
    scale) selects the sigmoid router (``route_sigmoid``) instead of softmax; ``shared``
    [n][H] is the dense term the combine adds before the slots."""
    logits = router_logits_f32(X, Wr)
    if sigmoid is None:
        sel, rw, probs = route(logits, k, renorm)
    else:
        sel, rw, probs = route_sigmoid(logits, sigmoid[0], k, sigmoid[1], sigmoid[2])
    E = Wr.shape[0]
    counts, lists = group(sel, E)
    U, D = moe_experts(X, sel, up, down, grouped=True, E=E)
    h_out, out = moe_combine(h, D, rw, w, eps, shared=shared)
    return {"logits": logits, "logits_f64": router_logits_f64(X, Wr), "sel": sel, "rw": rw,
            "probs": probs, "counts": counts, "lists": lists, "U": U, "D": D,
            "h": h_out, "out": out}


def rel_err(got, ref) -> float:
    """max_i |g_i - r_i| / max(|r_i|, rms(r)): elementwise relative error floored at
    the reference tensor's RMS (plain relative error is unbounded at outputs near 0)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), rms)
    den = np.where(den == 0.0, 1.0, den)
    return float(np.max(np.abs(got - ref) / den))
