"""Causal grouped-query prefill attention (attn_prefill) and the KV append
(attn_kv_append) against the CPU oracle, through the C ABI: the frame's head
layout (32 query heads, 8 KV heads of 128) for a first pass and for a pass late
in a 4096-position context (several key splits), a ragged last query block,
other head ratios and hd = 64, closed-form cases, and the argument errors."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

TOL_ATTN = 1e-5   # f32 scores, exp and sums over up to 4096 keys, against f64


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _run(pg, c):
    kc, vc = to_dev(c["kc"], torch), to_dev(c["vc"], torch)
    pg.attn_kv_append(to_dev(c["k"], torch), to_dev(c["v"], torch), kc, vc, c["pos0"])
    o = pg.attn_prefill(to_dev(c["q"], torch), kc, vc, c["pos0"], c["scale"])
    torch.cuda.synchronize()
    return o.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()


@pytest.mark.parametrize("n,pos0,nh,nkv,hd", [(64, 0, 32, 8, 128), (64, 4032, 32, 8, 128), (37, 100, 32, 8, 128),
                                              (1, 0, 32, 8, 128), (1, 777, 32, 8, 128), (20, 300, 8, 8, 64),
                                              (64, 1000, 16, 2, 128), (9, 64, 8, 1, 64)])
def test_attn_parity(pg, oracle, n, pos0, nh, nkv, hd):
    _case(f"attn n={n} pos0={pos0} nh={nh} nkv={nkv} hd={hd}")
    c = synth.attn_pass(n + pos0, n, pos0, nh, nkv, hd)
    o, kc, vc = _run(pg, c)
    kc_ref, vc_ref = oracle.kv_append(c["kc"], c["vc"], c["k"], c["v"], pos0)
    assert np.array_equal(kc, kc_ref) and np.array_equal(vc, vc_ref), "KV append"
    ref = oracle.attn_prefill(c["q"], kc_ref, vc_ref, pos0, c["scale"])
    err = oracle.rel_err(o, ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_ATTN


def test_attn_rising_and_jumping_scores(pg, oracle):
    """Scores that climb in a sawtooth over the context (up by about 6 in base-2 units a 64-key
    tile, falling back every 320 keys) and jump by about 17 at one key: each split's running
    maximum moves by steps below and above the softmax's rescaling threshold, and the merge
    meets splits of different maxima.  q has one nonzero dim, so the f32 scores carry no
    long sums and the test measures the softmax, not the scores' rounding."""
    _case("attn rising and jumping scores")
    n, pos0 = 64, 4032
    c = synth.attn_pass(17, n, pos0)
    j = np.arange(pos0 + n)
    saw = (18.0 * ((j % 320) / 320.0)).astype(np.float32)   # scores rise by 16 over 320 keys
    c["kc"][:pos0, :, 0] += saw[:pos0, None]
    c["k"][:, :, 0] += saw[pos0:, None]
    c["kc"][2000, :, 0] += 13.5
    c["q"][:] = 0.0
    c["q"][:, :, 0] = 10.0
    o, kc, vc = _run(pg, c)
    kc_ref, vc_ref = oracle.kv_append(c["kc"], c["vc"], c["k"], c["v"], pos0)
    ref = oracle.attn_prefill(c["q"], kc_ref, vc_ref, pos0, c["scale"])
    err = oracle.rel_err(o, ref)
    print(f"[info] rel err {err:.2e}", flush=True)
    assert err <= TOL_ATTN


def test_attn_closed_forms(pg, oracle):
    """The first position of a first pass sees only its own key: o = its v.  A zero query
    weighs all visible keys equally: o is the mean of their v rows."""
    _case("attn closed forms")
    c = synth.attn_pass(5, 16, 0, 8, 2, 64)
    c["q"][3:] = 0.0
    o, kc, vc = _run(pg, c)
    for h in range(8):
        np.testing.assert_allclose(o[0, h], c["v"][0, h // 4], rtol=1e-6, atol=1e-7)
    for b in range(3, 16):
        for h in range(8):
            np.testing.assert_allclose(o[b, h], vc[:b + 1, h // 4].astype(np.float64).mean(0), rtol=1e-5, atol=1e-6)


def test_attn_cache_rows_past_the_pass_unread(pg, oracle):
    """Rows of the cache past pos0 + n hold huge values; causality must keep them out."""
    _case("attn causal limit")
    c = synth.attn_pass(6, 30, 200, 32, 8, 128, ctx=400)
    c["kc"][230:] = 1e3
    c["vc"][230:] = 1e9
    o, kc, vc = _run(pg, c)
    ref = oracle.attn_prefill(c["q"], kc, vc, 200, c["scale"])
    assert oracle.rel_err(o, ref) <= TOL_ATTN and np.abs(o).max() < 100


def test_attn_errors(pg):
    _case("attn errors")
    L = pg.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    q = torch.zeros(4 * 8 * 64, device="cuda")
    kc = torch.zeros(16 * 2 * 64, device="cuda")
    o = torch.zeros(4 * 8 * 64, device="cuda")
    need = L.attn_prefill_workspace_bytes(4, 4, 8, 2, 64)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    P = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)

    def call(n=4, pos0=4, nh=8, nkv=2, hd=64, wsb=need, qp=None):
        return L.attn_prefill(qp or P(q), P(kc), P(kc), n, pos0, nh, nkv, hd, 0.125, P(o), P(ws), wsb, s)

    assert call() == pg.PG_OK
    torch.cuda.synchronize()
    assert call(hd=96) == pg.PG_EUNSUPPORTED
    assert call(nh=6, nkv=4) == pg.PG_EINVAL              # heads not a multiple of KV heads
    assert call(nh=24, nkv=1) == pg.PG_EUNSUPPORTED       # 64 % 24 != 0
    assert call(n=65) == pg.PG_EUNSUPPORTED
    assert call(wsb=need - 1) == pg.PG_EWORKSPACE
    assert call(qp=P(q, 4)) == pg.PG_EINVAL
    assert L.attn_kv_append(P(q), P(q), 4, 128, 10, P(kc), P(kc), 12, s) == pg.PG_EINVAL   # past the capacity
