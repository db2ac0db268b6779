"""The sigmoid + bias router (moe_route_sigmoid) and the routed-MoE pass with it
and a shared-expert term (moe_grouped_sigmoid), against the CPU oracle through
the C ABI.

The choice value sigmoid(l) + bias decides integers, so both sides take it as
the same fixed sequence of correctly rounded binary32 operations (a Cody-Waite
reduced exp with a Taylor polynomial, one add, one divide, then the bias add);
the selection must equal the oracle's bit for bit, order included, at every
position.  The weights are held to the f32 tolerance against the f64
definition; grouping is exact, and the pass's outputs are held to the q8
tolerance on every position."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import TOL_F32, TOL_Q8, q8_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def _check_selection(oracle, L, bias, k, norm, scale, sel, rw):
    """Selection equal to the oracle's at every position; weights at the f32 tolerance."""
    sel_ref, rw_ref, _ = oracle.route_sigmoid(L, bias, k, norm, scale)
    bad = np.flatnonzero(~np.all(sel == sel_ref, axis=1))
    assert bad.size == 0, (bad[:4], sel[bad[:4]], sel_ref[bad[:4]])
    assert oracle.rel_err(rw, rw_ref) <= TOL_F32


@pytest.mark.parametrize("E,k", [(6, 2), (64, 6), (128, 6), (256, 8), (1000, 16), (16, 16)])
@pytest.mark.parametrize("norm", [0, 1])
def test_route_sigmoid_parity(pg, oracle, E, k, norm):
    _case(f"route_sigmoid E={E} k={k} norm={norm}")
    rng = np.random.default_rng(E * 3 + k + norm)
    n = 64
    L = synth.normal(rng, (n, E))
    bias = synth.router_bias(rng, E)
    sel, rw = pg.moe_route_sigmoid(to_dev(L, torch), to_dev(bias, torch), k, renorm=norm, scale=2.5)
    torch.cuda.synchronize()
    _check_selection(oracle, L, bias, k, norm, 2.5, sel.cpu().numpy(), rw.cpu().numpy())


def test_route_sigmoid_wide_logits(pg, oracle):
    """Logits over [-120, 120] (past the clamp at 80 on both sides, and where sigmoid
    saturates), many near-equal values: still the oracle's selection bit for bit."""
    _case("route_sigmoid wide logits")
    rng = np.random.default_rng(77)
    n, E, k = 64, 256, 8
    L = (rng.standard_normal((n, E)) * 40.0).astype(np.float32)
    L[:, :32] = rng.uniform(-120, 120, (n, 32)).astype(np.float32)
    L[:, 32:64] = (L[:, 64:96] + np.float32(1e-6)).astype(np.float32)   # near ties
    bias = synth.router_bias(rng, E)
    bias[:16] = 0.0
    sel, rw = pg.moe_route_sigmoid(to_dev(L, torch), to_dev(bias, torch), k, renorm=1, scale=1.0)
    torch.cuda.synchronize()
    _check_selection(oracle, L, bias, k, 1, 1.0, sel.cpu().numpy(), rw.cpu().numpy())


def test_route_sigmoid_exact_ties(pg, oracle):
    """Equal logits and equal bias give equal f32 choice values on any exp: the lower index
    must come first, bit for bit."""
    _case("route_sigmoid ties")
    rng = np.random.default_rng(9)
    n, E, k = 16, 40, 6
    L = synth.normal(rng, (n, E))
    bias = synth.router_bias(rng, E)
    bias[3] = 0.5                              # 3, 17, 30 tie at the top (choice > 1.39)
    L[:, 3] += 10.0
    for a, b in [(3, 17), (3, 30), (8, 9)]:
        L[:, b] = L[:, a]
        bias[b] = bias[a]
    sel, _ = pg.moe_route_sigmoid(to_dev(L, torch), to_dev(bias, torch), k)
    torch.cuda.synchronize()
    sel = sel.cpu().numpy()
    assert (sel[:, :3] == [3, 17, 30]).all()


def _run(pg, c, bias, norm, scale, shared):
    up, down = q8_dev(c["up"], torch), q8_dev(c["down"], torch)
    h = to_dev(c["h"], torch)
    o = pg.moe_grouped(to_dev(c["X"], torch), to_dev(c["Wr"], torch), up, down, h, to_dev(c["w"], torch),
                       c["eps"], c["top_k"], renorm=norm, router_bias=to_dev(bias, torch), scale=scale,
                       shared=None if shared is None else to_dev(shared, torch))
    torch.cuda.synchronize()
    o = {key: v.cpu().numpy() for key, v in o.items()}
    o["h"] = h.cpu().numpy()
    return o


def _check_pass(oracle, c, o, bias, norm, scale, shared, pos=None):
    E = c["Wr"].shape[0]
    L = oracle.router_logits_f32(c["X"], c["Wr"])
    assert np.array_equal(o["logits"].view(np.uint32), L.view(np.uint32)), "logits bits"
    _check_selection(oracle, L, bias, c["top_k"], norm, scale, o["sel"], o["route_w"])
    counts, lists = oracle.group(o["sel"], E)
    assert np.array_equal(o["counts"], counts), "counts"
    for e in range(E):
        assert np.array_equal(o["lists"][e, :counts[e]], lists[e, :counts[e]]), f"list {e}"
    sel = o["sel"]
    s = _sigmoid(np.take_along_axis(L.astype(np.float64), sel.astype(np.int64), 1))
    rw = s / ((s.sum(1, keepdims=True) + 1e-20) if norm else 1.0) * scale
    pos = np.arange(c["X"].shape[0]) if pos is None else pos
    up = (c["up"].q, c["up"].scale, c["up"].bias)
    down = (c["down"].q, c["down"].scale, c["down"].bias)
    _, D = oracle.moe_experts(c["X"][pos], sel[pos], up, down, grouped=False)
    h_ref, out_ref = oracle.moe_combine(c["h"][pos], D, rw[pos], c["w"], c["eps"],
                                        shared=None if shared is None else shared[pos])
    assert oracle.rel_err(o["h"][pos], h_ref) <= TOL_Q8
    assert oracle.rel_err(o["out"][pos], out_ref) <= TOL_Q8


@pytest.mark.parametrize("shape", [synth.MoEShape(n=8, hidden=64, inter=96, experts=6, top_k=2),
                                   synth.MoEShape(n=40, hidden=256, inter=160, experts=16, top_k=4),
                                   synth.MoEShape(n=1, hidden=32, inter=32, experts=1, top_k=1),
                                   synth.MoEShape(n=48, hidden=4096, inter=160, experts=4, top_k=2)])
@pytest.mark.parametrize("norm,shared", [(1, True), (0, False)])
def test_moe_sigmoid_small(pg, oracle, shape, norm, shared):
    _case(f"moe sigmoid {shape} norm={norm} shared={shared}")
    c = synth.moe(shape.n + 7 * shape.experts, shape)
    rng = np.random.default_rng(shape.n + shape.experts)
    bias = synth.router_bias(rng, shape.experts)
    sh = synth.normal(rng, (shape.n, shape.hidden)) if shared else None
    o = _run(pg, c, bias, norm, 1.75, sh)
    _check_pass(oracle, c, o, bias, norm, 1.75, sh)


def test_moe_sigmoid_full_128_experts(pg, oracle):
    """The 64-position, 128-expert (2688 -> 1856 -> 2688, top-6) pass with the sigmoid router
    and a shared term; residual and norm outputs on every position."""
    _case("moe sigmoid full")
    c = synth.moe(0)
    rng = np.random.default_rng(21)
    bias = synth.router_bias(rng, c["Wr"].shape[0])
    sh = synth.normal(rng, c["h"].shape)
    o = _run(pg, c, bias, 1, 2.5, sh)
    print(f"[info] distinct experts selected: {int((o['counts'] > 0).sum())}", flush=True)
    _check_pass(oracle, c, o, bias, 1, 2.5, sh)


def test_moe_sigmoid_errors(pg):
    _case("moe sigmoid errors")
    L = pg.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    logits = torch.zeros(4 * 8, device="cuda")
    bias = torch.zeros(8, device="cuda")
    sel = torch.zeros(4 * 2, dtype=torch.int32, device="cuda")
    rw = torch.zeros(4 * 2, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    assert L.moe_route_sigmoid(P(logits), P(bias), 4, 8, 2, 1, 1.0, P(sel), P(rw), s) == pg.PG_OK
    torch.cuda.synchronize()
    assert L.moe_route_sigmoid(P(logits), None, 4, 8, 2, 1, 1.0, P(sel), P(rw), s) == pg.PG_EINVAL
    assert L.moe_route_sigmoid(P(logits), P(bias), 4, 8, 9, 1, 1.0, P(sel), P(rw), s) == pg.PG_EUNSUPPORTED
    assert L.moe_route_sigmoid(P(logits), P(bias), 0, 8, 2, 1, 1.0, P(sel), P(rw), s) == pg.PG_EINVAL
