"""Layer frames on the libpg calls (decode at one position, prefill over a pass):
stage-isolated parity of the calls the frame runs (each stage against the
definition applied to the device's own input to it), the end-to-end chain, and
graph replays equal to eager runs."""
import numpy as np
import pytest

import synth
from helpers import TOL_F32, TOL_Q8, assert_staged, oracle_frame, oracle_frame_staged, q8_dev, staged_errors, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

SMALL = synth.FrameShape(hidden=256, qkv=384, inter=512, vocab=1000)


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _frame(pg, f, n):
    return pg.Frame(q8_dev(f["qkv"], torch), q8_dev(f["up"], torch), q8_dev(f["down"], torch),
                    q8_dev(f["head"], torch), to_dev(f["w1"], torch), to_dev(f["w2"], torch),
                    f["eps"], n=n)


def _np(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("n", [1, 5, 64])
def test_frame_parity(pg, oracle, n):
    """Stage-isolated parity of the calls ``Frame.stages`` runs, each stage checked
    right after it runs against the definition applied to the device's own input
    to it; then the end-to-end chain against the oracle's chain."""
    _case(f"frame n={n}")
    f = synth.frame_weights(1, SMALL)
    inp = synth.frame_inputs(1, n, SMALL.hidden)
    fr = _frame(pg, f, n)
    H = SMALL.hidden
    x0 = to_dev(inp["x0"], torch)
    h = to_dev(inp["h0"], torch)
    stages = fr.stages(x0, h)
    b = fr.buf
    g = lambda m, x, act=0: oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
    if n == 1:
        # decode: gemv_q8_residual (QKV), gemv_q8_normed (up), gemv_q8_residual (down), gemv_q8_normed (head)
        h0 = inp["h0"].reshape(-1)
        stages[0]()
        torch.cuda.synchronize()
        qkv = _np(b["qkv"]).reshape(-1)
        assert oracle.rel_err(qkv, g(f["qkv"], inp["x0"].reshape(-1))) <= TOL_Q8
        h1 = _np(h).reshape(-1)
        assert oracle.rel_err(h1, (h0 + qkv[:H]).astype(np.float32)) <= TOL_F32
        assert oracle.rel_err(_np(b["xw1"]), f["w1"] * h1) <= TOL_F32
        ss = float(np.sum(h1.astype(np.float64) ** 2))
        assert abs(float(np.sum(_np(b["p1"]), dtype=np.float64)) - ss) <= TOL_F32 * ss
        stages[1]()
        torch.cuda.synchronize()
        _, x1 = oracle.add_rmsnorm(h1, None, f["w1"], f["eps"])
        assert oracle.rel_err(_np(b["u"]).reshape(-1), g(f["up"], x1, act=1)) <= TOL_Q8
        stages[2]()
        torch.cuda.synchronize()
        u = _np(b["u"]).reshape(-1)
        d = _np(b["d"]).reshape(-1)
        assert oracle.rel_err(d, g(f["down"], u)) <= TOL_Q8
        h2 = _np(h).reshape(-1)
        assert oracle.rel_err(h2, (h1 + d).astype(np.float32)) <= TOL_F32
        assert oracle.rel_err(_np(b["xw2"]), f["w2"] * h2) <= TOL_F32
        ss = float(np.sum(h2.astype(np.float64) ** 2))
        assert abs(float(np.sum(_np(b["p2"]), dtype=np.float64)) - ss) <= TOL_F32 * ss
        stages[3]()
        torch.cuda.synchronize()
        _, x2 = oracle.add_rmsnorm(h2, None, f["w2"], f["eps"])
        assert oracle.rel_err(_np(b["logits"]).reshape(-1), g(f["head"], x2)) <= TOL_Q8
    else:
        # prefill: the frame is one prefill_frame_q8 call
        assert len(stages) == 1
        stages[0]()
        torch.cuda.synchronize()
        dev = {k: _np(b[k]) for k in ("qkv", "u", "d", "logits")}
        dev["h2"] = _np(h)
        ref = oracle_frame_staged(oracle, f, inp["x0"], inp["h0"], dev)
        assert_staged(staged_errors(oracle, ref, dev))
    # end to end: the chain's error is reported; the first product and the residual are asserted
    ref = oracle_frame(oracle, f, inp["x0"], inp["h0"])
    h = to_dev(inp["h0"], torch)
    logits = fr.run(x0, h).cpu().numpy()
    assert oracle.rel_err(_np(fr.buf["qkv"]), ref["qkv"]) <= TOL_Q8
    assert oracle.rel_err(h.cpu().numpy(), ref["h2"]) <= TOL_Q8
    err = oracle.rel_err(logits, ref["logits"])
    print(f"[info] end-to-end logits rel err n={n}: {err:.2e}", flush=True)


@pytest.mark.parametrize("n", [1, 64])
def test_frame_graph_replay(pg, n):
    """Graph replays (with eager work and syncs in between) give the eager result each time."""
    _case(f"frame graph n={n}")
    f = synth.frame_weights(2, SMALL)
    inp = synth.frame_inputs(2, n, SMALL.hidden)
    fr = _frame(pg, f, n)
    x0 = to_dev(inp["x0"], torch)
    h = to_dev(inp["h0"], torch)
    h0 = h.clone()
    eager = fr.run(x0, h).clone()
    h_eager = h.clone()
    h.copy_(h0)
    fr.capture(x0, h)
    for _ in range(4):
        h.copy_(h0)
        torch.cuda.synchronize()
        fr.replay()
        torch.cuda.synchronize()
        assert torch.equal(fr.buf["logits"], eager)
        assert torch.equal(h, h_eager)
        _ = (x0 * 2).sum().item()   # unrelated eager work between replays
