"""Layer frames on the libpg calls (decode at one position, prefill over a pass):
stage-isolated parity (every device stage fed the oracle's f32 input),
end-to-end parity of the chain, and graph replays equal to eager runs."""
import numpy as np
import pytest

import synth
from helpers import TOL_Q8, oracle_frame, q8_dev, to_dev

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


@pytest.mark.parametrize("n", [1, 5, 64])
def test_frame_parity(pg, oracle, n):
    _case(f"frame n={n}")
    f = synth.frame_weights(1, SMALL)
    inp = synth.frame_inputs(1, n, SMALL.hidden)
    ref = oracle_frame(oracle, f, inp["x0"], inp["h0"])
    fr = _frame(pg, f, n)
    # stage-isolated: each device stage gets the oracle's f32 input
    mm = fr._mm
    y = torch.empty(n, SMALL.qkv, device="cuda")
    mm("qkv", to_dev(inp["x0"], torch), y)
    assert oracle.rel_err(y.cpu().numpy(), ref["qkv"]) <= TOL_Q8
    y = torch.empty(n, SMALL.inter, device="cuda")
    mm("up", to_dev(ref["x1"], torch), y, act=1)
    assert oracle.rel_err(y.cpu().numpy(), ref["u"]) <= TOL_Q8
    y = torch.empty(n, SMALL.hidden, device="cuda")
    mm("down", to_dev(ref["u"], torch), y)
    assert oracle.rel_err(y.cpu().numpy(), ref["d"]) <= TOL_Q8
    y = torch.empty(n, SMALL.vocab, device="cuda")
    mm("head", to_dev(ref["x2"], torch), y)
    assert oracle.rel_err(y.cpu().numpy(), ref["logits"]) <= TOL_Q8
    # end to end
    h = to_dev(inp["h0"], torch)
    logits = fr.run(to_dev(inp["x0"], torch), h).cpu().numpy()
    assert oracle.rel_err(h.cpu().numpy(), ref["h2"]) <= TOL_Q8
    err = oracle.rel_err(logits, ref["logits"])
    print(f"[info] end-to-end logits rel err n={n}: {err:.2e}", flush=True)
    assert err <= 4 * TOL_Q8


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
