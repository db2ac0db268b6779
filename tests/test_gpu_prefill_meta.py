"""prefill_frame_q8_meta: the prefill frame with the pass size {n, pos0} in a
device buffer, so that ONE captured graph serves every pass of a prompt.  Each
pass (graph replay after the buffer is set) must equal prefill_frame_q8 on the
same rows bit for bit; a full 420-position prompt (6 x 64 + 36) runs from one
graph and its last pass is checked stage by stage against the oracle; passes
outside the buffers write nothing."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import assert_staged, oracle_frame_staged, q8_dev, staged_errors, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def _weights(f):
    return {k: q8_dev(f[k], torch) for k in ("qkv", "up", "down", "head")}


def _static_passes(pg, W, f, X0, H0, passes):
    """The same prompt as separate prefill_frame_q8 calls on row slices."""
    H = H0.clone()
    R, hidden = X0.shape
    out = {"qkv": torch.empty(R, W["qkv"].rows, device="cuda"), "u": torch.empty(R, W["up"].rows, device="cuda"),
           "d": torch.empty(R, hidden, device="cuda"), "logits": torch.empty(R, W["head"].rows, device="cuda")}
    w1, w2 = to_dev(f["w1"], torch), to_dev(f["w2"], torch)
    for n, p0 in passes:
        ws = torch.empty(pg.prefill_frame_q8_workspace_bytes(hidden, W["qkv"].rows, W["up"].rows, W["head"].rows, n),
                         dtype=torch.uint8, device="cuda")
        Hs = H[p0:p0 + n].clone()
        o = {k: torch.empty(n, v.shape[1], device="cuda") for k, v in out.items()}
        pg.prefill_frame_q8(W["qkv"], W["up"], W["down"], W["head"], w1, w2, f["eps"], X0[p0:p0 + n].contiguous(),
                            Hs, o, ws)
        H[p0:p0 + n] = Hs
        for k in out:
            out[k][p0:p0 + n] = o[k]
    torch.cuda.synchronize()
    return out, H


@pytest.mark.parametrize("name,rows", [("small", 140), ("small", 64), ("small", 5), ("full", 420)])
def test_prompt_one_graph_equals_passes(pg, oracle, name, rows):
    shape = synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=1000) if name == "small" else synth.FrameShape()
    _case(f"prefill_frame_q8_meta {name} rows={rows}")
    f = synth.frame_weights(31, shape)
    inp = synth.frame_inputs(31, rows, shape.hidden)
    W = _weights(f)
    X0, H0 = to_dev(inp["x0"], torch), to_dev(inp["h0"], torch)
    H = H0.clone()
    pr = pg.Prompt(W["qkv"], W["up"], W["down"], W["head"], to_dev(f["w1"], torch), to_dev(f["w2"], torch), f["eps"],
                   X0, H)
    pr.capture()
    for k in pr.buf:
        pr.buf[k].fill_(np.nan)
    pr.run()
    torch.cuda.synchronize()
    ref, H_ref = _static_passes(pg, W, f, X0, H0, pr.passes)
    for k in ref:
        assert torch.equal(pr.buf[k], ref[k]), k
    assert torch.equal(H, H_ref)
    # the last pass, stage by stage against the oracle (on its own rows)
    n, p0 = pr.passes[-1]
    sl = slice(p0, p0 + n)
    dev = {k: pr.buf[k][sl].cpu().numpy() for k in ("qkv", "u", "d", "logits")}
    dev["h2"] = H[sl].cpu().numpy()
    r = oracle_frame_staged(oracle, f, inp["x0"][sl], inp["h0"][sl], dev)
    assert_staged(staged_errors(oracle, r, dev))


def test_prompt_replays_repeat(pg):
    """Replays of the one graph, with eager work between them, repeat bit for bit."""
    _case("prefill_frame_q8_meta replays")
    shape = synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=1000)
    f = synth.frame_weights(32, shape)
    inp = synth.frame_inputs(32, 100, shape.hidden)
    W = _weights(f)
    X0, H0 = to_dev(inp["x0"], torch), to_dev(inp["h0"], torch)
    H = H0.clone()
    pr = pg.Prompt(W["qkv"], W["up"], W["down"], W["head"], to_dev(f["w1"], torch), to_dev(f["w2"], torch), f["eps"],
                   X0, H)
    pr.capture()
    pr.run()
    first = {k: v.clone() for k, v in pr.buf.items()}
    H1 = H.clone()
    for _ in range(3):
        H.copy_(H0)
        _ = (X0 * 2).sum().item()
        pr.run()
        torch.cuda.synchronize()
        for k in first:
            assert torch.equal(pr.buf[k], first[k]), k
        assert torch.equal(H, H1)


@pytest.mark.parametrize("meta", [(0, 0), (65, 0), (-3, 0), (8, -1), (8, 95), (64, 40)])
def test_meta_outside_writes_nothing(pg, meta):
    """n outside 1..64, pos0 < 0 or pos0 + n beyond the 100 rows: the pass writes nothing."""
    _case(f"prefill_frame_q8_meta invalid meta {meta}")
    shape = synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=1000)
    f = synth.frame_weights(33, shape)
    inp = synth.frame_inputs(33, 100, shape.hidden)
    W = _weights(f)
    X0, H = to_dev(inp["x0"], torch), to_dev(inp["h0"], torch)
    H_before = H.clone()
    pr = pg.Prompt(W["qkv"], W["up"], W["down"], W["head"], to_dev(f["w1"], torch), to_dev(f["w2"], torch), f["eps"],
                   X0, H)
    for k in pr.buf:
        pr.buf[k].fill_(7.0)
    pr.meta.copy_(torch.tensor(meta, dtype=torch.int32))
    pr._call()
    torch.cuda.synchronize()
    assert torch.equal(H, H_before)
    for k in pr.buf:
        assert bool((pr.buf[k] == 7.0).all()), k


def test_meta_errors(pg):
    _case("prefill_frame_q8_meta errors")
    L = pg.lib()
    shape = synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=1000)
    f = synth.frame_weights(34, shape)
    W = _weights(f)
    Ws = [pg._lib.PgQ8(w.q.data_ptr(), w.scale.data_ptr(), w.bias.data_ptr(), w.rows, w.cols)
          for w in W.values()]
    R = 70
    keep = []

    def vec(nf):
        t = torch.zeros(nf, device="cuda")
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    ws = torch.empty(pg.prefill_frame_q8_workspace_bytes(1024, 1536, 2048, 1000, 64), dtype=torch.uint8, device="cuda")
    meta = torch.tensor([8, 0], dtype=torch.int32, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(meta_p, rows=R, ws_bytes=ws.numel()):
        return L.prefill_frame_q8_meta(*[ctypes.byref(w) for w in Ws], vec(1024), vec(1024), 1e-6, vec(R * 1024),
                                       vec(R * 1024), rows, meta_p, vec(R * 1536), vec(R * 2048), vec(R * 1024),
                                       vec(R * 1000), ctypes.c_void_p(ws.data_ptr()), ws_bytes, s)

    assert call(ctypes.c_void_p(meta.data_ptr())) == pg.PG_OK
    torch.cuda.synchronize()
    assert call(None) == pg.PG_EINVAL
    assert call(ctypes.c_void_p(meta.data_ptr()), rows=0) == pg.PG_EINVAL
    assert call(ctypes.c_void_p(meta.data_ptr()), ws_bytes=ws.numel() - 256) == pg.PG_EWORKSPACE
