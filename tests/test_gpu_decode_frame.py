"""decode_frame_q8: the whole q8 decode frame at one position in one
persistent launch, against the oracle's frame chain (every intermediate
rounded to its f32 buffer), at shapes that exercise empty, odd and
half-row shares, and at the full frame size; repeated launches on one
workspace (the barrier counters reset themselves) give identical results."""
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


SHAPES = {
    # hidden 1024: shares of 4 (hidden), 6 (qkv), 8 (up), 12 (head) rows per workgroup
    "h1024": synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=3000),
    # odd QKV row count, an odd number of steps in the down rows (no half-row units),
    # a head smaller than the grid (most workgroups own no head rows)
    "odd": synth.FrameShape(hidden=1024, qkv=1025, inter=3072, vocab=100),
    "h2048": synth.FrameShape(hidden=2048, qkv=3072, inter=6144, vocab=5000),
    "full": synth.FrameShape(),
}


def _run(pg, f, inp, ws=None):
    H = f["qkv"].cols
    W = {k: q8_dev(f[k], torch) for k in ("qkv", "up", "down", "head")}
    out = {"qkv": torch.empty(W["qkv"].rows, device="cuda"), "u": torch.empty(W["up"].rows, device="cuda"),
           "d": torch.empty(H, device="cuda"), "logits": torch.empty(W["head"].rows, device="cuda")}
    if ws is None:
        ws = pg.decode_frame_q8_workspace(H, W["up"].rows)
    h = to_dev(inp["h0"][0], torch)
    pg.decode_frame_q8(W["qkv"], W["up"], W["down"], W["head"], to_dev(f["w1"], torch), to_dev(f["w2"], torch),
                       f["eps"], to_dev(inp["x0"][0], torch), h, out, ws)
    torch.cuda.synchronize()
    return W, out, h, ws


@pytest.mark.parametrize("name", list(SHAPES))
def test_decode_frame_parity(pg, oracle, name):
    """Stage-isolated: every output of the persistent launch is compared with the
    definition applied to the device's own input to that stage."""
    shape = SHAPES[name]
    _case(f"decode_frame_q8 {name} {shape}")
    f = synth.frame_weights(11, shape)
    inp = synth.frame_inputs(11, 1, shape.hidden)
    _, out, h, ws = _run(pg, f, inp)
    pg.decode_frame_q8_status(ws)          # raises PGError (PG_ETIMEOUT) if a barrier wait gave up
    assert pg.decode_frame_timeouts(ws) == 0
    dev = {k: v.cpu().numpy() for k, v in out.items()}
    dev["h2"] = h.cpu().numpy()
    ref = oracle_frame_staged(oracle, f, inp["x0"], inp["h0"], dev)
    errs = staged_errors(oracle, ref, dev)
    print(f"[info] {name} rel errs " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert_staged(errs)


def test_decode_frame_repeat_and_vs_gemv_frame(pg):
    """Launches back to back on one workspace give bit-identical outputs
    (fixed summation orders; the barrier counters clear themselves), and the
    result matches the four-GEMV frame closely."""
    shape = SHAPES["h2048"]
    _case(f"decode_frame_q8 repeat {shape}")
    f = synth.frame_weights(12, shape)
    inp = synth.frame_inputs(12, 1, shape.hidden)
    W, out, h, ws = _run(pg, f, inp)
    first = {k: v.clone() for k, v in out.items()}
    h_first = h.clone()
    h0 = to_dev(inp["h0"][0], torch)
    w1, w2, x0 = to_dev(f["w1"], torch), to_dev(f["w2"], torch), to_dev(inp["x0"][0], torch)
    for _ in range(3):
        h.copy_(h0)
        pg.decode_frame_q8(W["qkv"], W["up"], W["down"], W["head"], w1, w2, f["eps"], x0, h, out, ws)
        torch.cuda.synchronize()
        for k in out:
            assert torch.equal(out[k], first[k]), k
        assert torch.equal(h, h_first)
    pg.decode_frame_q8_status(ws)
    assert pg.decode_frame_timeouts(ws) == 0
    fr = pg.Frame(W["qkv"], W["up"], W["down"], W["head"], w1, w2, f["eps"], n=1)
    h4 = h0.clone().view(1, -1)
    logits4 = fr.run(x0.view(1, -1), h4)
    torch.cuda.synchronize()
    import oracle
    assert oracle.rel_err(h.cpu().numpy(), h4.view(-1).cpu().numpy()) <= 1e-5
    assert oracle.rel_err(out["logits"].cpu().numpy(), logits4.view(-1).cpu().numpy()) <= 1e-4


def test_decode_frame_errors(pg):
    """Shape and workspace errors are reported before anything is launched."""
    _case("decode_frame_q8 errors")
    L = pg.lib()
    H = 1024
    dev = "cuda"

    keep = []

    def mat(rows, cols):
        t = (torch.zeros(rows * cols, dtype=torch.int8, device=dev), torch.zeros(rows * cols // 32, device=dev),
             torch.zeros(rows * cols // 32, device=dev))
        keep.append(t)
        return pg._lib.PgQ8(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), rows, cols)

    def vec(n):
        t = torch.zeros(n, device=dev)
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    ws = pg.decode_frame_q8_workspace(H, 2048)
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(qkv, up, down, head, ws_bytes=ws.numel()):
        return L.decode_frame_q8(ctypes.byref(qkv), ctypes.byref(up), ctypes.byref(down), ctypes.byref(head),
                                 vec(H), vec(H), 1e-6, vec(H), vec(H), vec(qkv.rows), vec(up.rows), vec(H),
                                 vec(head.rows), ctypes.c_void_p(ws.data_ptr()), ws_bytes, s)

    ok = (mat(1536, H), mat(2048, H), mat(H, 2048), mat(100, H))
    assert call(*ok) == pg.PG_OK
    torch.cuda.synchronize()
    assert call(*ok, ws_bytes=ws.numel() - 4) == pg.PG_EWORKSPACE
    assert call(mat(1536, H), mat(2048, H), mat(H, 1024), mat(100, H)) == pg.PG_EINVAL   # down.cols != up.rows
    assert call(mat(512, H), mat(2048, H), mat(H, 2048), mat(100, H)) == pg.PG_EINVAL    # qkv rows < hidden
    assert call(mat(1536, 1056), mat(2048, 1056), mat(1056, 2048), mat(100, 1056)) == pg.PG_EUNSUPPORTED
    # outputs overlapping inputs or each other
    big = torch.zeros(4 * 4096, device=dev)
    keep.append(big)
    p0 = ctypes.c_void_p(big.data_ptr())
    p1 = ctypes.c_void_p(big.data_ptr() + 4 * 1024)
    args = [ctypes.byref(m) for m in ok]
    assert L.decode_frame_q8(*args, vec(H), vec(H), 1e-6, p0, vec(H), p0, vec(2048), vec(H), vec(100),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), s) == pg.PG_EINVAL      # qkv == x0
    assert L.decode_frame_q8(*args, vec(H), vec(H), 1e-6, vec(H), vec(H), p0, p1, vec(H), vec(100),
                             ctypes.c_void_p(ws.data_ptr()), ws.numel(), s) == pg.PG_EINVAL      # u inside qkv
    assert L.decode_frame_q8_status(ctypes.c_void_p(ws.data_ptr()), ws.numel(), s) == pg.PG_OK
    assert L.decode_frame_q8_status(None, ws.numel(), s) == pg.PG_EWORKSPACE
    assert pg.decode_frame_timeouts(ws) == 0
