"""prefill_frame_q8: the q8 layer frame over one prefill pass in five launches
(x0 staging + four matrix-core passes whose epilogues carry the residual add,
the RMSNorm sums and the next product's staging), against the oracle's frame
chain (every intermediate rounded to its f32 buffer).  Shapes exercise K
splits (2 and 11 of them, so the in-pass reduction runs more than one batch of
splits), a last panel that ends inside a 16-row item, position counts that
leave one position tile partly empty, and the full frame at 64 positions."""
import numpy as np
import pytest

import synth
from helpers import TOL_Q8, assert_staged, oracle_frame_staged, q8_dev, staged_errors, to_dev

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
    # 2 K splits in QKV and up, head 1000 rows (the last panel ends 8 rows into an item)
    "h1024": synth.FrameShape(hidden=1024, qkv=1536, inter=2048, vocab=1000),
    # down: 176 blocks over 16 panels -> 11 splits
    "h2048": synth.FrameShape(hidden=2048, qkv=2048, inter=5632, vocab=3000),
    "full": synth.FrameShape(),
}


def _weights(f):
    return {k: q8_dev(f[k], torch) for k in ("qkv", "up", "down", "head")}


def _run(pg, W, f, x0, h0, ws=None):
    n, H = x0.shape
    out = {"qkv": torch.empty(n, W["qkv"].rows, device="cuda"), "u": torch.empty(n, W["up"].rows, device="cuda"),
           "d": torch.empty(n, H, device="cuda"), "logits": torch.empty(n, W["head"].rows, device="cuda")}
    if ws is None:
        ws = torch.empty(pg.prefill_frame_q8_workspace_bytes(H, W["qkv"].rows, W["up"].rows, W["head"].rows, n),
                         dtype=torch.uint8, device="cuda")
    h = to_dev(h0, torch)
    pg.prefill_frame_q8(W["qkv"], W["up"], W["down"], W["head"], to_dev(f["w1"], torch), to_dev(f["w2"], torch),
                        f["eps"], to_dev(x0, torch), h, out, ws)
    torch.cuda.synchronize()
    return out, h, ws


@pytest.mark.parametrize("name,n", [("h1024", 1), ("h1024", 5), ("h1024", 64), ("h2048", 33), ("full", 64)])
def test_prefill_frame_parity(pg, oracle, name, n):
    """Stage-isolated: every output of the one call is compared with the
    definition applied to the device's own input to that stage (its qkv, u, d
    and final residual), so the dense epilogues that only this call uses (the
    residual add with the next product's staging, and the 1/rms scaling) are
    each held to the q8 tolerance."""
    shape = SHAPES[name]
    _case(f"prefill_frame_q8 {name} n={n}")
    f = synth.frame_weights(21, shape)
    inp = synth.frame_inputs(21, n, shape.hidden)
    out, h, _ = _run(pg, _weights(f), f, inp["x0"], inp["h0"])
    dev = {k: v.cpu().numpy() for k, v in out.items()}
    dev["h2"] = h.cpu().numpy()
    ref = oracle_frame_staged(oracle, f, inp["x0"], inp["h0"], dev)
    errs = staged_errors(oracle, ref, dev)
    print(f"[info] {name} n={n} rel errs " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert_staged(errs)


def test_prefill_frame_repeat_and_vs_calls(pg):
    """Bit-identical on repeat (fixed orders for split partials and norm sums,
    tickets cleared by every call), and close to the frame built from
    prefill_gemm_q8 / prefill_gemm_q8_addnorm calls."""
    shape = SHAPES["h2048"]
    n = 48
    _case(f"prefill_frame_q8 repeat {shape} n={n}")
    f = synth.frame_weights(22, shape)
    inp = synth.frame_inputs(22, n, shape.hidden)
    W = _weights(f)
    out, h, ws = _run(pg, W, f, inp["x0"], inp["h0"])
    for _ in range(2):
        out2, h2, _ = _run(pg, W, f, inp["x0"], inp["h0"], ws)
        for k in out:
            assert torch.equal(out[k], out2[k]), k
        assert torch.equal(h, h2)
    H = shape.hidden
    w1, w2 = to_dev(f["w1"], torch), to_dev(f["w2"], torch)
    x0, hc = to_dev(inp["x0"], torch), to_dev(inp["h0"], torch)
    need = max(pg.prefill_gemm_q8_workspace_bytes(w.rows, w.cols, n) for w in W.values())
    wsc = torch.empty(need, dtype=torch.uint8, device="cuda")
    qkv = pg.prefill_gemm_q8(W["qkv"], x0, workspace=wsc)
    u = pg.prefill_gemm_q8_addnorm(W["up"], hc, qkv[:, :H], w1, f["eps"], act=1, H_out=hc, workspace=wsc)
    d = pg.prefill_gemm_q8(W["down"], u, workspace=wsc)
    logits = pg.prefill_gemm_q8_addnorm(W["head"], hc, d, w2, f["eps"], H_out=hc, workspace=wsc)
    torch.cuda.synchronize()
    import oracle
    # Both round their matrix-core inputs to bf16 hi + lo (about 2^-17), one
    # before the 1/rms scaling and one after, so they agree far inside the
    # oracle tolerance but not bit for bit.
    eh = oracle.rel_err(h.cpu().numpy(), hc.cpu().numpy())
    el = oracle.rel_err(out["logits"].cpu().numpy(), logits.cpu().numpy())
    print(f"[info] frame vs calls: h {eh:.2e} logits {el:.2e}", flush=True)
    assert eh <= TOL_Q8 / 10 and el <= TOL_Q8 / 10


def test_prefill_frame_errors(pg):
    """Argument errors are reported before anything is launched."""
    _case("prefill_frame_q8 errors")
    import ctypes
    L = pg.lib()
    keep = []

    def mat(rows, cols):
        t = (torch.zeros(rows * cols, dtype=torch.int8, device="cuda"), torch.zeros(rows * cols // 32, device="cuda"),
             torch.zeros(rows * cols // 32, device="cuda"))
        keep.append(t)
        return pg._lib.PgQ8(t[0].data_ptr(), t[1].data_ptr(), t[2].data_ptr(), rows, cols)

    def vec(nf):
        t = torch.zeros(nf, device="cuda")
        keep.append(t)
        return ctypes.c_void_p(t.data_ptr())

    H, n = 1024, 8
    ws = torch.empty(pg.prefill_frame_q8_workspace_bytes(H, 1536, 2048, 1000, n), dtype=torch.uint8, device="cuda")
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def call(qkv, up, down, head, nn=n, ws_bytes=ws.numel()):
        return L.prefill_frame_q8(ctypes.byref(qkv), ctypes.byref(up), ctypes.byref(down), ctypes.byref(head),
                                  vec(H), vec(H), 1e-6, vec(nn * H), vec(nn * H), nn, vec(nn * qkv.rows),
                                  vec(nn * up.rows), vec(nn * H), vec(nn * head.rows), ctypes.c_void_p(ws.data_ptr()),
                                  ws_bytes, s)

    ok = (mat(1536, H), mat(2048, H), mat(H, 2048), mat(1000, H))
    assert call(*ok) == pg.PG_OK
    torch.cuda.synchronize()
    assert call(*ok, ws_bytes=ws.numel() - 256) == pg.PG_EWORKSPACE
    assert call(*ok, nn=65) == pg.PG_EUNSUPPORTED
    assert call(*ok, nn=0) == pg.PG_EINVAL
    assert call(mat(1536, H), mat(2048, H), mat(H, 1024), mat(1000, H)) == pg.PG_EINVAL  # down.cols != up.rows
    assert call(mat(1536, H), mat(2048, H), mat(H, 2048), mat(1000, H + 32)) == pg.PG_EINVAL  # head.cols != H
    assert call(mat(1536, H), mat(2048, H), mat(H, 2048 + 16), mat(1000, H)) == pg.PG_EUNSUPPORTED
    # an output overlapping an input: refused before any launch
    X0 = vec(n * H)
    assert L.prefill_frame_q8(ctypes.byref(ok[0]), ctypes.byref(ok[1]), ctypes.byref(ok[2]), ctypes.byref(ok[3]),
                              vec(H), vec(H), 1e-6, X0, vec(n * H), n, X0, vec(n * 2048), vec(n * H),
                              vec(n * 1000), ctypes.c_void_p(ws.data_ptr()), ws.numel(), s) == pg.PG_EINVAL
