"""Decode GEMV parity (gemv_q8, gemv_f16, and the q8 GEMV + add + RMSNorm pair)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import synth
from helpers import TOL_F16, TOL_F32, TOL_Q8, exact_q8, int_acts, q8_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


def test_gemv_q8_add_norm_1024(pg, oracle):
    """The 1024x1024 q8 GEMV whose output is added into the residual and RMS-normed."""
    _case("gemv_q8 1024x1024 + add_rmsnorm")
    c = synth.gemv_add_norm(0)
    W = q8_dev(c["W"], torch)
    x, w = to_dev(c["x"], torch), to_dev(c["w"], torch)
    y_ref = oracle.gemm_q8(c["W"].q, c["W"].scale, c["W"].bias, c["x"])
    d_ref = y_ref.astype(np.float32)              # the product as the f32 buffer it lives in
    h_ref, out_ref = oracle.add_rmsnorm(c["h"], d_ref, c["w"], c["eps"])
    # stage 1: the product
    y = pg.gemv_q8(W, x)
    assert oracle.rel_err(y.cpu().numpy(), y_ref) <= TOL_Q8
    # stage 2 in isolation: the device norm fed the oracle's product
    h = to_dev(c["h"], torch).view(1, -1)
    out = pg.add_rmsnorm(h, to_dev(d_ref, torch).view(1, -1), w, c["eps"])
    assert oracle.rel_err(h.cpu().numpy(), h_ref) <= TOL_F32
    assert oracle.rel_err(out.cpu().numpy(), out_ref) <= TOL_F32
    # end to end on the device
    h = to_dev(c["h"], torch).view(1, -1)
    out = pg.add_rmsnorm(h, y.view(1, -1), w, c["eps"])
    assert oracle.rel_err(h.cpu().numpy(), h_ref) <= TOL_Q8
    assert oracle.rel_err(out.cpu().numpy(), out_ref) <= TOL_Q8


@pytest.mark.parametrize("rows,cols", [(1, 32), (37, 96), (8, 1024), (133, 2688), (70, 1856),
                                       (24, 14336), (9, 32768)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q8_shapes(pg, oracle, rows, cols, act):
    _case(f"gemv_q8 {rows}x{cols} act={act}")
    rng = np.random.default_rng(rows * 7 + cols)
    m = synth.q8(rng, rows, cols)
    x = synth.normal(rng, cols)
    y = pg.gemv_q8(q8_dev(m, torch), to_dev(x, torch), act=act)
    torch.cuda.synchronize()
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
    assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL_Q8


def test_gemv_q8_exact_bitwise(pg, oracle):
    """Scale 2^-3, bias 0, integer activations: every partial sum is exact in f32,
    so the device result equals the oracle's exactly, whatever the order."""
    _case("gemv_q8 exact")
    rng = np.random.default_rng(5)
    m = exact_q8(rng, 301, 4096)
    x = int_acts(rng, 4096)
    y = pg.gemv_q8(q8_dev(m, torch), to_dev(x, torch))
    torch.cuda.synchronize()
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, x)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


def test_gemv_q8_frame_matrices_sampled(pg, oracle):
    """Full-size decode frame matrices (hidden 4096): sampled rows against the oracle."""
    f = synth.frame_weights(0)
    rng = np.random.default_rng(11)
    for name in ("qkv", "up", "down", "head"):
        _case(f"gemv_q8 frame {name}")
        m = f[name]
        x = synth.normal(rng, m.cols)
        y = pg.gemv_q8(q8_dev(m, torch), to_dev(x, torch)).cpu().numpy()
        idx = np.unique(np.concatenate([rng.choice(m.rows, 192, replace=False), [0, m.rows - 1]]))
        ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, x)[0]
        assert oracle.rel_err(y[idx], ref) <= TOL_Q8, name


def test_gemv_f16_4096(pg, oracle):
    _case("gemv_f16 4096x4096")
    c = synth.f16_gemv(0)
    Wd = to_dev(c["W"], torch)
    x = to_dev(c["x"], torch)
    y = pg.gemv_f16(Wd, x)
    torch.cuda.synchronize()
    ref = oracle.gemm_f16(c["W"], c["x"])
    assert oracle.rel_err(y.cpu().numpy(), ref) <= TOL_F16
    for _ in range(3):          # repeated launches give the same bits
        assert torch.equal(pg.gemv_f16(Wd, x), y)


@pytest.mark.parametrize("rows,cols", [(1, 8), (13, 24), (100, 1000), (65, 4104)])
def test_gemv_f16_shapes(pg, oracle, rows, cols):
    _case(f"gemv_f16 {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    W = synth.f16(rng, rows, cols)
    x = synth.normal(rng, cols)
    y = pg.gemv_f16(to_dev(W, torch), to_dev(x, torch), act=1)
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), oracle.gemm_f16(W, x, act=1)) <= TOL_F16


def test_gemv_f16_exact_bitwise(pg, oracle):
    _case("gemv_f16 exact")
    rng = np.random.default_rng(6)
    W = (rng.integers(-64, 65, size=(77, 2048)) / 16).astype(np.float16)
    x = int_acts(rng, 2048)
    y = pg.gemv_f16(to_dev(W, torch), to_dev(x, torch))
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().numpy().astype(np.float64), oracle.gemm_f16(W, x))


def test_gemv_errors_on_device(pg):
    _case("gemv errors")
    W = pg.Q8Weight(torch.zeros(4, 48, dtype=torch.int8, device="cuda"),
                    torch.zeros(4, 1, device="cuda"), torch.zeros(4, 1, device="cuda"))
    with pytest.raises(pg.PGError) as e:
        pg.gemv_q8(W, torch.zeros(48, device="cuda"))
    assert e.value.code == pg.PG_EUNSUPPORTED
