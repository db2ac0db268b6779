"""Decode GEMV parity (gemv_q8, gemv_f16, and the q8 GEMV + add + RMSNorm pair)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import synth
from helpers import TOL_F16, TOL_F32, TOL_Q8, exact_q8, int_acts, plant_q8_edges, q8_dev, to_dev

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


@pytest.mark.parametrize("rows,cols", [(301, 4096), (64, 14336)])
def test_gemv_q8_exact_edges_bitwise(pg, oracle, rows, cols):
    """The exact case with the format's edges planted: q = -128 rows, blocks and entries,
    and scale-0 blocks (bias alone, multiples of 1/8) -- still bit for bit."""
    _case(f"gemv_q8 exact edges {rows}x{cols}")
    rng = np.random.default_rng(rows + cols)
    m = plant_q8_edges(exact_q8(rng, rows, cols), rng, exact=True)
    x = int_acts(rng, cols, lim=4)
    for act in (0, 1):
        y = pg.gemv_q8(q8_dev(m, torch), to_dev(x, torch), act=act)
        torch.cuda.synchronize()
        ref = oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
        if act == 0:
            assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)
        else:   # relu^2 rounds the square once in f32
            assert np.array_equal(y.cpu().numpy(), ref.astype(np.float32))


def test_gemv_q8_edges_tolerance(pg, oracle):
    """Random scales and biases with the edges planted: within the q8 tolerance."""
    _case("gemv_q8 edges")
    rng = np.random.default_rng(91)
    m = plant_q8_edges(synth.q8(rng, 700, 2048), rng)
    x = synth.normal(rng, 2048)
    y = pg.gemv_q8(q8_dev(m, torch), to_dev(x, torch))
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), oracle.gemm_q8(m.q, m.scale, m.bias, x)) <= TOL_Q8


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


# ------------------------------------------------------------------ add + RMSNorm fused into the GEMV

@pytest.mark.parametrize("rows,cols,delta,outs", [(1024, 1024, True, True), (37, 96, False, True),
                                                  (133, 2688, True, False), (6, 32768, True, True),
                                                  (14336, 4096, True, True), (1, 32, True, True)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q8_addnorm(pg, oracle, rows, cols, delta, outs, act):
    """y = act(W (rmsnorm(h + delta) w)) in one launch, against the oracle's norm then product."""
    _case(f"gemv_q8_addnorm {rows}x{cols} delta={delta} outs={outs} act={act}")
    rng = np.random.default_rng(rows * 13 + cols + act)
    m = synth.q8(rng, rows, cols)
    h = synth.normal(rng, cols)
    d = synth.normal(rng, cols) if delta else None
    w = synth.norm_weight(rng, cols)
    h_ref, x_ref = oracle.add_rmsnorm(h, d, w, 1e-6)
    y_ref = oracle.gemm_q8(m.q, m.scale, m.bias, x_ref, act=act)
    hd = to_dev(h, torch)
    ho = torch.full((cols,), float("nan"), device="cuda") if outs else None
    xo = torch.full((cols,), float("nan"), device="cuda") if outs else None
    y = pg.gemv_q8_addnorm(q8_dev(m, torch), hd, None if d is None else to_dev(d, torch), to_dev(w, torch),
                           1e-6, act=act, h_out=ho, x_out=xo)
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), y_ref) <= TOL_Q8
    assert np.array_equal(hd.cpu().numpy(), h)            # the input residual is left alone
    if outs:
        assert oracle.rel_err(ho.cpu().numpy(), h_ref) <= TOL_F32
        assert oracle.rel_err(xo.cpu().numpy(), x_ref) <= TOL_F32


def test_gemv_q8_addnorm_matches_two_calls(pg):
    """The fused call and add_rmsnorm followed by gemv_q8 agree (same inputs, f32 both ways)."""
    _case("gemv_q8_addnorm vs add_rmsnorm + gemv_q8")
    rng = np.random.default_rng(5)
    m = synth.q8(rng, 6144, 4096)
    W = q8_dev(m, torch)
    h = to_dev(synth.normal(rng, 4096), torch)
    d = to_dev(synth.normal(rng, 4096), torch)
    w = to_dev(synth.norm_weight(rng, 4096), torch)
    y = pg.gemv_q8_addnorm(W, h, d, w, 1e-6, act=1)
    h2 = h.clone().view(1, -1)
    x = pg.add_rmsnorm(h2, d.view(1, -1), w, 1e-6)
    y2 = pg.gemv_q8(W, x.view(-1), act=1)
    assert float((y - y2).abs().max() / y2.pow(2).mean().sqrt()) <= 1e-5


def test_gemv_q8_addnorm_exact(pg, oracle):
    """Exact case: integer residual with sum of squares = cols (rms 1), unit weights,
    eps 0, scale 2^-3, bias 0, so every step is exact and the result is bit for bit."""
    _case("gemv_q8_addnorm exact")
    rng = np.random.default_rng(21)
    rows, cols = 300, 2048
    m = exact_q8(rng, rows, cols)
    h = rng.choice(np.array([-1.0, 1.0], np.float32), size=cols)
    y = pg.gemv_q8_addnorm(q8_dev(m, torch), to_dev(h, torch), None, torch.ones(cols, device="cuda"), 0.0)
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, h)
    assert np.array_equal(y.cpu().numpy().astype(np.float64), ref)


# ------------------------------------------------------------------ add + RMSNorm split across two GEMVs

def _parts(hp, nparts):
    """Sums of squares over the consecutive, equal row ranges of gemv_q8_residual's partition, in f64."""
    hp = np.asarray(hp, np.float64)
    g = -(-hp.size // nparts)
    pad = np.zeros(nparts * g)
    pad[:hp.size] = hp
    return (pad.reshape(nparts, g) ** 2).sum(1)


@pytest.mark.parametrize("rows,cols,hidden,inplace", [(6144, 4096, 4096, True), (4096, 14336, 4096, False),
                                                      (100, 96, 37, True), (1024, 1024, 1024, False),
                                                      (8, 32768, 3, True)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q8_residual(pg, oracle, rows, cols, hidden, inplace, act):
    _case(f"gemv_q8_residual {rows}x{cols} hidden={hidden} inplace={inplace} act={act}")
    rng = np.random.default_rng(rows + cols + hidden + act)
    m = synth.q8(rng, rows, cols)
    x = synth.normal(rng, cols)
    h = synth.normal(rng, hidden)
    w = synth.norm_weight(rng, hidden)
    y_ref = oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
    h_ref, _ = oracle.add_rmsnorm(h, y_ref[:hidden].astype(np.float32), w, 1e-6)
    hd = to_dev(h, torch)
    ho = hd if inplace else torch.full((hidden,), float("nan"), device="cuda")
    xw = torch.full((hidden,), float("nan"), device="cuda")
    parts = torch.full((pg.norm_parts(hidden),), float("nan"), device="cuda")
    y = pg.gemv_q8_residual(q8_dev(m, torch), to_dev(x, torch), hd, to_dev(w, torch), xw, parts, act=act,
                            h_out=ho)
    torch.cuda.synchronize()
    assert oracle.rel_err(y.cpu().numpy(), y_ref) <= TOL_Q8
    assert oracle.rel_err(ho.cpu().numpy(), h_ref) <= TOL_Q8
    assert oracle.rel_err(xw.cpu().numpy(), w.astype(np.float64) * h_ref) <= TOL_Q8
    assert oracle.rel_err(parts.cpu().numpy(), _parts(h_ref, pg.norm_parts(hidden))) <= TOL_Q8
    assert abs(float(parts.double().sum()) / float((h_ref ** 2).sum()) - 1) <= TOL_Q8
    if not inplace:
        assert np.array_equal(hd.cpu().numpy(), h)


@pytest.mark.parametrize("rows,cols", [(14336, 4096), (32000, 4096), (77, 1056)])
@pytest.mark.parametrize("act", [0, 1])
def test_gemv_q8_normed(pg, oracle, rows, cols, act):
    """Stage-isolated: fed w * h' and the parts of the oracle's h', the product equals the
    oracle's product on rmsnorm(h') * w."""
    _case(f"gemv_q8_normed {rows}x{cols} act={act}")
    rng = np.random.default_rng(rows * 3 + cols + act)
    m = synth.q8(rng, rows, cols)
    h = synth.normal(rng, cols)
    d = synth.normal(rng, cols)
    w = synth.norm_weight(rng, cols)
    h_ref, x_ref = oracle.add_rmsnorm(h, d, w, 1e-6)
    xw = (w.astype(np.float64) * h_ref).astype(np.float32)
    parts = _parts(h_ref, pg.norm_parts(cols)).astype(np.float32)
    y = pg.gemv_q8_normed(q8_dev(m, torch), to_dev(xw, torch), to_dev(parts, torch), 1e-6, act=act)
    torch.cuda.synchronize()
    idx = np.unique(rng.choice(rows, min(rows, 500), replace=False))
    ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, x_ref, act=act)[0]
    assert oracle.rel_err(y.cpu().numpy()[idx], ref) <= TOL_Q8


def test_gemv_q8_residual_then_normed(pg, oracle):
    """The pair end to end: W2 . (rmsnorm(h + W1 x) w) against the oracle chain."""
    _case("gemv_q8_residual -> gemv_q8_normed")
    rng = np.random.default_rng(44)
    m1, m2 = synth.q8(rng, 1536, 1024), synth.q8(rng, 2000, 1024)
    x, h, w = synth.normal(rng, 1024), synth.normal(rng, 1024), synth.norm_weight(rng, 1024)
    y1 = oracle.gemm_q8(m1.q, m1.scale, m1.bias, x).astype(np.float32)
    h_ref, x_ref = oracle.add_rmsnorm(h, y1[:1024], w, 1e-6)
    y2_ref = oracle.gemm_q8(m2.q, m2.scale, m2.bias, x_ref, act=1)
    hd = to_dev(h, torch)
    xw = torch.empty(1024, device="cuda")
    parts = torch.empty(pg.norm_parts(1024), device="cuda")
    pg.gemv_q8_residual(q8_dev(m1, torch), to_dev(x, torch), hd, to_dev(w, torch), xw, parts, h_out=hd)
    y2 = pg.gemv_q8_normed(q8_dev(m2, torch), xw, parts, 1e-6, act=1)
    torch.cuda.synchronize()
    assert oracle.rel_err(hd.cpu().numpy(), h_ref) <= TOL_Q8
    assert oracle.rel_err(y2.cpu().numpy(), y2_ref) <= 2 * TOL_Q8
