"""Batched prefill product parity (prefill_gemm_q8) against the CPU oracle,
through the C ABI: ragged tiles, both tile heights, split and unsplit K, the
exact-integer case bit for bit, agreement with the decode GEMV, and the
full-size frame matrices on sampled rows."""
import numpy as np
import pytest

import synth
from helpers import TOL_F32, TOL_Q8, exact_q8, int_acts, plant_q8_edges, q8_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def pg():
    import prefill_gemm_amd as pg
    assert torch.cuda.is_available()
    return pg


def _case(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("n", [1, 5, 32, 33, 36, 64])
@pytest.mark.parametrize("rows,cols", [(300, 544), (128, 32), (45, 4096), (257, 1856)])
def test_prefill_small(pg, oracle, n, rows, cols):
    _case(f"prefill {rows}x{cols} n={n} splits={pg.lib().prefill_gemm_q8_workspace_bytes(rows, cols, n)}")
    rng = np.random.default_rng(n * 1000 + rows + cols)
    m = synth.q8(rng, rows, cols)
    X = synth.normal(rng, (n, cols))
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch))
    torch.cuda.synchronize()
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, X)
    assert oracle.rel_err(Y.cpu().numpy(), ref) <= TOL_Q8


@pytest.mark.parametrize("rows,cols,n", [(25600, 64, 64), (300, 4096, 40), (1000, 2688, 17)])
def test_prefill_relu2(pg, oracle, rows, cols, n):
    """relu^2 in the epilogue, on an unsplit (>= 200 panels) and a split pass."""
    _case(f"prefill relu2 {rows}x{cols} n={n}")
    rng = np.random.default_rng(rows + n)
    m = synth.q8(rng, rows, cols)
    X = synth.normal(rng, (n, cols))
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch), act=1)
    torch.cuda.synchronize()
    idx = np.unique(rng.choice(rows, min(rows, 400), replace=False))
    ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, X, act=1)
    assert oracle.rel_err(Y.cpu().numpy()[:, idx], ref) <= TOL_Q8


@pytest.mark.parametrize("rows,cols,n", [(300, 4096, 64), (25600, 64, 36), (130, 1024, 7)])
def test_prefill_exact_bitwise(pg, oracle, rows, cols, n):
    """Scale 2^-3, bias 0, integer activations: exact in f32, so bit for bit."""
    _case(f"prefill exact {rows}x{cols} n={n}")
    rng = np.random.default_rng(rows * n)
    m = exact_q8(rng, rows, cols)
    X = int_acts(rng, (n, cols))
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch))
    torch.cuda.synchronize()
    idx = np.unique(rng.choice(rows, min(rows, 300), replace=False))
    ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, X)
    assert np.array_equal(Y.cpu().numpy()[:, idx].astype(np.float64), ref)


def test_prefill_exact_bias_bitwise(pg, oracle):
    """Bias values exact in bf16 and integer activations: the bias contraction is exact too."""
    _case("prefill exact with bias")
    rng = np.random.default_rng(77)
    rows, cols, n = 200, 1024, 24
    m = exact_q8(rng, rows, cols)
    m.bias[:] = (rng.integers(-64, 65, size=m.bias.shape) / 64).astype(np.float32)
    X = int_acts(rng, (n, cols), lim=4)
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch))
    torch.cuda.synchronize()
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, X)
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)


@pytest.mark.parametrize("rows,cols,n", [(200, 1024, 24), (640, 4096, 64), (300, 14336, 7)])
def test_prefill_exact_edges_bitwise(pg, oracle, rows, cols, n):
    """The exact case with the format's edges planted (q = -128 rows, blocks and entries;
    scale-0 blocks holding their bias alone), K splits included: bit for bit."""
    _case(f"prefill exact edges {rows}x{cols} n={n}")
    rng = np.random.default_rng(rows + cols + n)
    m = plant_q8_edges(exact_q8(rng, rows, cols), rng, exact=True)
    X = int_acts(rng, (n, cols), lim=4)
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch))
    torch.cuda.synchronize()
    ref = oracle.gemm_q8(m.q, m.scale, m.bias, X)
    assert np.array_equal(Y.cpu().numpy().astype(np.float64), ref)


def test_prefill_edges_tolerance(pg, oracle):
    """Random scales and biases with the edges planted: within the q8 tolerance."""
    _case("prefill edges")
    rng = np.random.default_rng(92)
    m = plant_q8_edges(synth.q8(rng, 500, 4096), rng)
    X = synth.normal(rng, (64, 4096))
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch), act=1)
    torch.cuda.synchronize()
    assert oracle.rel_err(Y.cpu().numpy(), oracle.gemm_q8(m.q, m.scale, m.bias, X, act=1)) <= TOL_Q8


def test_prefill_rows_match_gemv(pg):
    """A pass over n positions and n single-position GEMVs are one computation:
    equal bit for bit in the exact case, within tolerance otherwise."""
    _case("prefill vs gemv")
    rng = np.random.default_rng(9)
    m = exact_q8(rng, 640, 2048)
    X = int_acts(rng, (12, 2048))
    W = q8_dev(m, torch)
    Xd = to_dev(X, torch)
    Y = pg.prefill_gemm_q8(W, Xd)
    for b in range(12):
        assert torch.equal(Y[b], pg.gemv_q8(W, Xd[b].contiguous()))
    m2 = synth.q8(rng, 640, 2048)
    W2 = q8_dev(m2, torch)
    X2 = to_dev(synth.normal(rng, (12, 2048)), torch)
    Y2 = pg.prefill_gemm_q8(W2, X2)
    for b in range(12):
        g = pg.gemv_q8(W2, X2[b].contiguous())
        assert float((Y2[b] - g).abs().max() / g.pow(2).mean().sqrt()) <= 2 * TOL_Q8


def test_prefill_frame_matrices_sampled(pg, oracle):
    """Full-size frame matrices (hidden 4096) at n = 64 and at the partial pass n = 36."""
    f = synth.frame_weights(0)
    rng = np.random.default_rng(12)
    for n in (64, 36):
        for name in ("qkv", "up", "down", "head"):
            _case(f"prefill frame {name} n={n}")
            m = f[name]
            X = synth.normal(rng, (n, m.cols))
            Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch)).cpu().numpy()
            idx = np.unique(np.concatenate([rng.choice(m.rows, 96, replace=False), [0, m.rows - 1]]))
            ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, X)
            assert oracle.rel_err(Y[:, idx], ref) <= TOL_Q8, (name, n)


def test_prefill_heavy_tailed_input(pg, oracle):
    """Inputs like a relu^2 output (large, heavy tailed) keep the tolerance."""
    _case("prefill heavy tail")
    rng = np.random.default_rng(13)
    m = synth.q8(rng, 256, 14336)
    X = (np.maximum(synth.normal(rng, (64, 14336)) * 25, 0) ** 2).astype(np.float32)
    Y = pg.prefill_gemm_q8(q8_dev(m, torch), to_dev(X, torch)).cpu().numpy()
    assert oracle.rel_err(Y, oracle.gemm_q8(m.q, m.scale, m.bias, X)) <= TOL_Q8


# ------------------------------------------------------------------ add + RMSNorm fused into the staging

@pytest.mark.parametrize("n,rows,cols,stride", [(1, 300, 544, None), (5, 45, 4096, 6144), (33, 257, 1856, 0),
                                                (64, 640, 2688, None), (36, 128, 16384, None),
                                                (64, 14336, 4096, 6144)])
@pytest.mark.parametrize("act", [0, 1])
def test_prefill_addnorm(pg, oracle, n, rows, cols, stride, act):
    """Y = act((rmsnorm(H + delta) w) W^T), the norm done while staging, against the oracle."""
    _case(f"prefill_addnorm {rows}x{cols} n={n} stride={stride} act={act}")
    rng = np.random.default_rng(n * 31 + rows + cols + act)
    m = synth.q8(rng, rows, cols)
    H = synth.normal(rng, (n, cols))
    w = synth.norm_weight(rng, cols)
    if stride == 0:
        d = dd = None
    else:
        wide = synth.normal(rng, (n, stride or cols))
        d, dd = wide, to_dev(wide, torch)[:, :cols]
    h_ref, x_ref = oracle.add_rmsnorm(H, d, w, 1e-6, delta_stride=stride or None)
    idx = np.unique(rng.choice(rows, min(rows, 300), replace=False))
    y_ref = oracle.gemm_q8_rows(m.q, m.scale, m.bias, idx, x_ref, act=act)
    Hd = to_dev(H, torch)
    Xo = torch.full((n, cols), float("nan"), device="cuda")
    Y = pg.prefill_gemm_q8_addnorm(q8_dev(m, torch), Hd, dd, to_dev(w, torch), 1e-6, act=act, H_out=Hd,
                                   X_out=Xo)
    torch.cuda.synchronize()
    assert oracle.rel_err(Y.cpu().numpy()[:, idx], y_ref) <= TOL_Q8
    assert oracle.rel_err(Hd.cpu().numpy(), h_ref) <= TOL_F32     # residual updated in place
    assert oracle.rel_err(Xo.cpu().numpy(), x_ref) <= TOL_F32


def test_prefill_addnorm_matches_gemv_addnorm(pg):
    """Each position of a fused prefill pass equals the fused decode call on that position."""
    _case("prefill_addnorm vs gemv_q8_addnorm")
    rng = np.random.default_rng(8)
    m = synth.q8(rng, 500, 1024)
    W = q8_dev(m, torch)
    H = to_dev(synth.normal(rng, (9, 1024)), torch)
    D = to_dev(synth.normal(rng, (9, 1024)), torch)
    w = to_dev(synth.norm_weight(rng, 1024), torch)
    Y = pg.prefill_gemm_q8_addnorm(W, H, D, w, 1e-6)
    for b in range(9):
        g = pg.gemv_q8_addnorm(W, H[b].contiguous(), D[b].contiguous(), w, 1e-6)
        assert float((Y[b] - g).abs().max() / g.pow(2).mean().sqrt()) <= 2 * TOL_Q8
