"""add_rmsnorm and moe_grouped parity against the CPU oracle, through the C ABI.

Routing is compared bit for bit (f32 logits in the shared fixed order, the
selected experts, the per-expert counts and lists); floating outputs within
tolerance.  The full 128-expert pass is checked on every routing output and on
the residual/norm outputs of every position."""
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


# ------------------------------------------------------------------ add + RMSNorm

@pytest.mark.parametrize("n,H,stride", [(1, 1024, None), (7, 4096, 6144), (64, 2688, None),
                                        (3, 16384, None), (2, 4, None), (5, 4096, 0)])
def test_add_rmsnorm(pg, oracle, n, H, stride):
    _case(f"add_rmsnorm n={n} H={H} stride={stride}")
    rng = np.random.default_rng(n * H)
    h = synth.normal(rng, (n, H))
    w = synth.norm_weight(rng, H)
    if stride == 0:                       # no residual input
        delta, dd = None, None
    else:
        wide = synth.normal(rng, (n, stride or H))
        delta, dd = wide, to_dev(wide, torch)
    hd = to_dev(h, torch)
    out = pg.add_rmsnorm(hd, None if dd is None else dd[:, :H], to_dev(w, torch), 1e-6,
                         delta_stride=None if stride in (None, 0) else stride)
    torch.cuda.synchronize()
    h_ref, out_ref = oracle.add_rmsnorm(h, delta, w, 1e-6, delta_stride=stride or None)
    assert oracle.rel_err(hd.cpu().numpy(), h_ref) <= TOL_F32
    assert oracle.rel_err(out.cpu().numpy(), out_ref) <= TOL_F32


def test_add_rmsnorm_unit_weight_invariant(pg):
    _case("add_rmsnorm invariant")
    rng = np.random.default_rng(3)
    h = to_dev(synth.normal(rng, (9, 4096)), torch)
    out = pg.add_rmsnorm(h, None, torch.ones(4096, device="cuda"), 1e-6)
    m = h.double().pow(2).mean(1)
    rms = out.double().pow(2).mean(1).sqrt()
    assert torch.allclose(rms, (m / (m + 1e-6)).sqrt(), rtol=1e-5)


# ------------------------------------------------------------------ routed MoE

def _run_moe(pg, c, renorm=0):
    up, down = q8_dev(c["up"], torch), q8_dev(c["down"], torch)
    h = to_dev(c["h"], torch)
    o = pg.moe_grouped(to_dev(c["X"], torch), to_dev(c["Wr"], torch), up, down, h,
                       to_dev(c["w"], torch), c["eps"], c["top_k"], renorm=renorm)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in o.items()}
    o["h"] = h.cpu().numpy()
    return o


def _check_routing(oracle, c, o, renorm=0):
    E = c["Wr"].shape[0]
    L = oracle.router_logits_f32(c["X"], c["Wr"])
    assert np.array_equal(o["logits"].view(np.uint32), L.view(np.uint32)), "logits bits"
    sel, rw, _ = oracle.route(L, c["top_k"], renorm)
    assert np.array_equal(o["sel"], sel), "selection"
    assert oracle.rel_err(o["route_w"], rw) <= TOL_F32
    counts, lists = oracle.group(sel, E)
    assert np.array_equal(o["counts"], counts), "counts"
    for e in range(E):
        assert np.array_equal(o["lists"][e, :counts[e]], lists[e, :counts[e]]), f"list {e}"
    return sel, rw


@pytest.mark.parametrize("shape", [synth.MoEShape(n=8, hidden=64, inter=96, experts=6, top_k=2),
                                   synth.MoEShape(n=40, hidden=256, inter=160, experts=16, top_k=4),
                                   synth.MoEShape(n=1, hidden=32, inter=32, experts=1, top_k=1),
                                   synth.MoEShape(n=64, hidden=128, inter=64, experts=3, top_k=3),
                                   # about 24 entries per expert over 4096 columns: two entry
                                   # groups per item, each staged in column chunks
                                   synth.MoEShape(n=48, hidden=4096, inter=160, experts=4, top_k=2)])
@pytest.mark.parametrize("renorm", [0, 1])
def test_moe_small(pg, oracle, shape, renorm):
    _case(f"moe {shape} renorm={renorm}")
    c = synth.moe(shape.n + shape.experts, shape)
    o = _run_moe(pg, c, renorm)
    sel, rw = _check_routing(oracle, c, o, renorm)
    up = (c["up"].q, c["up"].scale, c["up"].bias)
    down = (c["down"].q, c["down"].scale, c["down"].bias)
    _, D = oracle.moe_experts(c["X"], sel, up, down, grouped=True, E=shape.experts)
    h_ref, out_ref = oracle.moe_combine(c["h"], D, rw, c["w"], c["eps"])
    assert oracle.rel_err(o["h"], h_ref) <= TOL_Q8
    assert oracle.rel_err(o["out"], out_ref) <= TOL_Q8


def test_moe_router_ties(pg, oracle):
    """Duplicate router rows tie exactly; the lower expert index must win."""
    _case("moe ties")
    shape = synth.MoEShape(n=16, hidden=128, inter=64, experts=12, top_k=5)
    c = synth.moe(3, shape)
    c["Wr"][7] = c["Wr"][2]
    c["Wr"][10] = c["Wr"][2]
    c["Wr"][5] = c["Wr"][4]
    o = _run_moe(pg, c)
    sel, _ = _check_routing(oracle, c, o)
    L = o["logits"]
    assert np.array_equal(L[:, 2], L[:, 7]) and np.array_equal(L[:, 2], L[:, 10])
    for b in range(16):
        pos = {int(e): t for t, e in enumerate(sel[b])}
        if 7 in pos:
            assert 2 in pos and pos[2] < pos[7]


def _moe_entries(pg, c, o, ws):
    """U [n k][I] and D [n k][H]: the per-entry expert outputs moe_grouped leaves at the
    start of its workspace."""
    n, H = c["X"].shape
    I = c["up"].q.shape[-2]
    nk = n * c["top_k"]
    U = ws[:nk * I * 4].view(torch.float32).view(nk, I).cpu().numpy()
    d0 = -(-(nk * I * 4) // 256) * 256
    D = ws[d0:d0 + nk * H * 4].view(torch.float32).view(nk, H).cpu().numpy()
    return U, D


@pytest.mark.parametrize("exact", [False, True])
def test_moe_bank_edges(pg, oracle, exact):
    """Both expert banks with the format's edges planted (q = -128 rows, blocks and entries;
    scale-0 blocks holding their bias alone).  Routing exact; each entry's up row U against
    the oracle on X (bit for bit in the exact case: scale 2^-3, biases multiples of 1/8,
    activations in {-1, 0, 1}), its down row D against the oracle on the device's U, and the
    pass's outputs at the q8 tolerance."""
    _case(f"moe bank edges exact={exact}")
    shape = synth.MoEShape(n=24, hidden=128, inter=96, experts=6, top_k=2)
    c = synth.moe(5 + exact, shape)
    rng = np.random.default_rng(93 + exact)
    E, I, H = shape.experts, shape.inter, shape.hidden
    if exact:
        c["up"] = exact_q8(rng, I, H, lead=(E,))
        c["down"] = exact_q8(rng, H, I, lead=(E,))
        c["X"] = int_acts(rng, (shape.n, H), lim=1)
    plant_q8_edges(c["up"], rng, exact=exact)
    plant_q8_edges(c["down"], rng, exact=exact)
    ws = torch.empty(pg.moe_grouped_workspace_bytes(shape.n, H, I, E, shape.top_k), dtype=torch.uint8,
                     device="cuda")
    up, down = q8_dev(c["up"], torch), q8_dev(c["down"], torch)
    h = to_dev(c["h"], torch)
    o = pg.moe_grouped(to_dev(c["X"], torch), to_dev(c["Wr"], torch), up, down, h, to_dev(c["w"], torch),
                       c["eps"], c["top_k"], workspace=ws)
    torch.cuda.synchronize()
    o = {k: v.cpu().numpy() for k, v in o.items()}
    o["h"] = h.cpu().numpy()
    sel, rw = _check_routing(oracle, c, o)
    U, D = _moe_entries(pg, c, o, ws)
    t_up = (c["up"].q, c["up"].scale, c["up"].bias)
    t_dn = (c["down"].q, c["down"].scale, c["down"].bias)
    U_ref, _ = oracle.moe_experts(c["X"], sel, t_up, t_dn)
    if exact:
        assert np.max(U_ref) < 2.0 ** 18      # relu^2 of a multiple of 1/8 below 512: exact in f32
        assert np.array_equal(U.astype(np.float64), U_ref)
    else:
        assert oracle.rel_err(U, U_ref) <= TOL_Q8
    k = c["top_k"]
    D_ref = np.stack([oracle.gemm_q8(*(a[sel.reshape(-1)[j]] for a in t_dn), U[j]) for j in range(U.shape[0])])
    assert oracle.rel_err(D, D_ref) <= TOL_Q8
    h_ref, out_ref = oracle.moe_combine(c["h"], D_ref, rw, c["w"], c["eps"])
    assert oracle.rel_err(o["h"], h_ref) <= TOL_Q8
    assert oracle.rel_err(o["out"], out_ref) <= TOL_Q8
    assert k == sel.shape[1]


def test_moe_full_128_experts(pg, oracle):
    """The full pass: 64 positions, hidden 2688, 128 experts of 2688 -> 1856 -> 2688, top-6."""
    _case("moe full")
    c = synth.moe(0)
    o = _run_moe(pg, c)
    sel, rw = _check_routing(oracle, c, o)
    distinct = int((o["counts"] > 0).sum())
    print(f"[info] distinct experts selected: {distinct}", flush=True)
    up = (c["up"].q, c["up"].scale, c["up"].bias)
    down = (c["down"].q, c["down"].scale, c["down"].bias)
    _, D = oracle.moe_experts(c["X"], sel, up, down, grouped=False)
    h_ref, out_ref = oracle.moe_combine(c["h"], D, rw, c["w"], c["eps"])
    assert oracle.rel_err(o["h"], h_ref) <= TOL_Q8
    assert oracle.rel_err(o["out"], out_ref) <= TOL_Q8
