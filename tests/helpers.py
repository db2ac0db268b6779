"""Shared helpers of the parity tests: tolerances, device transfers, sampling."""
import numpy as np

import synth

# Output tolerance (max relative error floored at the output's RMS, see oracle.rel_err):
TOL_Q8 = 1e-3    # int8 block weights, f32 accumulation
TOL_F16 = 2e-3   # binary16 weights, f32 accumulation
TOL_F32 = 1e-5   # f32 elementwise stages (add + RMSNorm, softmax weights)


def to_dev(a, torch):
    return torch.as_tensor(np.ascontiguousarray(a)).to("cuda")


def q8_dev(m: synth.Q8, torch):
    from prefill_gemm_amd import Q8Weight
    return Q8Weight(to_dev(m.q, torch), to_dev(m.scale, torch), to_dev(m.bias, torch))


def exact_q8(rng, rows, cols, lead=()):
    """A q8 matrix whose products are exact in f32: scale 2^-3, bias 0."""
    q = rng.integers(-127, 128, size=lead + (rows, cols), dtype=np.int8)
    scale = np.full(lead + (rows, cols // 32), 0.125, np.float32)
    bias = np.zeros(lead + (rows, cols // 32), np.float32)
    return synth.Q8(q, scale, bias)


def int_acts(rng, shape, lim=8):
    return rng.integers(-lim, lim + 1, size=shape).astype(np.float32)


def oracle_frame(oracle, f, x0, h0):
    """The frame chain on the oracle, every intermediate rounded to the f32 buffer it lives in."""
    H = f["qkv"].cols
    g = lambda m, x, act=0: oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
    s = {}
    s["qkv"] = g(f["qkv"], x0).astype(np.float32)
    s["h1"], x1 = oracle.add_rmsnorm(h0, s["qkv"], f["w1"], f["eps"], delta_stride=s["qkv"].shape[1])
    s["x1"] = x1.astype(np.float32)
    s["u"] = g(f["up"], s["x1"], act=1).astype(np.float32)
    s["d"] = g(f["down"], s["u"]).astype(np.float32)
    s["h2"], x2 = oracle.add_rmsnorm(s["h1"].astype(np.float32), s["d"], f["w2"], f["eps"])
    s["x2"] = x2.astype(np.float32)
    s["logits"] = g(f["head"], s["x2"])
    return s


def oracle_frame_staged(oracle, f, x0, h0, dev):
    """Every stage of the frame on the oracle, fed the device's own input to that stage.

    ``dev`` holds the device's outputs as numpy arrays: ``qkv`` [n][R_qkv], ``u``
    [n][I], ``d`` [n][H] and ``h2`` [n][H] (the residual after the frame).  Each
    product is then compared with the definition applied to exactly what the
    device fed it, so it is held to its own tolerance with no error carried in
    from earlier stages:

        qkv    = W_qkv x0
        h1     = h0 + qkv_dev[:, :H]                 (one f32 add, as the device)
        u      = relu^2(W_up rmsnorm(h1) w1)
        d      = W_down u_dev
        h2     = h1 + d_dev                          (one f32 add)
        logits = W_head rmsnorm(h2_dev) w2
    """
    H = f["qkv"].cols
    g = lambda m, x, act=0: oracle.gemm_q8(m.q, m.scale, m.bias, x, act=act)
    n = np.atleast_2d(x0).shape[0]
    qkv_dev = np.asarray(dev["qkv"], np.float32).reshape(n, -1)
    u_dev = np.asarray(dev["u"], np.float32).reshape(n, -1)
    d_dev = np.asarray(dev["d"], np.float32).reshape(n, -1)
    h2_dev = np.asarray(dev["h2"], np.float32).reshape(n, -1)
    h0 = np.asarray(h0, np.float32).reshape(n, -1)
    r = {"qkv": g(f["qkv"], np.atleast_2d(x0))}
    r["h1"] = (h0 + qkv_dev[:, :H]).astype(np.float32)
    _, x1 = oracle.add_rmsnorm(r["h1"], None, f["w1"], f["eps"])
    r["u"] = g(f["up"], x1, act=1)
    r["d"] = g(f["down"], u_dev)
    r["h2"] = (r["h1"] + d_dev).astype(np.float32)
    _, x2 = oracle.add_rmsnorm(h2_dev, None, f["w2"], f["eps"])
    r["logits"] = g(f["head"], x2)
    return r


def staged_errors(oracle, ref, dev):
    """rel_err of each frame output against ``oracle_frame_staged``'s reference."""
    return {k: oracle.rel_err(np.asarray(dev[k]).reshape(ref[k].shape), ref[k])
            for k in ("qkv", "u", "d", "h2", "logits")}


def assert_staged(errs):
    """Products at the q8 tolerance; the residual (two f32 adds) at the f32 stage tolerance."""
    for k in ("qkv", "u", "d", "logits"):
        assert errs[k] <= TOL_Q8, (k, errs[k])
    assert errs["h2"] <= TOL_F32, ("h2", errs["h2"])


def plant_q8_edges(m: synth.Q8, rng, exact: bool = False) -> synth.Q8:
    """Plant the block format's edge cases into a q8 matrix (or stack), in place:
    q = -128 (outside the generator's [-127, 127], decoded as -128) on a whole row,
    on whole blocks and on scattered entries; scale 0 (the block is its bias
    alone) on scattered blocks and on a whole row.  With ``exact`` the planted
    biases are multiples of 1/8 in [-2, 2], so with scale 2^-3 and integer
    activations every f32 (and bf16 hi + lo) step stays exact."""
    q, scale, bias = m.q, m.scale, m.bias
    rows, nb = scale.shape[-2], scale.shape[-1]
    q[..., 0, :] = -128
    for _ in range(max(1, rows // 8)):
        r, b = int(rng.integers(rows)), int(rng.integers(nb))
        q[..., r, 32 * b:32 * b + 32] = -128
    mask = rng.random(q.shape) < 0.02
    q[mask] = -128
    zero = rng.random(scale.shape) < 0.05
    zero[..., rows // 2, :] = True
    scale[zero] = 0.0
    if exact:
        bias[zero] = (rng.integers(-16, 17, size=int(zero.sum())) / 8).astype(np.float32)
    return m
