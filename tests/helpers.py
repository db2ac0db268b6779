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
