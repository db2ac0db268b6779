"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the CPU oracle.

This module only draws numbers: it holds none of the products, norms or
routing arithmetic.  Every tensor is drawn on the host with numpy's PCG64
generators spawned from one ``SeedSequence``, in a fixed order per workload,
so the GPU and the oracle see the same bytes.

Distributions (the workloads' statement of their inputs):
  * packed int8 weights: q uniform on the integers [-127, 127], in blocks of
    32 consecutive columns of a row; each block has an f32 scale ~ U(1e-3, 1e-2)
    and an f32 bias ~ N(0, 1e-3);
  * f16 weights: N(0, 0.02) rounded to binary16 (the f16 bits are the input);
  * activations and residuals: N(0, 1) f32;
  * RMSNorm weights: U(0.5, 1.5) f32, eps = 1e-6;
  * router weights: N(0, 0.02) f32.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

BLOCK = 32
EPS = 1e-6


def streams(seed: int, count: int) -> list[np.random.Generator]:
    """``count`` independent generators spawned from ``SeedSequence(seed)``."""
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(count)]


@dataclass
class Q8:
    """A packed int8 matrix: q [rows][cols] int8, scale/bias [rows][cols/32] f32."""

    q: np.ndarray
    scale: np.ndarray
    bias: np.ndarray

    @property
    def rows(self) -> int:
        return self.q.shape[-2]

    @property
    def cols(self) -> int:
        return self.q.shape[-1]

    def nbytes(self) -> int:
        return self.q.nbytes + self.scale.nbytes + self.bias.nbytes


def q8(rng: np.random.Generator, rows: int, cols: int, lead: tuple = ()) -> Q8:
    """Draw a q8 matrix (or a stack of them with leading shape ``lead``)."""
    assert cols % BLOCK == 0
    q = rng.integers(-127, 128, size=lead + (rows, cols), dtype=np.int8)
    scale = rng.uniform(1e-3, 1e-2, size=lead + (rows, cols // BLOCK)).astype(np.float32)
    bias = rng.normal(0.0, 1e-3, size=lead + (rows, cols // BLOCK)).astype(np.float32)
    return Q8(q, scale, bias)


class Q82:
    """A q8_2f matrix: int8 body [rows][cols], binary16 row scales [rows] and column field [cols]."""

    def __init__(self, q: np.ndarray, rs: np.ndarray, cf: np.ndarray):
        self.q, self.rs, self.cf = q, rs, cf


def q82(rng: np.random.Generator, rows: int, cols: int) -> Q82:
    """Draw a q8_2f matrix: q U[-127, 127], row scales U(1e-3, 1e-2) and column field
    U(0.5, 1.5), both rounded to binary16 (the pages fix no distribution; these keep the
    weights in the block format's range)."""
    q = rng.integers(-127, 128, size=(rows, cols), dtype=np.int8)
    rs = rng.uniform(1e-3, 1e-2, size=rows).astype(np.float16)
    cf = rng.uniform(0.5, 1.5, size=cols).astype(np.float16)
    return Q82(q, rs, cf)


class Q4TP:
    """A q4tp matrix: nib uint8 [rows][cols/2] (two 4-bit codes a byte), params uint32 [rows]
    (binary16 base in the low half, step in the high half), codes uint8 [rows][ceil(5 cols/32 / 8)]
    (one 5-bit log-scale code per 32 columns)."""

    def __init__(self, nib: np.ndarray, params: np.ndarray, codes: np.ndarray):
        self.nib, self.params, self.codes = nib, params, codes

    @property
    def rows(self) -> int:
        return self.nib.shape[0]

    @property
    def cols(self) -> int:
        return 2 * self.nib.shape[1]


def q4tp(rng: np.random.Generator, rows: int, cols: int) -> Q4TP:
    """Draw a q4tp matrix: uniform random nibble and code bytes (every 4-bit weight code and
    5-bit scale code equally likely), base U(-9, -7) and step U(0.05, 0.1) rounded to binary16,
    so group scales span about 2^-9 .. 2^-4 (the pages fix no distribution)."""
    assert cols % 32 == 0
    nib = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    codes = rng.integers(0, 256, size=(rows, (5 * (cols // 32) + 7) // 8), dtype=np.uint8)
    base = rng.uniform(-9.0, -7.0, rows).astype(np.float16)
    step = rng.uniform(0.05, 0.1, rows).astype(np.float16)
    params = base.view(np.uint16).astype(np.uint32) | (step.view(np.uint16).astype(np.uint32) << 16)
    return Q4TP(nib, params.astype(np.uint32), codes)


def logits(rng: np.random.Generator, n: int, vocab: int) -> np.ndarray:
    """N(0, 4) logits [n][vocab] f32 (a head output's spread)."""
    return (2.0 * rng.standard_normal((n, vocab))).astype(np.float32)


def f16(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """N(0, 0.02) weights rounded to binary16 (round to nearest even)."""
    return rng.normal(0.0, 0.02, size=(rows, cols)).astype(np.float16)


def normal(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(size=shape, dtype=np.float32)


def norm_weight(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.uniform(0.5, 1.5, size=n).astype(np.float32)


def router_weight(rng: np.random.Generator, experts: int, hidden: int) -> np.ndarray:
    return rng.normal(0.0, 0.02, size=(experts, hidden)).astype(np.float32)


# ---------------------------------------------------------------- workloads
# Each builder draws its tensors in the order written, one spawned stream per
# tensor, so adding a tensor at the end never changes the earlier ones.

def gemv_add_norm(seed: int = 0, rows: int = 1024, cols: int = 1024) -> dict:
    """One q8 GEMV (rows x cols) whose output is added into a residual and RMS-normed."""
    r = streams(seed, 4)
    return {"W": q8(r[0], rows, cols), "x": normal(r[1], cols),
            "h": normal(r[2], rows), "w": norm_weight(r[3], rows), "eps": EPS}


def f16_gemv(seed: int = 0, rows: int = 4096, cols: int = 4096) -> dict:
    r = streams(seed, 2)
    return {"W": f16(r[0], rows, cols), "x": normal(r[1], cols)}


@dataclass
class FrameShape:
    hidden: int = 4096
    qkv: int = 6144
    inter: int = 14336
    vocab: int = 32000


def frame_weights(seed: int = 0, shape: FrameShape = FrameShape()) -> dict:
    """Weights of one layer frame: QKV, up, down, head (q8) and the two norm weights."""
    r = streams(seed, 6)
    H = shape.hidden
    return {"qkv": q8(r[0], shape.qkv, H), "up": q8(r[1], shape.inter, H),
            "down": q8(r[2], H, shape.inter), "head": q8(r[3], shape.vocab, H),
            "w1": norm_weight(r[4], H), "w2": norm_weight(r[5], H), "eps": EPS}


def frame_inputs(seed: int, n: int, hidden: int = 4096) -> dict:
    """Per-position inputs of a frame: x0 (the matrix input) and h0 (the residual)."""
    r = streams(seed + 1_000_003, 2)
    return {"x0": normal(r[0], (n, hidden)), "h0": normal(r[1], (n, hidden))}


@dataclass
class MoEShape:
    n: int = 64
    hidden: int = 2688
    inter: int = 1856
    experts: int = 128
    top_k: int = 6


def attn_pass(seed: int, n: int, pos0: int, nh: int = 32, nkv: int = 8, hd: int = 128,
              ctx: int | None = None) -> dict:
    """A prefill pass's attention inputs: q [n][nh][hd] and the pass's k, v [n][nkv][hd],
    N(0, 1); caches [ctx][nkv][hd] holding N(0, 1) rows for the pos0 earlier positions and
    zeros after (ctx defaults to pos0 + n).  The default heads follow the hidden-4096 frame's
    QKV split (6144 = 32 query heads + 2 x 8 KV heads of 128)."""
    r = streams(seed, 5)
    ctx = pos0 + n if ctx is None else ctx
    kc = np.zeros((ctx, nkv, hd), np.float32)
    vc = np.zeros((ctx, nkv, hd), np.float32)
    kc[:pos0] = normal(r[0], (pos0, nkv, hd))
    vc[:pos0] = normal(r[1], (pos0, nkv, hd))
    return {"q": normal(r[2], (n, nh, hd)), "k": normal(r[3], (n, nkv, hd)), "v": normal(r[4], (n, nkv, hd)),
            "kc": kc, "vc": vc, "pos0": pos0, "scale": float(hd) ** -0.5}


def router_bias(rng: np.random.Generator, E: int) -> np.ndarray:
    """Selection bias of the sigmoid router, U(-0.1, 0.1) per expert (the pages fix no
    distribution; this range reorders experts whose sigmoids are close)."""
    return rng.uniform(-0.1, 0.1, size=E).astype(np.float32)


def moe(seed: int = 0, shape: MoEShape = MoEShape()) -> dict:
    """A routed-MoE pass: input, residual, router, up/down expert banks, norm weight."""
    r = streams(seed, 6)
    n, H, I, E = shape.n, shape.hidden, shape.inter, shape.experts
    return {"X": normal(r[0], (n, H)), "h": normal(r[1], (n, H)),
            "Wr": router_weight(r[2], E, H),
            "up": q8(r[3], I, H, lead=(E,)), "down": q8(r[4], H, I, lead=(E,)),
            "w": norm_weight(r[5], H), "eps": EPS, "top_k": shape.top_k}
