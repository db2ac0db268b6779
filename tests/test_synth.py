"""The seeded input generators: determinism, shapes and the stated distributions."""
import numpy as np

import synth


def test_q8_distribution_and_determinism():
    a = synth.q8(synth.streams(0, 1)[0], 256, 512)
    b = synth.q8(synth.streams(0, 1)[0], 256, 512)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.scale, b.scale)
    assert a.q.dtype == np.int8 and a.q.min() >= -127 and a.q.max() <= 127
    assert a.q.min() == -127 and a.q.max() == 127
    assert a.scale.shape == (256, 16) and a.scale.dtype == np.float32
    assert a.scale.min() >= 1e-3 and a.scale.max() <= 1e-2
    assert abs(float(a.bias.std()) - 1e-3) < 1e-4
    assert a.nbytes() == 256 * 512 * 5 // 4


def test_frame_and_moe_shapes():
    m = synth.moe(0, synth.MoEShape(n=4, hidden=64, inter=96, experts=5, top_k=2))
    assert m["up"].q.shape == (5, 96, 64) and m["down"].q.shape == (5, 64, 96)
    assert m["up"].scale.shape == (5, 96, 2) and m["down"].scale.shape == (5, 64, 3)
    f = synth.frame_inputs(0, 3, hidden=64)
    assert f["x0"].shape == (3, 64) and f["x0"].dtype == np.float32
    w = synth.f16(synth.streams(1, 1)[0], 8, 32)
    assert w.dtype == np.float16


def test_streams_independent_of_later_tensors():
    a = synth.streams(5, 3)
    b = synth.streams(5, 6)
    assert np.array_equal(a[2].integers(0, 1 << 30, 8), b[2].integers(0, 1 << 30, 8))
