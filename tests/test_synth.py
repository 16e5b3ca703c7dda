"""The seeded generators: determinism, chunking, and the magnitudes they are
meant to stand in for (Fig. 2 of the pages: a few activation channels with
column maxima far above the rest, weight column maxima well below 0.6)."""
import numpy as np

import synth


def test_chunked_equals_whole():
    g1 = synth.rng(5)
    whole = g1.standard_normal((10, 7), dtype=np.float32)
    g2 = synth.rng(5)
    parts = np.concatenate([g2.standard_normal((3, 7), dtype=np.float32),
                            g2.standard_normal((7, 7), dtype=np.float32)])
    assert np.array_equal(whole, parts)


def test_generator_determinism_and_chunk_boundary(monkeypatch):
    a = synth.TINY.make_x()
    b = synth.TINY.make_x()
    assert np.array_equal(a, b)
    monkeypatch.setattr(synth, "CHUNK_ROWS", 37)
    c = synth.TINY.make_x()
    assert np.array_equal(a, c)


def test_tiny_magnitudes():
    w = synth.TINY
    X = w.make_x()
    W = w.make_w()
    assert X.shape == (256, 512) and X.dtype == np.float32
    assert W.shape == (1024, 512) and W.dtype == np.float32
    ch = synth.pick_channels(512, 0.02, 101)
    assert ch.size == 10 and np.unique(ch).size == 10
    cmax = np.abs(X).max(axis=0)
    bulk = np.delete(cmax, ch)
    assert bulk.max() < 1.5 and cmax[ch].min() > 6.0
    assert np.abs(W).max() <= 0.6


def test_bf16_rounding_bits():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -0.0], np.float32)
    assert synth.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0x8000]
    assert np.array_equal(synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))[:1], x[:1])


def test_large_workload_small_slice():
    w = synth.FFN0_480P
    X = w.make_x(M=64)
    assert X.dtype == np.uint16 and X.shape == (64, 5120)
    f = synth.bf16_bits_to_f32(X)
    ch = synth.pick_channels(5120, 0.02, 201)
    assert ch.size == 102
    assert np.abs(f[:, ch]).max() > 6.0
    g = synth.FFN2_480P.make_x(M=8)
    assert g.shape == (8, 13824)
    assert synth.pick_channels(13824, 0.01, 301).size == 138
    h = synth.bf16_bits_to_f32(g)
    # a GELU output: negatives no lower than its minimum (about -0.1700 at
    # z = -0.7518), decaying to -0 for very negative z; a heavy positive tail
    assert h.min() >= -0.1702 and (h < 0).mean() > 0.3
    assert h[:, synth.pick_channels(13824, 0.01, 301)].max() > 20.0


def test_gelu_input_recipe():
    """The down-projection input recipe is GELU-tanh of its pre-activation:
    GELU(0) = 0, GELU(z) -> z for large z, -> 0 for very negative z, its
    minimum near z = -0.752, and GELU(z) - GELU(-z) = z (the odd part of z
    Phi(z)-like gates) up to float32 rounding."""
    z = np.array([0.0, 10.0, -10.0, -0.7518, 1.0, -1.0], np.float32)
    h = synth.gelu_tanh_input_f32(z)
    assert h[0] == 0.0 and abs(h[1] - 10.0) < 1e-5 and abs(h[2]) < 1e-5
    assert -0.1701 < h[3] < -0.1699
    assert abs((h[4] - h[5]) - 1.0) < 1e-6
