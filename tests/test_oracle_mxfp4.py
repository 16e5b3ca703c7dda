"""Pins for the oracle's MXFP4 encode/decode against things other than itself.

* exhaustive E2M1 rounding over every finite bf16 value and several scale codes
  versus a brute-force nearest-grid search in exact integer arithmetic;
* the E8M0 scale rule versus math.frexp over every positive finite bf16 amax;
* grid round-trip: blocks built from grid values times a power of two decode exactly;
* hand-worked examples (tests/golden/mxfp4_hand.txt).
"""
import math
import os

import numpy as np
import pytest

from oracle import mxfp4

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mxfp4_hand.txt")
GRID2 = [0, 1, 2, 3, 4, 6, 8, 12]            # the E2M1 grid times 2 (integers)


def _all_finite_bf16_f32():
    b = np.arange(0, 1 << 16, dtype=np.uint32)
    f = (b << np.uint32(16)).view(np.float32)
    return f[np.isfinite(f)]


def _brute_code(mant: int, exp: int) -> int:
    """Nearest grid code to r = mant * 2^exp >= 0, ties to the even code, exact ints."""
    S = 400
    R = mant << (exp + S)
    best, bestd = None, None
    for code, g2 in enumerate(GRID2):
        d = abs(R - (g2 << (S - 1)))
        if bestd is None or d < bestd or (d == bestd and code % 2 == 0):
            best, bestd = code, d
    return best


@pytest.mark.parametrize("c", [0, 1, 100, 125, 127, 130, 200, 252])
def test_e2m1_exhaustive_vs_bruteforce(c):
    v = _all_finite_bf16_f32()
    nib = mxfp4.encode_with_scale(v, np.full(v.shape, c, dtype=np.uint8))
    # brute force over the distinct magnitudes
    mags = np.unique(np.abs(v).astype(np.float64))
    want = {}
    for m in mags:
        if m == 0.0:
            want[0.0] = 0
            continue
        fr, e = math.frexp(float(m))           # m = fr * 2^e, fr in [0.5, 1)
        mant = int(fr * (1 << 24))              # exact (bf16 has 8 significant bits)
        want[float(m)] = _brute_code(mant, e - 24 + 127 - c)
    exp_code = np.array([want[float(abs(x))] for x in v.astype(np.float64)], dtype=np.uint8)
    exp_nib = (np.signbit(v).astype(np.uint8) << 3) | exp_code
    bad = np.nonzero(nib != exp_nib)[0]
    assert bad.size == 0, (c, v[bad[:5]], nib[bad[:5]], exp_nib[bad[:5]])


def test_e8m0_vs_frexp_all_bf16():
    v = _all_finite_bf16_f32()
    v = v[v > 0]
    c = mxfp4.e8m0_from_amax(v).astype(np.int64)
    want = np.array([max(math.frexp(float(x))[1] - 1 - 2 + 127, 0) for x in v], dtype=np.int64)
    assert np.array_equal(c, want)
    # Above the clamp the scaled amax lands in [4, 8): the top binade of E2M1.
    normal = want > 0
    r = np.ldexp(v[normal].astype(np.float64), 127 - c[normal])
    assert r.min() >= 4.0 and r.max() < 8.0
    assert mxfp4.e8m0_from_amax(np.zeros(3, np.float32)).tolist() == [0, 0, 0]


@pytest.mark.parametrize("e", [-120, -20, -3, 0, 5, 60, 100])
def test_grid_roundtrip(e):
    g = np.random.default_rng(e + 1000)
    for top in (0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0):
        allowed = mxfp4.GRID[mxfp4.GRID <= top]
        vals = g.choice(allowed, size=32) * g.choice([-1.0, 1.0], size=32)
        vals[g.integers(32)] = top * g.choice([-1.0, 1.0])
        v = np.ldexp(vals, e).astype(np.float32)[None, :]
        packed, sc = mxfp4.encode_rows(v)
        back = mxfp4.decode_rows(packed, sc)
        assert np.array_equal(back, v.astype(np.float64)), (e, top)


def test_pack_nibble_order():
    nib = np.arange(16, dtype=np.uint8)[None, :]
    b = mxfp4.pack_nibbles(nib)
    assert b.tolist() == [[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]]
    assert np.array_equal(mxfp4.unpack_nibbles(b), nib)


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        left, sc, nibs = line.split("|")
        parts = left.split()
        vals = [float(x) for x in parts[1:]]
        rows.append((parts[0], vals, int(sc), [int(x, 16) for x in nibs.split()]))
    return rows


@pytest.mark.parametrize("row", _golden_rows(), ids=lambda r: r[0])
def test_hand_worked(row):
    _, vals, sc, nibs = row
    v = np.zeros((1, 32), dtype=np.float32)
    v[0, :len(vals)] = vals
    packed, scales = mxfp4.encode_rows(v)
    assert int(scales[0, 0]) == sc
    got = mxfp4.unpack_nibbles(packed)[0, :len(vals)].tolist()
    assert got == nibs


def test_tile_scales_cover_32x32():
    g = np.random.default_rng(7)
    v = (g.standard_normal((64, 64)) * 0.1).astype(np.float32)
    v[40, 3] = 50.0                       # lands in tile (1, 0)
    packed, c_rows, ct = mxfp4.encode_tiles(v)
    assert ct.shape == (2, 2)
    assert ct[1, 0] == mxfp4.e8m0_from_amax(np.float32(50.0))
    for tr in range(2):
        for tb in range(2):
            t = v[tr * 32:(tr + 1) * 32, tb * 32:(tb + 1) * 32]
            assert ct[tr, tb] == mxfp4.e8m0_from_amax(np.abs(t).max())
            assert np.all(c_rows[tr * 32:(tr + 1) * 32, tb] == ct[tr, tb])
    # a 1x32 encode of the same matrix differs only where the tile scale is coarser
    p1, s1 = mxfp4.encode_rows(v)
    assert np.all(s1 <= c_rows)


def test_stripe_scales_128x1():
    """128x1 K-major stripes: one E8M0 per 128 consecutive K of a row.  Pins:
    the stripe code is the E8M0 of the stripe's amax computed independently
    (frexp), it equals the largest of the stripe's four 1x32 codes (E8M0 is
    monotone in the amax), the last (short) stripe of a ragged row covers only
    its own blocks, and decoding loses at most the grid spacing of the
    stripe's scale."""
    g = np.random.default_rng(21)
    v = (g.standard_normal((5, 352)) * 0.2).astype(np.float32)     # K = 352: stripes 128, 128, 96
    v[2, 200] = 40.0
    v[4, 340] = -9.0
    packed, c_blocks, cs = mxfp4.encode_stripes(v, 128)
    assert cs.shape == (5, 3) and c_blocks.shape == (5, 11)
    _, s1 = mxfp4.encode_rows(v)
    for r in range(5):
        for sidx in range(3):
            seg = v[r, sidx * 128:min(352, (sidx + 1) * 128)]
            m, e = math.frexp(float(np.abs(seg).max()))       # amax = m 2^e, 0.5 <= m < 1
            assert cs[r, sidx] == max(e - 1 - 2 + 127, 0)
            blocks = range(sidx * 4, min(11, sidx * 4 + 4))
            assert cs[r, sidx] == max(int(s1[r, b]) for b in blocks)
            assert all(c_blocks[r, b] == cs[r, sidx] for b in blocks)
    dec = mxfp4.decode_rows(packed, c_blocks)
    step = np.repeat(np.exp2(c_blocks.astype(np.float64) - 127), 32, axis=1)   # grid spacing <= 2 x 2^(c-127)
    assert np.all(np.abs(dec - v) <= np.maximum(step, np.abs(v) / 4) + 1e-30)
