"""The activation quantizer divides bf16 x by the smoothing scale s with
Markstein's correction instead of a division instruction:

    q0 = RN(x * rcp),  t = RN(q0 * s - x) (one fused multiply-add),
    q  = RN(q0 - t * rcp) (one fused multiply-add),  rcp = RN(1 / s),

and claims the result is the IEEE quotient RN(x / s) -- the division the
integration paragraph of "W4A4 Quantization for Inference on Wan2.2-I2V-A14B"
prescribes (activations divided by s) -- whenever x = 0 or 2^-100 <= |x| <=
2^100 and 2^-20 <= s <= 2^20 (other rows take a correctly rounded division).

This test emulates those three roundings exactly on the CPU (f32 rounding with
gradual underflow, which is the kernels' f32 denormal mode) and compares them
with numpy's IEEE f32 division for EVERY finite bf16 x of the fast range
(both signs, every exponent from -100 to 100, every mantissa, and +-0) at

* every smoothing scale of the synthetic workloads' plans (the 480p up- and
  down-projections and the 720p up-projection at alpha 0.5 / 0.6 / 0.7), and
* 2048 scales drawn log-uniformly over the whole fast range [2^-20, 2^20].

Exactness of the emulation: x * rcp has at most 8 + 24 significant bits and
q0 * s - x at most 48 (q0 * s is within a few ulps of x), so both are exact in
float64 before their one rounding to f32.  q0 - t * rcp can need more than 53
bits; its float64 value is rounded again to f32, which differs from the single
rounding only when the float64 value lies exactly on an f32 rounding midpoint
-- those elements are recomputed with exact rationals.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import layer


def _fast_range_bf16() -> np.ndarray:
    """Every bf16 x with x = +-0 or 2^-100 <= |x| <= 2^100, as float64."""
    e = np.arange(-100, 101, dtype=np.float64)
    m = 1.0 + np.arange(128, dtype=np.float64) / 128.0
    pos = (m[None, :] * np.exp2(e)[:, None]).reshape(-1)
    pos = pos[pos <= 2.0 ** 100]
    return np.concatenate([[0.0, -0.0], pos, -pos])


def _f32_rn_exact(v: Fraction) -> np.float32:
    """Round a rational to the nearest f32, ties to the even significand."""
    a = np.float32(float(v))
    cands = [np.nextafter(a, np.float32(-np.inf)), a, np.nextafter(a, np.float32(np.inf))]
    best = None
    for c in cands:
        d = abs(Fraction(float(c)) - v)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def markstein_f32(x64: np.ndarray, s: np.float32, rcp: np.float32) -> np.ndarray:
    """The three roundings of the kernel's division, for float64 x (bf16 values)."""
    s64, r64 = float(s), float(rcp)
    q0 = (x64 * r64).astype(np.float32)                       # exact product, one rounding
    t = (q0.astype(np.float64) * s64 - x64).astype(np.float32)   # exact q0*s - x, one rounding
    v64 = q0.astype(np.float64) - t.astype(np.float64) * r64      # may round in float64
    q = v64.astype(np.float32)
    low = v64.view(np.uint64) & np.uint64((1 << 29) - 1)
    mid = (low == np.uint64(1 << 28)) & (np.abs(q) >= np.float32(2.0 ** -126))
    for i in np.flatnonzero(mid):                              # double-rounding candidates
        exact = Fraction(float(q0[i])) - Fraction(float(t[i])) * Fraction(r64)
        q[i] = _f32_rn_exact(exact)
    # results in the f32 subnormal range do not occur: |q| >= 2^-120
    assert np.all((np.abs(q) >= np.float32(2.0 ** -121)) | (q == 0))
    return q


def _plan_scales() -> np.ndarray:
    out = []
    for w in (synth.FFN0_480P, synth.FFN2_480P, synth.FFN0_720P):
        a = layer.act_max(w.make_x())
        wr = layer.weight_range(w.make_w())
        alphas = synth.SWEEP_ALPHA if w is synth.FFN0_720P else (w.alpha,)
        for alpha in alphas:
            out.append(layer.smooth_scales(a, wr, alpha)[0])
    return np.unique(np.concatenate(out))


def _check(scales: np.ndarray) -> int:
    x64 = _fast_range_bf16()
    x32 = x64.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x64)       # every x is an exact bf16/f32 value
    bad = 0
    for s in scales:
        s = np.float32(s)
        assert 2.0 ** -20 <= s <= 2.0 ** 20
        rcp = np.float32(1.0) / s
        got = markstein_f32(x64, s, rcp)
        want = x32 / s                                         # IEEE f32 division
        diff = got.view(np.uint32) != want.view(np.uint32)
        bad += int(diff.sum())
        assert not diff.any(), (float(s), x64[diff][:4], got[diff][:4], want[diff][:4])
    return bad


def test_exact_rounding_helper_ties_to_even():
    one = Fraction(1)
    assert _f32_rn_exact(one + Fraction(1, 2 ** 24)) == np.float32(1.0)                 # tie, even below
    assert _f32_rn_exact(one + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)    # tie, even above
    assert _f32_rn_exact(one + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 60)) == np.float32(1.0 + 2.0 ** -23)
    assert _f32_rn_exact(-one / 3) == np.float32(-1.0) / np.float32(3.0)


def test_emulation_catches_a_reciprocal_product():
    """The comparison can fail: RN(x * rcp) alone (no correction) differs from
    the quotient on many x, while the corrected form does not."""
    x64 = _fast_range_bf16()
    s = np.float32(2.9)
    rcp = np.float32(1.0) / s
    naive = (x64 * float(rcp)).astype(np.float32)
    assert (naive.view(np.uint32) != (x64.astype(np.float32) / s).view(np.uint32)).sum() > 1000
    assert np.array_equal(markstein_f32(x64, s, rcp), x64.astype(np.float32) / s)


def test_markstein_exact_at_random_scales():
    g = np.random.default_rng(20260)
    scales = np.exp2(g.uniform(-20.0, 20.0, 2048)).astype(np.float32)
    scales = np.concatenate([scales, np.float32([2.0 ** -20, 2.0 ** 20, 1.0, 3.0, 1.5, 0.75])])
    assert _check(scales) == 0


@pytest.mark.slow
def test_markstein_exact_at_workload_plan_scales():
    scales = _plan_scales()
    assert scales.size > 5000
    assert _check(scales) == 0
