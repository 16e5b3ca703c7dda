"""The activation quantizer divides bf16 x by the smoothing scale s with
Markstein's correction instead of a division instruction:

    q0 = RN(x * rcp),  t = RN(q0 * s - x) (one fused multiply-add),
    q  = RN(q0 - t * rcp) (one fused multiply-add),  rcp = RN(1 / s),

and takes its codes to be those of the IEEE quotient RN(x / s) -- the
division the integration paragraph of "W4A4 Quantization for Inference on
Wan2.2-I2V-A14B" prescribes (activations divided by s) -- under conditions it
checks on values the encoder forms anyway (a wave that fails them redoes the
row with a correctly rounded division).  For s in [2^-20, 2^20]:

A. |x| >= 2^-100 and |q0| < 2^126: q is the IEEE quotient.
B. 0 < |x| < 2^-100: q and the IEEE quotient both lie below 2^-79 in
   magnitude and carry the sign of x; a q of +-0 stands for an IEEE quotient
   of +-0 or +-2^-149.  Such a value gets a zero code (sign kept) under any
   block whose maximum is at least 2^-74 -- the E8M0 scale is then at least
   2^-76 and the value at most 2^-3 of it -- so the kernel only needs block
   maxima of 0 or >= 2^-74 (C checks the encoder side of this on the oracle).
D. The outlier value is stored itself (bf16): q in [2^-78, 2^126) is the
   IEEE quotient, and q = +-0 rounds to the same bf16 as the IEEE quotient.

This test emulates the three roundings on the CPU (f32 rounding with gradual
underflow, which is the kernels' f32 denormal mode) and compares them with
numpy's IEEE f32 division for EVERY finite bf16 x (both signs, all exponents
and mantissas, subnormals and +-0) at

* every smoothing scale of the synthetic workloads' plans (the 480p up- and
  down-projections and the 720p up-projection at alpha 0.5 / 0.6 / 0.7), and
* 2048 scales drawn log-uniformly over the whole range [2^-20, 2^20].

Exactness of the emulation where A and D claim equality (|x| >= 2^-100):
x * rcp has at most 8 + 24 significant bits and q0 * s - x at most 48 (q0 * s
is within a few ulps of x), so both are exact in float64 before their one
rounding to f32; q0 - t * rcp can need more than 53 bits, and its float64
value is rounded again to f32, which differs from the single rounding only
when the float64 value lies exactly on an f32 rounding midpoint -- those
elements are recomputed with exact rationals.  Under B (tiny x) the
emulation is used only for magnitude and sign bounds with wide margins.
"""
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import layer, mxfp4

P126, PM74, PM78, PM79 = 2.0 ** 126, 2.0 ** -74, 2.0 ** -78, 2.0 ** -79


def _all_finite_bf16() -> np.ndarray:
    """Every finite bf16 value (both zeros included), as float64."""
    b = np.arange(1 << 16, dtype=np.uint32)
    b = b[(b & 0x7F80) != 0x7F80]
    return (b << 16).view(np.float32).astype(np.float64)


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


def markstein_f32(x64: np.ndarray, s: np.float32, rcp: np.float32, exact: bool = True):
    """(q0, q): the kernel's first product and its corrected quotient, for
    float64 x (bf16 values).  exact=True recomputes float64 midpoints of the
    last rounding with rationals (needed where equality is claimed)."""
    s64, r64 = float(s), float(rcp)
    with np.errstate(over="ignore", invalid="ignore"):
        q0 = (x64 * r64).astype(np.float32)                          # exact product, one rounding
        t = (q0.astype(np.float64) * s64 - x64).astype(np.float32)    # q0*s - x, one rounding
        v64 = q0.astype(np.float64) - t.astype(np.float64) * r64       # may round in float64
        q = v64.astype(np.float32)
    if exact:
        low = v64.view(np.uint64) & np.uint64((1 << 29) - 1)
        mid = (low == np.uint64(1 << 28)) & np.isfinite(v64) & (np.abs(q) >= np.float32(2.0 ** -126))
        for i in np.flatnonzero(mid):                                  # double-rounding candidates
            ex = Fraction(float(q0[i])) - Fraction(float(t[i])) * Fraction(r64)
            q[i] = _f32_rn_exact(ex)
    return q0, q


def _plan_scales() -> np.ndarray:
    out = []
    for w in (synth.FFN0_480P, synth.FFN2_480P, synth.FFN0_720P):
        a = layer.act_max(w.make_x())
        wr = layer.weight_range(w.make_w())
        alphas = synth.SWEEP_ALPHA if w is synth.FFN0_720P else (w.alpha,)
        for alpha in alphas:
            out.append(layer.smooth_scales(a, wr, alpha)[0])
    return np.unique(np.concatenate(out))


def _bits(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def _check(scales: np.ndarray) -> dict:
    x64 = _all_finite_bf16()
    x32 = x64.astype(np.float32)
    assert np.array_equal(x32.astype(np.float64), x64)          # every x is an exact bf16/f32 value
    big = np.abs(x64) >= 2.0 ** -100
    tiny = (x64 != 0) & ~big
    xa, xt = x64[big | (x64 == 0)], x64[tiny]
    stats = {"A": 0, "D": 0, "rejected": 0}
    for s in scales:
        s = np.float32(s)
        assert 2.0 ** -20 <= s <= 2.0 ** 20
        rcp = np.float32(1.0) / s
        with np.errstate(over="ignore"):
            want_a = xa.astype(np.float32) / s                   # IEEE f32 division
            want_t = xt.astype(np.float32) / s
        # A: |x| >= 2^-100 (and 0) with |q0| < 2^126 -> exact
        q0, q = markstein_f32(xa, s, rcp)
        acc = np.abs(q0.astype(np.float64)) < P126
        diff = acc & (_bits(q) != _bits(want_a))
        assert not diff.any(), ("A", float(s), xa[diff][:4], q[diff][:4], want_a[diff][:4])
        stats["A"] += int(acc.sum())
        stats["rejected"] += int((~acc).sum())
        # D on the same x: |q| in [2^-78, 2^126) -> exact
        aq = np.abs(q.astype(np.float64))
        win = (aq >= PM78) & (aq < P126)
        diff = win & (_bits(q) != _bits(want_a))
        assert not diff.any(), ("D", float(s), xa[diff][:4])
        stats["D"] += int(win.sum())
        # B: 0 < |x| < 2^-100
        q0t, qt = markstein_f32(xt, s, rcp, exact=False)
        assert np.all(np.abs(qt.astype(np.float64)) < PM79), ("B fast", float(s))
        assert np.all(np.abs(want_t.astype(np.float64)) < PM79), ("B exact", float(s))
        neg = xt < 0
        assert np.array_equal(np.signbit(qt), neg) and np.array_equal(np.signbit(want_t), neg), ("B sign", float(s))
        z = qt == 0
        assert np.all(np.abs(want_t[z].astype(np.float64)) <= 2.0 ** -149), ("B zero", float(s))
        # D for the tiny x: none falls in the window; a fast +-0 gives the IEEE quotient's bf16
        assert not np.any(np.abs(qt.astype(np.float64)) >= PM78)
        assert np.array_equal(layer.bf16_rne(qt[z]), layer.bf16_rne(want_t[z]))
    return stats


def test_exact_rounding_helper_ties_to_even():
    one = Fraction(1)
    assert _f32_rn_exact(one + Fraction(1, 2 ** 24)) == np.float32(1.0)                 # tie, even below
    assert _f32_rn_exact(one + Fraction(3, 2 ** 24)) == np.float32(1.0 + 2.0 ** -22)    # tie, even above
    assert _f32_rn_exact(one + Fraction(1, 2 ** 24) + Fraction(1, 2 ** 60)) == np.float32(1.0 + 2.0 ** -23)
    assert _f32_rn_exact(-one / 3) == np.float32(-1.0) / np.float32(3.0)


def test_emulation_catches_a_reciprocal_product():
    """The comparison can fail: RN(x * rcp) alone (no correction) differs from
    the quotient on many x, while the corrected form does not."""
    x64 = _all_finite_bf16()
    x64 = x64[(np.abs(x64) >= 2.0 ** -100) & (np.abs(x64) < 2.0 ** 100)]
    s = np.float32(2.9)
    rcp = np.float32(1.0) / s
    naive = (x64 * float(rcp)).astype(np.float32)
    assert (naive.view(np.uint32) != (x64.astype(np.float32) / s).view(np.uint32)).sum() > 1000
    assert np.array_equal(markstein_f32(x64, s, rcp)[1], x64.astype(np.float32) / s)


def test_large_quotients_are_rejected_not_wrong():
    """Near overflow the check on q0 is what keeps the fast path exact: with
    s = 2^-20 the largest bf16 values overflow q0, and the accepted ones
    (|q0| < 2^126) are exact."""
    s = np.float32(2.0 ** -20)
    rcp = np.float32(1.0) / s
    x64 = _all_finite_bf16()
    q0, q = markstein_f32(x64, s, rcp)
    assert np.isinf(q0).any()                                         # overflowing x exist ...
    assert np.isnan(q[np.isinf(q0)]).all()                            # ... and give NaN, not a value
    st = _check(np.float32([2.0 ** -20]))
    assert st["rejected"] > 0 and st["A"] > 0


def test_tiny_values_encode_to_zero_under_accepted_block_maxima():
    """C: with a block maximum of at least 2^-74 (the smallest the kernel
    accepts besides 0) every |q| < 2^-79 gets a zero magnitude code and the
    scale code does not depend on it (oracle encoder)."""
    g = np.random.default_rng(7)
    for amax in (2.0 ** -74, 1.5 * 2.0 ** -74, 2.0 ** -60, 1.0, 2.0 ** 100):
        v = np.zeros((64, 32), np.float32)
        v[:, 0] = np.float32(amax)
        tiny = np.float32(np.exp2(g.uniform(-149.0, -79.0, (64, 31))) * g.choice([-1.0, 1.0], (64, 31)))
        tiny[:, 0] = -np.float32(2.0 ** -79) * np.float32(1 - 2.0 ** -23)   # the largest magnitude allowed
        v[:, 1:] = tiny
        c = mxfp4.e8m0_from_amax(np.abs(v).max(axis=1))
        assert np.all(c == mxfp4.e8m0_from_amax(np.full(64, np.float32(amax))))
        nib = mxfp4.encode_with_scale(v, np.repeat(c[:, None], 32, axis=1))
        assert np.all((nib[:, 1:] & 7) == 0)                           # magnitude code 0
        assert np.array_equal(nib[:, 1:] >> 3, (v[:, 1:] < 0).astype(nib.dtype))   # sign kept


def test_markstein_at_random_scales():
    g = np.random.default_rng(20260)
    scales = np.exp2(g.uniform(-20.0, 20.0, 2048)).astype(np.float32)
    scales = np.concatenate([scales, np.float32([2.0 ** -20, 2.0 ** 20, 1.0, 3.0, 1.5, 0.75])])
    st = _check(scales)
    assert st["A"] > 0 and st["D"] > 0


@pytest.mark.slow
def test_markstein_at_workload_plan_scales():
    scales = _plan_scales()
    assert scales.size > 5000
    st = _check(scales)
    assert st["A"] > 0
