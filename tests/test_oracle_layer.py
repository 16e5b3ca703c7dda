"""Pins for the oracle's calibrate / plan / forward against closed forms,
identities, brute force and exact rational arithmetic.

Equation numbers refer to "W4A4 Quantization for Inference on Wan2.2-I2V-A14B"
(arXiv 2606.29337).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import layer, mxfp4

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
        Fraction(4), Fraction(6)]


def _bf16(x):
    return layer.bf16_rne(np.asarray(x, np.float32))


def _small_layer(M, K, N, seed, outl=3, mult=25.0):
    g = np.random.default_rng(seed)
    X = (g.standard_normal((M, K)) * 0.25).astype(np.float32)
    ch = g.choice(K, size=outl, replace=False)
    X[:, ch] *= mult
    W = np.clip(g.standard_normal((N, K)) * 0.05, -0.6, 0.6).astype(np.float32)
    return X, W, ch


# ----------------------------------------------------------------------------- calibration

def test_act_max_bruteforce_and_invariances():
    X, W, _ = _small_layer(37, 64, 8, 1)
    a = layer.act_max(X)
    want = [max(abs(float(X[t, j])) for t in range(X.shape[0])) for j in range(X.shape[1])]
    assert a.tolist() == want
    perm = np.random.default_rng(2).permutation(X.shape[0])
    assert np.array_equal(layer.act_max(X[perm]), a)
    run = layer.act_max(X[:10])
    run = layer.act_max(X[10:11], run)
    run = layer.act_max(X[11:], run)
    assert np.array_equal(run, a)
    Xb = _bf16(X)
    assert np.array_equal(layer.act_max(Xb), np.abs(layer.as_f32(Xb)).max(axis=0))


def test_weight_range_bruteforce():
    _, W, _ = _small_layer(4, 64, 9, 3)
    w = layer.weight_range(W)
    assert w.tolist() == [max(abs(float(W[n, j])) for n in range(W.shape[0])) for j in range(64)]


# ----------------------------------------------------------------------------- Eq. (2)

@pytest.mark.parametrize("alpha", [0.3, 0.5, 0.6, 0.7])
def test_smooth_scale_closed_form(alpha):
    X, W, _ = _small_layer(64, 128, 16, 4)
    a, w = layer.act_max(X), layer.weight_range(W)
    s, rcp = layer.smooth_scales(a, w, alpha)
    for j in range(0, 128, 7):
        want = math.exp(alpha * math.log(float(a[j])) - (1 - alpha) * math.log(float(w[j])))
        assert abs(float(s[j]) - want) <= 2 ** -23 * want        # within one f32 rounding
        # (a/s) and (w s) are the two geometric forms of the fold
        assert math.isclose(float(a[j]) / float(s[j]), (float(a[j]) * float(w[j])) ** (1 - alpha),
                            rel_tol=1e-6)
        assert math.isclose(float(w[j]) * float(s[j]), (float(a[j]) * float(w[j])) ** alpha,
                            rel_tol=1e-6)
        assert float(rcp[j]) == float(np.float32(1.0) / s[j])
    # larger alpha pushes more of the channel-to-channel dynamic range into W:
    # the spread of the folded weight maxima (a w)^alpha grows, that of the
    # smoothed activation maxima (a w)^(1-alpha) shrinks
    s2, _ = layer.smooth_scales(a, w, min(alpha + 0.1, 0.9))
    spread = lambda v: float(v.max() / v.min())
    assert spread(w * s2) > spread(w * s) and spread(a / s2) < spread(a / s)


def _f32_neighbours(x: float) -> set:
    """The f32 values next to the real x (one of them is any faithful rounding)."""
    lo = float(np.float32(x))
    if lo > x:
        lo = float(np.nextafter(np.float32(lo), np.float32(-np.inf)))
    return {lo, float(np.nextafter(np.float32(lo), np.float32(np.inf)))}


def test_smooth_scale_floor_at_zero_statistics():
    """Eq. (2) on dead channels (reading: both statistics are floored at 1e-5
    before the powers).  Pinned without the oracle's own pow: at a = w = 0 the
    scale is 1e-5^(2 alpha - 1) -- exactly 1 at alpha = 0.5, sqrt(1e-5) at
    0.75, 1/sqrt(1e-5) at 0.25 --, a zero activation channel with a live
    weight column gives exp(alpha ln 1e-5 - (1 - alpha) ln w), a live
    activation channel with a zero weight column exp(alpha ln a - (1 - alpha)
    ln 1e-5); everything below the floor (zero, subnormals, 1e-6) gives the
    same s as the floor itself, and just above it s moves."""
    z = np.zeros(1, np.float32)
    s, rcp = layer.smooth_scales(z, z, 0.5)
    assert float(s[0]) == 1.0 and float(rcp[0]) == 1.0
    s, _ = layer.smooth_scales(z, z, 0.75)
    assert float(s[0]) in _f32_neighbours(math.sqrt(1e-5))
    s, _ = layer.smooth_scales(z, z, 0.25)
    assert float(s[0]) in _f32_neighbours(1.0 / math.sqrt(1e-5))
    w = np.array([0.09, 0.5, 3e-5], np.float32)
    for alpha in (0.3, 0.5, 0.6, 0.7):
        s, _ = layer.smooth_scales(np.zeros(3, np.float32), w, alpha)
        for j in range(3):
            want = math.exp(alpha * math.log(1e-5) - (1 - alpha) * math.log(float(w[j])))
            assert float(s[j]) in _f32_neighbours(want), (alpha, j)
        a = np.array([0.7, 25.0, 2e-5], np.float32)
        s, _ = layer.smooth_scales(a, np.zeros(3, np.float32), alpha)
        for j in range(3):
            want = math.exp(alpha * math.log(float(a[j])) - (1 - alpha) * math.log(1e-5))
            assert float(s[j]) in _f32_neighbours(want), (alpha, j)
    below = np.array([0.0, 1e-45, 1e-38, 1e-6, 9.9e-6, 1e-5], np.float32)
    below[-1] = np.float32(1e-5) if float(np.float32(1e-5)) <= 1e-5 else np.nextafter(np.float32(1e-5), np.float32(0))
    wcol = np.full(below.size, 0.2, np.float32)
    s_a, _ = layer.smooth_scales(below, wcol, 0.6)
    s_w, _ = layer.smooth_scales(wcol, below, 0.6)
    assert np.unique(s_a).size == 1 and np.unique(s_w).size == 1
    above = np.array([2e-5], np.float32)
    assert layer.smooth_scales(above, wcol[:1], 0.6)[0][0] > s_a[0]
    assert layer.smooth_scales(wcol[:1], above, 0.6)[0][0] < s_w[0]


def test_smooth_off_is_identity():
    a = np.array([3.0, 0.5], np.float32)
    s, rcp = layer.smooth_scales(a, a, 0.5, smooth=False)
    assert s.tolist() == [1.0, 1.0] and rcp.tolist() == [1.0, 1.0]


def test_alpha_half_balances_maxima():
    """At alpha = 0.5 the activation and weight maxima of each channel are equal
    after the fold (up to f32 rounding), and the smoothed activation maximum is
    exactly RN(a_j / s_j) because rounding is monotone."""
    X, W, _ = _small_layer(128, 64, 32, 5)
    a, w = layer.act_max(X), layer.weight_range(W)
    s, _ = layer.smooth_scales(a, w, 0.5)
    q = X / s[None, :]
    qmax = np.abs(q).max(axis=0)
    assert np.array_equal(qmax, (a / s).astype(np.float32))
    wmax = np.abs(W * s[None, :]).max(axis=0)
    assert np.allclose(qmax, wmax, rtol=4 * 2 ** -23, atol=0)


# ----------------------------------------------------------------------------- Eq. (1)

def test_fold_identity_f64():
    X, W, _ = _small_layer(16, 64, 24, 6)
    a, w = layer.act_max(X), layer.weight_range(W)
    s, _ = layer.smooth_scales(a, w, 0.6)
    s64 = s.astype(np.float64)
    Y0 = X.astype(np.float64) @ W.astype(np.float64).T
    Y1 = (X.astype(np.float64) / s64) @ (W.astype(np.float64) * s64).T
    assert np.abs(Y1 - Y0).max() <= 1e-13 * np.abs(Y0).max()


# ----------------------------------------------------------------------------- Eq. (4)

def test_topk_bruteforce_with_ties():
    a = np.array([3, 1, 3, 2, 5, 1, 3, 0, 2, 5], np.float32)
    K = a.size
    for k in range(K + 1):
        O, pos = layer.outlier_set(a, k)
        winners = []
        for sub in itertools.combinations(range(K), k):
            rest = [j for j in range(K) if j not in sub]
            # every member outranks every non-member under (score desc, index asc)
            if all((a[i] > a[r]) or (a[i] == a[r] and i < r) for i in sub for r in rest):
                winners.append(sub)
        assert len(winners) == 1
        assert O.tolist() == list(winners[0])
        assert all(pos[O[i]] == i for i in range(k))
        assert np.sum(pos >= 0) == k


# ----------------------------------------------------------------------------- forward pieces

def test_quantize_divides_exactly():
    """q = x / s rounded once to f32 (checked against exact rationals)."""
    g = np.random.default_rng(8)
    x = (g.standard_normal(64) * 3).astype(np.float32)
    s = (np.abs(g.standard_normal(64)) * 5 + 0.1).astype(np.float32)
    q = (x / s).astype(np.float32)
    for xi, si, qi in zip(x, s, q):
        exact = Fraction(float(xi)) / Fraction(float(si))
        lo = np.nextafter(qi, np.float32(-np.inf))
        hi = np.nextafter(qi, np.float32(np.inf))
        d = abs(Fraction(float(qi)) - exact)
        assert d <= abs(Fraction(float(lo)) - exact) and d <= abs(Fraction(float(hi)) - exact)


def test_outlier_columns_leave_block_scales():
    """Routing: an O column is gathered to XO and zeroed in the bulk, so its
    magnitude cannot set the bulk block scale (the point of the split)."""
    X = np.full((2, 64), 0.1, np.float32)
    X[:, 5] = 1000.0
    s = np.ones(64, np.float32)
    O = np.array([5], np.int32)
    r = layer.quantize_act(X, s, O)
    assert np.all(r["As"] == mxfp4.e8m0_from_amax(np.float32(0.1)))
    assert np.all(mxfp4.unpack_nibbles(r["Aq"])[:, 5] == 0)
    assert np.all(layer.as_f32(r["XO"])[:, 0] == 1000.0)
    r0 = layer.quantize_act(X, s, np.zeros(0, np.int32))
    assert r0["As"][0, 0] == mxfp4.e8m0_from_amax(np.float32(1000.0))


def _decode_fraction(packed_row, scale_row, K):
    out = []
    for j in range(K):
        byte = int(packed_row[j // 2])
        nib = byte & 0xF if j % 2 == 0 else byte >> 4
        v = E2M1[nib & 7] * Fraction(2) ** (int(scale_row[j // 32]) - 127)
        out.append(-v if nib & 8 else v)
    return out


def _bf16_fraction(bits):
    return Fraction(float(layer.as_f32(np.asarray([bits], np.uint16))[0]))


@pytest.mark.parametrize("k", [0, 2, 64])
def test_tiny_gemm_exact_rational(k):
    M, K, N = 3, 64, 5
    X, W, _ = _small_layer(M, K, N, 9, outl=4)
    a, w = layer.act_max(X), layer.weight_range(W)
    p = layer.plan(a, w, W, 0.5, k)
    qa = layer.quantize_act(X, p["s"], p["O"])
    Y = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    assert Y.shape == (M, N)
    for m in range(M):
        xa = _decode_fraction(qa["Aq"][m], qa["As"][m], K)
        for n in range(N):
            wb = _decode_fraction(p["Wq"][n], p["Ws"][n], K)
            acc = sum(xi * wi for xi, wi in zip(xa, wb))
            for i in range(k):
                acc += _bf16_fraction(qa["XO"][m, i]) * _bf16_fraction(p["WO"][n, i])
            assert abs(Fraction(float(Y[m, n])) - acc) <= Fraction(1, 10 ** 12) * (1 + abs(acc))


def test_k_equals_K_is_bf16_gemm():
    """k = K routes every channel to the high-precision branch: the bulk is all
    zero codes and Y is the f64 product of bf16(X/s) and bf16(s*W); with
    smoothing off that is the plain bf16 GEMM of X and W."""
    M, K, N = 24, 64, 40
    X, W, _ = _small_layer(M, K, N, 10)
    Xb, Wb = _bf16(X), _bf16(W)
    a, w = layer.act_max(Xb), layer.weight_range(Wb)
    p = layer.plan(a, w, Wb, 0.5, K, smooth=False)
    qa = layer.quantize_act(Xb, p["s"], p["O"])
    assert np.all(qa["Aq"] == 0) and np.all(p["Wq"] == 0)
    Y = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    ref = layer.as_f32(Xb).astype(np.float64) @ layer.as_f32(Wb).astype(np.float64).T
    assert np.abs(Y - ref).max() <= 1e-14 * np.abs(ref).max()
    # smoothing on: the fold keeps the product within two bf16 roundings
    p = layer.plan(a, w, Wb, 0.6, K)
    qa = layer.quantize_act(Xb, p["s"], p["O"])
    Y = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    bound = (2 * 2 ** -9 + 2 ** -16) * (np.abs(layer.as_f32(Xb)).astype(np.float64)
                                         @ np.abs(layer.as_f32(Wb)).astype(np.float64).T)
    assert np.all(np.abs(Y - ref) <= bound)


def test_k_zero_is_pure_w4a4():
    M, K, N = 8, 96, 12
    X, W, _ = _small_layer(M, K, N, 11)
    a, w = layer.act_max(X), layer.weight_range(W)
    p = layer.plan(a, w, W, 0.6, 0)
    assert p["O"].size == 0 and np.all(p["pos"] == -1) and p["WO"].shape == (N, 0)
    qa = layer.quantize_act(X, p["s"], p["O"])
    assert qa["XO"].shape == (M, 0)
    Y = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    # the bulk codes are exactly the uniform MXFP4 encodes of X/s and s*W
    q = (X / p["s"][None, :]).astype(np.float32)
    Aq, As = mxfp4.encode_rows(q)
    assert np.array_equal(Aq, qa["Aq"]) and np.array_equal(As, qa["As"])
    ref = mxfp4.decode_rows(Aq, As) @ mxfp4.decode_rows(p["Wq"], p["Ws"]).T
    assert np.array_equal(Y, ref)


def test_sign_symmetry_and_power_of_two():
    M, K, N = 16, 64, 32
    X, W, _ = _small_layer(M, K, N, 12)
    a, w = layer.act_max(X), layer.weight_range(W)
    p = layer.plan(a, w, W, 0.5, 4)
    Y = layer.forward_f64(X, p)
    Yn = layer.forward_f64(-X, p)
    assert np.array_equal(Yn, -Y)
    # smoothing off: X * 2^3 and W * 2^-2 scale Y by exactly 2^1
    p0 = layer.plan(a, w, W, 0.5, 4, smooth=False)
    p1 = layer.plan(a * 8, w / 4, (W / 4).astype(np.float32), 0.5, 4, smooth=False)
    Y0 = layer.forward_f64(X, p0)
    Y1 = layer.forward_f64((X * 8).astype(np.float32), p1)
    assert np.array_equal(Y1, Y0 * 2)


def test_fold_pack_tiles_match_rows_on_uniform_tiles():
    """When every 32-row group of a 32-column block has the same amax in every
    row, the 32x32 tile scale equals the 1x32 scale and the codes agree."""
    N, K = 64, 64
    g = np.random.default_rng(13)
    W = (g.uniform(-0.5, 0.5, (N, K))).astype(np.float32)
    W[:, ::32] = 0.5                      # every row of every block has amax 0.5
    s = np.ones(K, np.float32)
    O = np.zeros(0, np.int32)
    r1 = layer.fold_pack(W, s, O, "1x32")
    r2 = layer.fold_pack(W, s, O, "32x32")
    assert np.array_equal(r1["Wq"], r2["Wq"]) and np.array_equal(r1["Ws"], r2["Ws"])
    assert r2["Wst"].shape == (2, 2)


def test_gelu_closed_form():
    ys = np.array([-6.0, -1.5, -0.3, 0.0, 0.2, 1.0, 3.7, 10.0])
    got = layer.gelu_tanh(ys)
    for y, gv in zip(ys, got):
        want = 0.5 * y * (1 + math.tanh(math.sqrt(2 / math.pi) * (y + 0.044715 * y ** 3)))
        assert math.isclose(gv, want, rel_tol=1e-14, abs_tol=1e-300)
    assert got[3] == 0.0 and math.isclose(got[-1], 10.0)
    # close to the exact erf GELU (the tanh form's purpose), within its known 1e-3 error
    for y, gv in zip(ys, got):
        exact = 0.5 * y * (1 + math.erf(y / math.sqrt(2)))
        assert abs(gv - exact) < 1e-3


def test_bf16_rne_ties():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: ties to even -> 1.0
    assert int(_bf16([1 + 2 ** -8])[0]) == 0x3F80
    # 1 + 3*2^-8 is halfway between 1.0078125 (odd) and 1.015625 (even)
    assert int(_bf16([1 + 3 * 2 ** -8])[0]) == 0x3F82
    assert int(_bf16([-2.0])[0]) == 0xC000


def test_quantize_uses_division_not_reciprocal_product():
    """The activation is divided by s (Reading: one IEEE f32 division).  At an
    E2M1 tie the exact quotient picks the even code; a product with a rounded
    reciprocal lands off the tie for these s and would pick the other code."""
    g = np.random.default_rng(14)
    found = 0
    for t, even_code in ((0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)):
        for _ in range(20000):
            s = np.float32(np.ldexp(float(g.integers(1 << 12, 1 << 13)), int(g.integers(-14, -8))))
            x = np.float32(t * float(s))
            assert float(x) == t * float(s)
            if np.float32(x * (np.float32(1.0) / s)) != np.float32(t):
                break
        else:
            continue
        found += 1
        X = np.zeros((1, 32), np.float32)
        X[0, 0] = np.float32(6.0) * s            # block amax -> quotient 6 -> scale 2^0
        X[0, 1] = x
        S = np.full(32, s, np.float32)
        r = layer.quantize_act(X, S, np.zeros(0, np.int32))
        assert int(r["As"][0, 0]) == 127
        assert int(mxfp4.unpack_nibbles(r["Aq"])[0, 1]) == even_code, t
    assert found >= 3


def test_fold_pack_stripes_match_rows_on_uniform_stripes():
    """When all four 32-blocks of every 128-stripe have the same amax, the
    128x1 stripe codes equal the 1x32 codes and the nibbles agree; Wst holds
    one code per row and stripe."""
    N, K = 8, 256
    g = np.random.default_rng(17)
    W = g.uniform(-0.5, 0.5, (N, K)).astype(np.float32)
    W[:, ::32] = 0.5
    s = np.ones(K, np.float32)
    O = np.zeros(0, np.int32)
    r1 = layer.fold_pack(W, s, O, "1x32")
    r2 = layer.fold_pack(W, s, O, "128x1")
    assert np.array_equal(r1["Wq"], r2["Wq"]) and np.array_equal(r1["Ws"], r2["Ws"])
    assert r2["Wst"].shape == (N, 2) and np.all(r2["Wst"] == r1["Ws"][:, ::4])


def test_smoothed_score_ranks_by_product():
    """With smoothing, a_j / s_j = (a_j w_j)^(1 - alpha) (Eq. (2)), a monotone
    function of a_j w_j: the smoothed-score top-k is the top-k of a_j w_j
    (values spread far apart, so f32 rounding cannot reorder them).  With
    smoothing off the smoothed score is the raw score."""
    K, k = 40, 7
    g = np.random.default_rng(5)
    rank = g.permutation(K)
    a = (np.exp(g.uniform(-2, 3, K))).astype(np.float32)
    w = (1.5 ** (rank - 30.0) / a).astype(np.float32)            # products a_j w_j ~ 1.5^rank_j
    prod = a.astype(np.float64) * w.astype(np.float64)
    order = np.argsort(-prod)
    assert np.all(np.diff(prod[order]) < -0.3 * prod[order][1:])      # well separated
    for alpha in (0.3, 0.5, 0.7):
        s, _ = layer.smooth_scales(a, w, alpha)
        O, _ = layer.outlier_set(layer.outlier_score(a, s, "smoothed"), k)
        assert np.array_equal(O, np.sort(order[:k]))
    s1, _ = layer.smooth_scales(a, w, 0.5, smooth=False)
    assert np.array_equal(layer.outlier_score(a, s1, "smoothed"), a)
    # the score is the largest smoothed activation of the channel
    X = (g.standard_normal((50, K)) * a[None, :]).astype(np.float32)
    a_x = layer.act_max(X)
    s, _ = layer.smooth_scales(a_x, w, 0.6)
    q = layer.as_f32(X) / s[None, :]
    assert np.array_equal(layer.outlier_score(a_x, s, "smoothed"), np.abs(q).max(axis=0).astype(np.float32))


# ----------------------------------------------------------------------------- percentile statistic

def _percentile_by_counting(cols, q):
    """The nearest-rank q-quantile written as a count: the smallest value v
    among the column's magnitudes with #{t : |x_t| <= v} >= ceil(q T)."""
    out = []
    for c in cols:
        mags = [abs(float(x)) for x in c]
        T = len(mags)
        r = min(T, max(1, math.ceil(q * T)))
        out.append(min(v for v in mags if sum(1 for u in mags if u <= v) >= r))
    return out


@pytest.mark.parametrize("q", [0.5, 0.9, 0.99, 0.999, 1.0, 1e-9])
def test_act_percentile_bruteforce(q):
    g = np.random.default_rng(11)
    X = _bf16((g.standard_normal((53, 9)) * np.exp(g.uniform(-3, 3, 9))[None, :]).astype(np.float32))
    X[g.random(X.shape) < 0.2] = 0x8000                    # signed zeros and ties at 0
    X[:7, 4] = X[7, 4]                                     # ties in the middle
    got = layer.act_percentile([X], q)
    want = _percentile_by_counting(layer.as_f32(X).T, q)
    assert got.tolist() == want


def test_act_percentile_special_cases_and_batches():
    g = np.random.default_rng(12)
    X = _bf16((g.standard_normal((300, 16)) * 3.0).astype(np.float32))
    parts = [X[:120], X[120:121], X[121:]]
    # q = 1 is the running maximum over the batches; q <= 1/T the minimum magnitude
    assert np.array_equal(layer.act_percentile(parts, 1.0),
                          layer.act_max(parts[2], layer.act_max(parts[1], layer.act_max(parts[0]))))
    assert np.array_equal(layer.act_percentile(parts, 1.0 / 300), np.abs(layer.as_f32(X)).min(axis=0))
    # the statistic of the union: independent of how rows are split or ordered
    perm = g.permutation(300)
    for q in (0.3, 0.95, 0.999):
        whole = layer.act_percentile([X], q)
        assert np.array_equal(layer.act_percentile(parts, q), whole)
        assert np.array_equal(layer.act_percentile([X[perm[:77]], X[perm[77:]]], q), whole)


def test_act_percentile_closed_form():
    """A column holding c, 2c, ..., Tc (shuffled, signs mixed): the q-quantile
    of rank ceil(q T) is ceil(q T) c exactly."""
    T = 200
    g = np.random.default_rng(13)
    c = 0.125
    vals = (np.arange(1, T + 1) * c * np.where(g.random(T) < 0.5, -1.0, 1.0)).astype(np.float32)
    X = _bf16(g.permutation(vals)[:, None])
    for q in (0.5, 0.9, 0.955, 0.995, 1.0):
        assert float(layer.act_percentile([X], q)[0]) == math.ceil(q * T) * c


def test_plan_ranks_the_given_statistic():
    """Eq. (4) over a percentile statistic: O is the top-k of that statistic,
    while s still comes from the maxima."""
    X, W, _ = _small_layer(64, 96, 8, 14)
    a, w = layer.act_max(X), layer.weight_range(W)
    pct = layer.act_percentile([X], 0.9)
    p = layer.plan(a, w, W, 0.5, 6, rank=pct)
    O, _ = layer.outlier_set(pct, 6)
    s, _ = layer.smooth_scales(a, w, 0.5)
    assert np.array_equal(p["O"], O) and np.array_equal(p["s"], s)
    ps = layer.plan(a, w, W, 0.5, 6, score="smoothed", rank=pct)
    assert np.array_equal(ps["O"], layer.outlier_set(layer.outlier_score(pct, s, "smoothed"), 6)[0])
