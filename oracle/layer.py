"""Calibrate -> plan(alpha, k) -> forward of the dual-branch W4A4 layer -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

All equations are from "W4A4 Quantization for Inference on Wan2.2-I2V-A14B"
(arXiv 2606.29337).  Readings of points the pages leave open are marked
"Reading:" and are the same readings the GPU path implements.

Shapes: X [M][K] (tokens x input channels), W [N][K] (nn.Linear layout);
bf16 arrays are uint16 bit patterns, f32 arrays float32.
"""
from __future__ import annotations

import math

import numpy as np

from . import mxfp4

EPS = 1e-5   # Reading: floor on the calibration statistics before the power in Eq. (2).


# ----------------------------------------------------------------------------- numerics

def as_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) or float32 -> float32 (exact)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32)
    assert x.dtype == np.float32
    return x


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite values)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    assert np.all(np.isfinite(x))
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    return ((bits + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint16)


# ----------------------------------------------------------------------------- calibration

def act_max(X: np.ndarray, prev: np.ndarray | None = None) -> np.ndarray:
    """Per-input-channel activation maximum a_j = max_t |x_tj| (Eq. (4)'s score,
    the calibration paragraph's per-input-channel activation maxima), as a
    running maximum over calibration batches when ``prev`` is given."""
    x = as_f32(X)
    assert np.all(np.isfinite(x))
    a = np.abs(x).max(axis=0).astype(np.float32)
    return a if prev is None else np.maximum(prev, a)


def act_percentile(batches, q: float) -> np.ndarray:
    """Per-input-channel tail statistic for the channel mask: the q-quantile of
    |x_tj| over every calibration row t of every batch (the tail-aware
    percentile calibration page: a percentile of the activation tail builds
    the channel mask, damping rare calibration outliers; it gives no formula
    and no level).

    Reading: nearest rank.  With T rows in total, the value of rank
    r = ceil(q T) (1-based, clamped to [1, T]) in ascending order of |x_tj|,
    for 0 < q <= 1; q = 1 is the maximum a_j.  bf16 (or f32) inputs, f32 out
    (exact: the result is one of the inputs' magnitudes)."""
    assert 0.0 < q <= 1.0
    xs = np.concatenate([np.abs(as_f32(X)) for X in batches], axis=0)
    assert np.all(np.isfinite(xs))
    T = xs.shape[0]
    r = min(T, max(1, math.ceil(q * T)))
    return np.sort(xs, axis=0)[r - 1].astype(np.float32)


def weight_range(W: np.ndarray) -> np.ndarray:
    """Weight column range of input channel j.  Reading: max_n |W[n][j]| (the
    magnitude counterpart of the activation maximum in Eq. (2))."""
    return np.abs(as_f32(W)).max(axis=0).astype(np.float32)


# ----------------------------------------------------------------------------- plan

def smooth_scales(a: np.ndarray, w: np.ndarray, alpha: float, smooth: bool = True
                  ) -> tuple[np.ndarray, np.ndarray]:
    """Eq. (2): s_j = a_j^alpha / w_j^(1-alpha), alpha in (0, 1).

    Reading: evaluated in float64 on max(stat, 1e-5), rounded once to f32.
    s = 1 when smoothing is off.  Also returns rcp = RN_f32(1 / s), the
    reciprocal the GPU uses inside its division (not part of the semantics)."""
    K = a.shape[0]
    if not smooth:
        s = np.ones(K, dtype=np.float32)
    else:
        assert 0.0 < alpha < 1.0
        a64 = np.maximum(a.astype(np.float64), EPS)
        w64 = np.maximum(w.astype(np.float64), EPS)
        s = (a64 ** alpha / w64 ** (1.0 - alpha)).astype(np.float32)
    rcp = (np.float32(1.0) / s).astype(np.float32)
    return s, rcp


def outlier_set(a: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Eq. (4): O = the top-k input channels by score a_j.

    Reading: order by (a_j descending, j ascending) so ties go to the lower
    channel; O is stored ascending (a sparse index list); pos[j] = index of j
    in O, or -1 for bulk channels."""
    K = a.shape[0]
    assert 0 <= k <= K
    order = np.lexsort((np.arange(K), -a.astype(np.float64)))
    O = np.sort(order[:k]).astype(np.int32)
    pos = np.full(K, -1, dtype=np.int32)
    pos[O] = np.arange(k, dtype=np.int32)
    return O, pos


def outlier_score(a: np.ndarray, s: np.ndarray, mode: str = "max") -> np.ndarray:
    """The per-channel score Eq. (4) ranks.  "max": the calibration maximum
    a_j (Eq. (4) as written).  "smoothed": the maximum of the smoothed
    activations, max_t |x_tj / s_j| = RN32(a_j / s_j) (RN is monotone), i.e.
    the channels that stay largest after the fold (the reading in which the
    split follows the smoothing)."""
    if mode == "max":
        return a.astype(np.float32)
    if mode == "smoothed":
        return (a.astype(np.float32) / s.astype(np.float32)).astype(np.float32)
    raise ValueError(mode)


def fold_pack(W: np.ndarray, s: np.ndarray, O: np.ndarray, layout: str = "1x32") -> dict:
    """Eq. (1) fold and the block packing of the weights.

    W' = RN_f32(s_j * W[n][j]) (s folded into the master weights before
    packing); the outlier columns W'[:, O] are extracted to bf16 (WO [N][k]);
    the bulk weights are W' with the O columns set to +0 (masked in place,
    keeping 32-block alignment) and MXFP4-encoded with 1x32 K-blocks, 32x32
    tiles or 128x1 K-major stripes (the block-packing paragraph and Fig. 8 of
    the paper's text).  Returns Wq [N][K/2], Ws [N][K/32] (per-block codes; for
    tiles the tile code repeated over its 32 rows, for stripes the stripe code
    repeated over its 4 blocks), Wst (the compact codes: [N/32][K/32] for tiles,
    [N][ceil(K/128)] for stripes; None for 1x32), WO [N][k]."""
    Wf = (as_f32(W) * s[None, :].astype(np.float32)).astype(np.float32)
    WO = bf16_rne(Wf[:, O]) if O.size else np.zeros((W.shape[0], 0), np.uint16)
    WB = Wf.copy()
    WB[:, O] = 0.0
    if layout == "1x32":
        Wq, Ws = mxfp4.encode_rows(WB)
        Wst = None
    elif layout == "32x32":
        Wq, Ws, Wst = mxfp4.encode_tiles(WB)
    elif layout == "128x1":
        Wq, Ws, Wst = mxfp4.encode_stripes(WB, 128)
    else:
        raise ValueError(layout)
    return dict(Wq=Wq, Ws=Ws, Wst=Wst, WO=WO)


def plan(a: np.ndarray, w: np.ndarray, W: np.ndarray, alpha: float, k: int,
         layout: str = "1x32", smooth: bool = True, score: str = "max",
         rank: np.ndarray | None = None) -> dict:
    """Eq. (2) scales from the maxima a; Eq. (4) ranks a, or the per-channel
    statistic ``rank`` when given (e.g. act_percentile), raw or divided by s
    (``score``); then the fold and packing."""
    s, rcp = smooth_scales(a, w, alpha, smooth)
    O, pos = outlier_set(outlier_score(a if rank is None else rank, s, score), k)
    p = dict(s=s, rcp=rcp, O=O, pos=pos)
    p.update(fold_pack(W, s, O, layout))
    return p


# ----------------------------------------------------------------------------- forward

def quantize_act(X: np.ndarray, s: np.ndarray, O: np.ndarray) -> dict:
    """Runtime activation path: divide by s, route, quantize.

    q = RN_f32(x / s_j) (Reading: IEEE f32 division, no intermediate rounding);
    XO [M][k] = bf16(q[:, O]); the bulk q with the O columns set to +0 is
    MXFP4-encoded with 1x32 K-blocks -> Aq [M][K/2], As [M][K/32]."""
    x = as_f32(X)
    assert np.all(np.isfinite(x))
    q = (x / s[None, :].astype(np.float32)).astype(np.float32)
    XO = bf16_rne(q[:, O]) if O.size else np.zeros((x.shape[0], 0), np.uint16)
    q[:, O] = 0.0
    Aq, As = mxfp4.encode_rows(q)
    return dict(Aq=Aq, As=As, XO=XO)


def dual_gemm_f64(Aq, As, Wq, Ws, XO, WO) -> np.ndarray:
    """Eq. (5) (Eq. (3) with a static O): Y = X_J W^(q)_J + X_O W^(hp)_O.

    The bulk operands are decoded exactly to float64 with their block scales
    (Eq. (3)'s per-group scales); the outlier operands are the bf16 values.
    Every decoded value and product is exact in float64; the sums use float64
    matrix products.  Returns the unrounded float64 Y [M][N]."""
    Ad = mxfp4.decode_rows(Aq, As)
    Wd = mxfp4.decode_rows(Wq, Ws)
    Y = Ad @ Wd.T
    if XO.shape[1]:
        Y = Y + as_f32(XO).astype(np.float64) @ as_f32(WO).astype(np.float64).T
    return Y


def forward_f64(X, p: dict) -> np.ndarray:
    qa = quantize_act(X, p["s"], p["O"])
    return dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])


def gelu_tanh(y: np.ndarray) -> np.ndarray:
    """GELU with the tanh approximation, float64:
    0.5 y (1 + tanh(sqrt(2/pi) (y + 0.044715 y^3)))."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (y + 0.044715 * y ** 3)))


# ----------------------------------------------------------------------------- fidelity

def reference_f64(X, W) -> np.ndarray:
    """Unquantized layer output X W^T in float64."""
    return as_f32(X).astype(np.float64) @ as_f32(W).astype(np.float64).T


def rel_fro(Y: np.ndarray, Yref: np.ndarray) -> float:
    Y = np.asarray(Y, dtype=np.float64)
    return float(np.linalg.norm(Y - Yref) / np.linalg.norm(Yref))


def max_rel(Y: np.ndarray, Yref: np.ndarray) -> float:
    """max |Y - Yref| / max |Yref| (the output parity measure)."""
    Y = np.asarray(Y, dtype=np.float64)
    return float(np.abs(Y - Yref).max() / np.abs(Yref).max())
