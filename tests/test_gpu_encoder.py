"""The quantizer's MXFP4 encoding on every finite bf16 value (Eq. (5)'s 4-bit
bulk operand; E8M0 scale = floor(log2 amax) - 2, elements rounded to the
nearest E2M1 value, ties to the even code, saturating, sign kept).

The kernel encodes with the gfx950 converter (v_cvt_scalef32_pk_fp4_f32).  Here
every finite bf16 bit pattern -- both signs, all 255 exponent fields including
zero and the subnormals, all 128 mantissas -- is placed in 32-blocks whose
first element sets the block maximum 0 .. 6 binades above the value's own
binade, so each value is encoded at every position of the E2M1 grid relative
to its block scale (from the saturating top down to the codes that round to
zero).  The input goes through mg_quantize_act with

* s = 1 (the quotient is the bf16 value itself), and
* per-channel scales: those of the 480p up-projection's plan (alpha 0.6) and
  log-uniform draws over 1 .. 2^30, and over 2^-30 .. 1 on the values below
  2^98 (so that no quotient overflows) -- quotients with full f32 mantissas;
  rows whose values or scales leave the fast division range take the
  correctly rounded division --

and Aq / As are compared bit for bit with the oracle's threshold encoder,
which is pinned on the CPU against an exact brute-force nearest search.
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from oracle import layer
from tests.gpu_util import aq_rows, dev, scale_rows

pytestmark = pytest.mark.gpu
K = 512


def every_bf16_in_setter_blocks(emax: int = 254) -> np.ndarray:
    """[rows][512] bf16 bits: blocks [setter, 31 test values], for the biased
    exponent fields 0 .. emax (254: every finite value)."""
    blocks = []
    for sign in (0, 1):
        for E in range(emax + 1):
            vals = (sign << 15) | (E << 7) | np.arange(128, dtype=np.uint16)
            chunks = [vals[i:i + 31] for i in range(0, 128, 31)]
            chunks[-1] = np.resize(chunks[-1], 31)
            for d in range(7):
                if E + d > emax:
                    continue
                setter = np.uint16(((E + d) << 7) | (0 if d else 127))   # d = 0: the binade's largest value
                for c in chunks:
                    blocks.append(np.concatenate([[setter], c]).astype(np.uint16))
    b = np.stack(blocks)
    rows = -(-b.shape[0] // (K // 32))
    pad = rows * (K // 32) - b.shape[0]
    b = np.concatenate([b, np.zeros((pad, 32), np.uint16)])
    X = b.reshape(rows, K)
    finite = (X & 0x7F80) != 0x7F80
    assert finite.all()
    return X


def _run(Xd, X, s: np.ndarray):
    desc = mg.make_desc(K, 32, 0, 0.5, "1x32", smooth=False)
    p = mg.Plan.empty(desc)
    s = s.astype(np.float32)
    rcp = (np.float32(1.0) / s).astype(np.float32)
    p.s.copy_(torch.from_numpy(s))
    p.rcp.copy_(torch.from_numpy(rcp))
    p.pos.fill_(-1)
    a = mg.Act.empty(desc, X.shape[0])
    mg.mg_quantize_act(p, Xd, a)
    torch.cuda.synchronize()
    o = layer.quantize_act(X, s, np.zeros(0, np.int32))
    Aq, As = aq_rows(a.Aq, X.shape[0], K), scale_rows(a.As, X.shape[0], K)
    for name, g_, o_ in (("Aq", Aq, o["Aq"]), ("As", As, o["As"])):
        if not np.array_equal(g_, o_):
            bad = np.argwhere(g_ != o_)
            raise AssertionError(f"{name} differs at {bad[:5].tolist()} ({len(bad)} places)")
    return Aq


def test_every_bf16_at_unit_scale():
    X = every_bf16_in_setter_blocks()
    print(f"\n[encoder] {X.shape[0]} rows x {K}, s = 1", flush=True)
    Aq = _run(dev(X), X, np.ones(K, np.float32))
    nib = np.stack([Aq & 15, Aq >> 4], axis=-1)
    assert set(np.unique(nib).tolist()) == set(range(16))      # every code, both signs, occurs


def test_every_bf16_at_plan_and_random_scales():
    X = every_bf16_in_setter_blocks()
    Xd = dev(X)
    w = synth.FFN0_480P
    s_plan = layer.smooth_scales(layer.act_max(w.make_x()), layer.weight_range(w.make_w()), w.alpha)[0]
    g = np.random.default_rng(5150)
    sets = [s_plan[i:i + K] for i in range(0, w.K, K)]
    sets += [np.exp2(g.uniform(0.0, 30.0, K)).astype(np.float32) for _ in range(3)]
    for i, s in enumerate(sets):
        print(f"[encoder] scale set {i}: s in [{s.min():.3g}, {s.max():.3g}]", flush=True)
        _run(Xd, X, s)
    Xs = every_bf16_in_setter_blocks(emax=127 + 97)
    Xsd = dev(Xs)
    for i in range(3):
        s = np.exp2(g.uniform(-30.0, 0.0, K)).astype(np.float32)
        print(f"[encoder] small scale set {i}: s in [{s.min():.3g}, {s.max():.3g}]", flush=True)
        _run(Xsd, Xs, s)


def test_large_quotients_take_the_exact_division():
    """Quotients of 2^126 and more: every finite bf16 below 2^127 under
    scales in [0.5, 1) (quotients up to just below 2^128, all finite).  The
    kernel's fast division is used only while |x * RN(1/s)| < 2^126, so the
    rows holding these values go through the correctly rounded division; Aq /
    As must still be the oracle's bit for bit."""
    X = every_bf16_in_setter_blocks(emax=253)
    Xd = dev(X)
    g = np.random.default_rng(4242)
    for i in range(2):
        s = g.uniform(0.5, 1.0, K).astype(np.float32)
        q = np.abs(layer.as_f32(X).astype(np.float64)) / s.astype(np.float64)[None, :]
        assert q.max() >= 2.0 ** 126 and np.isfinite(q.astype(np.float32)).all()
        print(f"[encoder] large-quotient set {i}: s in [{s.min():.3g}, {s.max():.3g}]", flush=True)
        _run(Xd, X, s)
