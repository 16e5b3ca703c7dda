"""GPU parity at the full workload sizes (the launch configuration the
benchmark times).

Per-channel statistics, s, rcp, O, pos and the packed weights (Wq, Ws, Wst,
WO) are compared in full, bit-exactly, and so are the activation codes (Aq,
As, XO) of every row (the oracle quantizes the rows in chunks on a thread
pool; the weight-layout variants, whose activation path is the same, compare
sampled rows).  The output is compared on sampled rows: the GEMM's fp32 result
within max|Y32 - Y64| / max|Y64| <= 2e-3 of the float64 oracle, the bf16
output exactly its round-to-nearest-even.  The sampled rows always include the
first row and the rows of the last (ragged) row tile.
"""
import concurrent.futures as cf
import dataclasses
import os

import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from oracle import layer
from tests.gpu_util import aq_rows, check_output, dev, host, outlier_cols, scale_rows

pytestmark = pytest.mark.gpu

SAMPLE = 48
CHUNK = 2048
THREADS = min(8, len(os.sched_getaffinity(0)))


def _rows(M, seed):
    g = np.random.default_rng(seed)
    tail = np.arange(max(0, (M - 1) // 256 * 256), M)
    rows = np.unique(np.concatenate([[0, 1], g.choice(M, SAMPLE, replace=False), tail[-16:]]))
    return rows


def _bits_equal(a, b, name):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (name, a.shape, b.shape)
    if a.dtype.kind == "f":
        ok = np.array_equal(a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32))
    else:
        ok = np.array_equal(a.astype(np.int64), b.astype(np.int64))
    if not ok:
        bad = np.argwhere(a != b)
        raise AssertionError(f"{name} differs at {bad[:5].tolist()} ({len(bad)} places)")


def _codes_all_rows(X, op, g, M, K, k):
    """Aq, As, XO of every row against the oracle, chunk by chunk."""
    def check(r0):
        r1 = min(M, r0 + CHUNK)
        oq = layer.quantize_act(X[r0:r1], op["s"], op["O"])
        _bits_equal(g["Aq"][r0:r1], oq["Aq"], f"Aq rows {r0}..{r1}")
        _bits_equal(g["As"][r0:r1], oq["As"], f"As rows {r0}..{r1}")
        _bits_equal(g["XO"][r0:r1], oq["XO"], f"XO rows {r0}..{r1}")
        return r1 - r0
    with cf.ThreadPoolExecutor(THREADS) as ex:
        assert sum(ex.map(check, range(0, M, CHUNK))) == M


def _run_full(w: synth.Workload, layout="1x32", score="max", all_rows=True):
    print(f"\n[full-size] {w.name} layout={layout} score={score} k={w.k} alpha={w.alpha} all_rows={all_rows}",
          flush=True)
    X, W = w.make_x(), w.make_w()
    M, K, N = X.shape[0], X.shape[1], W.shape[0]
    Xd, Wd = dev(X), dev(W)
    act_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_calib_reset(act_max)
    mg.mg_calib_act(Xd, act_max)
    w_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_weight_range(Wd, w_max)
    desc = mg.make_desc(K, N, w.k, w.alpha, layout, True, score)
    p = mg.Plan.empty(desc)
    mg.mg_plan_build(p, act_max, w_max, Wd)
    a = mg.Act.empty(desc, M)
    mg.mg_quantize_act(p, Xd, a)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.mg_dual_gemm(p, a, Y)
    rows = _rows(M, 7)
    ridx = torch.from_numpy(rows).cuda()
    Y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mg.mg_dual_gemm(p, a, Y32)
    torch.cuda.synchronize()
    g = dict(act_max=host(act_max), w_max=host(w_max), Y=host(Y[ridx]), Y32=host(Y32[ridx]))
    if all_rows:
        g.update(Aq=aq_rows(a.Aq, M, K), As=scale_rows(a.As, M, K), XO=outlier_cols(a.XO, M, w.k))
    else:
        g.update(Aq=aq_rows(a.Aq, M, K)[rows], As=scale_rows(a.As, M, K)[rows], XO=outlier_cols(a.XO, M, w.k)[rows])
    g.update({n: host(t) for n, t in p.tensors().items()})
    g["Ws"] = scale_rows(p.Ws, N, K)
    g["Wq"] = aq_rows(p.Wq, N, K)
    g["WO"] = outlier_cols(p.WO, N, w.k)
    del Y, Y32, a, Xd, Wd
    torch.cuda.empty_cache()

    # oracle: plan on the full data, codes on every (or the sampled) rows, output on the sampled rows
    o_a = layer.act_max(X)
    o_w = layer.weight_range(W)
    op = layer.plan(o_a, o_w, W, w.alpha, w.k, layout, True, score)
    _bits_equal(g["act_max"], o_a, "act_max")
    _bits_equal(g["w_max"], o_w, "w_max")
    for name in ("s", "rcp", "O", "pos", "Wq", "Ws", "WO"):
        _bits_equal(g[name], op[name], name)
    if layout != "1x32":
        _bits_equal(g["Wst"], op["Wst"], "Wst")
    oq = layer.quantize_act(X[rows], op["s"], op["O"])
    if all_rows:
        _codes_all_rows(X, op, g, M, K, w.k)
        print(f"[full-size] {w.name}: Aq, As, XO equal on all {M} rows", flush=True)
    else:
        for name in ("Aq", "As", "XO"):
            _bits_equal(g[name], oq[name], name)
    Y64 = layer.dual_gemm_f64(oq["Aq"], oq["As"], op["Wq"], op["Ws"], oq["XO"], op["WO"])
    err = check_output(g["Y"], g["Y32"], Y64)
    print(f"[full-size] {w.name}: max|dY32|/max|Y| = {err:.3e} on {rows.size} rows", flush=True)


def test_ffn0_480p():
    _run_full(synth.FFN0_480P)


def test_ffn2_480p():
    _run_full(synth.FFN2_480P)


def test_ffn0_720p_k128_alpha07():
    _run_full(dataclasses.replace(synth.FFN0_720P, k=128, alpha=0.7))


def test_ffn0_480p_tile_scales():
    _run_full(synth.FFN0_480P, layout="32x32", all_rows=False)


def test_ffn0_480p_stripe_scales():
    _run_full(synth.FFN0_480P, layout="128x1", all_rows=False)


def test_ffn2_480p_smoothed_score():
    _run_full(synth.FFN2_480P, score="smoothed")
