"""GPU parity of per-step outlier routing by prediction.

- mg_quantize_act_stats equals mg_quantize_act plus mg_calib_act on the same
  input, bit for bit (bf16 and f32, ragged shapes, running over batches);
- DynamicRouter over a drifting batch sequence: at every step the operands
  and the output equal the oracle's plan whose Eq. (4) set is the top-k of the
  previous batch's maxima (the calibration maxima at the first step), with s
  from the calibration maxima throughout.
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from oracle import layer
from tests.gpu_util import aq_rows, check_output, dev, host, outlier_cols, scale_rows

pytestmark = pytest.mark.gpu

TOL = 2e-3


def _act_bits(a: mg.Act) -> dict:
    return {n: getattr(a, n).detach().contiguous().view(torch.uint8).clone() for n in ("Aq", "As", "XO")}


@pytest.mark.parametrize("M,K,k,bf16", [(1000, 1024, 40, True), (257, 96, 5, True), (33, 256, 0, True),
                                        (256, 512, 8, False)])
def test_quantize_stats_equals_quantize_and_calib(M, K, k, bf16):
    X = synth.heavy_tail_act(M, K, sigma=0.25, frac=0.03, mult=25.0, ch_seed=K + k, x_seed=K + k + 1, bf16=bf16)
    W = synth.weights(64, K, sigma=0.02, clip=0.6, seed=K, bf16=bf16)
    Xd, Wd = dev(X), dev(W)
    p = mg.plan(mg.calibrate([Xd], K), Wd, 0.6, k)
    a1, a2 = mg.Act.empty(p.desc, M), mg.Act.empty(p.desc, M)
    mg.mg_quantize_act(p, Xd, a1)
    stats = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_calib_reset(stats)
    mg.mg_quantize_act_stats(p, Xd, a2, stats)
    torch.cuda.synchronize()
    want = _act_bits(a1)
    for n, v in _act_bits(a2).items():
        assert torch.equal(v, want[n]), n
    assert torch.equal(stats, mg.calibrate([Xd], K))
    # running: a second batch accumulates like mg_calib_act does
    X2 = synth.heavy_tail_act(M // 2 + 1, K, sigma=0.5, frac=0.03, mult=25.0, ch_seed=K + 7, x_seed=K + 8, bf16=bf16)
    X2d = dev(X2)
    mg.mg_quantize_act_stats(p, X2d, mg.Act.empty(p.desc, X2.shape[0]), stats)
    assert torch.equal(stats, mg.calibrate([Xd, X2d], K))


@pytest.mark.parametrize("score", ["max", "smoothed"])
def test_dynamic_router_follows_previous_step(score):
    M, K, N, k, steps = 1500, 1024, 384, 32, 4
    batches = synth.drifting_act(M, K, steps + 1, sigma=0.25, frac=0.03, mult=25.0, drift=0.25,
                                 ch_seed=301, x_seed=310)
    W = synth.weights(N, K, sigma=0.02, clip=0.6, seed=320, bf16=True)
    Wd = dev(W)
    a_cal = layer.act_max(batches[0])                          # offline calibration batch
    w = layer.weight_range(W)
    router = mg.DynamicRouter(Wd, dev(a_cal), 0.6, k, score=score)
    prev = a_cal
    static_O = layer.plan(a_cal, w, W, 0.6, k, score=score)["O"]
    moved = 0
    for t in range(1, steps + 1):
        X = batches[t]
        print(f"\n[dynamic] step {t} ({score})", flush=True)
        Xd = dev(X)
        act = mg.Act.empty(router.desc, M)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        router.step(Xd, act, Y)
        torch.cuda.synchronize()
        op = layer.plan(a_cal, w, W, 0.6, k, score=score, rank=prev)
        oq = layer.quantize_act(X, op["s"], op["O"])
        got = dict(Aq=aq_rows(act.Aq, M, K), As=scale_rows(act.As, M, K), XO=outlier_cols(act.XO, M, k))
        for n in ("Aq", "As", "XO"):
            assert np.array_equal(np.asarray(got[n]).view(np.uint8), np.asarray(oq[n]).view(np.uint8)), (t, n)
        Y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
        used = router.plans[router.cur ^ 1]                   # the plan this step ran on
        mg.mg_dual_gemm(used, act, Y32)
        torch.cuda.synchronize()
        assert np.array_equal(host(used.O), op["O"]), t
        Y64 = layer.dual_gemm_f64(oq["Aq"], oq["As"], op["Wq"], op["Ws"], oq["XO"], op["WO"])
        check_output(host(Y), host(Y32), Y64, TOL)
        moved += int(not np.array_equal(op["O"], static_O))
        prev = layer.act_max(X)
    assert moved > 0                                           # the routed set did follow the drift
