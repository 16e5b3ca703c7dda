"""GPU parity: every stage of the HIP path against the CPU oracle on the same
seeded inputs, at sizes the oracle finishes in seconds that still span several
tiles and ragged tails.

Bar: calibration maxima, s, rcp, O, pos, Wq, Ws, Wst, WO, Aq, As, XO
bit-exact; the GEMM's fp32 result within max|Y_gpu - Y64| / max|Y64| <= 2e-3
of the unrounded float64 oracle output, and the bf16 output exactly that
result rounded to nearest-even.  (A bf16 output alone cannot meet 2e-3 in this
norm: bf16 has 8 significant bits, so one rounding may move a value by up to
2^-8 = 3.9e-3 of itself.)
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from oracle import layer
from tests.gpu_util import aq_rows, assert_faithful_bf16, bf16_to_f64, check_output, dev, host, outlier_cols, run_pipeline, scale_rows

pytestmark = pytest.mark.gpu
TOL = 2e-3


def _oracle(X, W, alpha, k, layout="1x32", smooth=True, score="max"):
    a = layer.act_max(X)
    w = layer.weight_range(W)
    p = layer.plan(a, w, W, alpha, k, layout, smooth, score)
    qa = layer.quantize_act(X, p["s"], p["O"])
    Y64 = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    return dict(act_max=a, w_max=w, Y64=Y64, **p, **qa)


def _compare(g, o, layout="1x32"):
    for name in ("act_max", "w_max", "s", "rcp", "O", "pos", "Wq", "Ws", "WO", "Aq", "As", "XO"):
        gv, ov = np.asarray(g[name]), np.asarray(o[name])
        assert gv.shape == ov.shape, (name, gv.shape, ov.shape)
        if gv.dtype.kind == "f":
            same = np.array_equal(gv.view(np.uint32), ov.view(np.uint32))
        else:
            same = np.array_equal(gv.astype(np.int64), ov.astype(np.int64))
        if not same:
            bad = np.argwhere(gv != ov)
            raise AssertionError(f"{name} differs at {bad[:5].tolist()} ({len(bad)} places)")
    if layout != "1x32":
        assert np.array_equal(g["Wst"], o["Wst"])
    return check_output(g["Y"], g["Y32"], o["Y64"], TOL)


def _heavy(M, K, N, seed, frac=0.02, bf16=True):
    X = synth.heavy_tail_act(M, K, sigma=0.25, frac=frac, mult=25.0, ch_seed=seed, x_seed=seed + 1, bf16=bf16)
    W = synth.weights(N, K, sigma=0.02, clip=0.6, seed=seed + 2, bf16=bf16)
    return X, W


def test_tiny_workload_all_stages():
    w = synth.TINY
    X, W = w.make_x(), w.make_w()
    g = run_pipeline(X, W, w.alpha, w.k)
    _compare(g, _oracle(X, W, w.alpha, w.k))


@pytest.mark.parametrize("M,K,N,k", [(257, 512, 192, 16), (1000, 1024, 320, 64), (64, 96, 64, 5),
                                     (33, 256, 96, 0), (130, 128, 64, 128), (4095, 640, 256, 40),
                                     (300, 768, 256, 24), (200, 384, 128, 6), (300, 512, 192, 70),
                                     (1, 32, 32, 0), (5, 32, 32, 1), (513, 1056, 288, 16),
                                     (100, 1568, 64, 31), (64, 4128, 96, 130)])
def test_bf16_shapes(M, K, N, k):
    """Shapes across the GEMM's code paths: scale windows whole (K % 512 == 0)
    or with a partial last window (K = 768 also has an odd number of 256-deep
    stages, so the last window's second half is all pad; K = 4128 ends in a
    window of one block; K = 32 is one block in one stage), M and N not
    multiples of the 256x256 tile (M = 1 included), and every k: the outlier
    rows are padded to a multiple of 8 values, so k % 8 != 0 leaves pad columns
    inside the last 16-byte chunk, and k = 70 and 130 span two and three
    outlier stages, the last one partial."""
    X, W = _heavy(M, K, N, 1000 + M)
    g = run_pipeline(X, W, 0.6, k)
    _compare(g, _oracle(X, W, 0.6, k))


@pytest.mark.parametrize("layout", ["1x32", "32x32", "128x1"])
def test_dead_channels(layout):
    """Eq. (2) at the floor of its statistics (reading: 1e-5 on both before the
    powers): all-zero activation channels (as after a gate), all-zero weight
    columns, one channel zero in both; with k = 24 the dead activation
    channels stay in the bulk, with k = K - 3 all but three channels, the dead
    ones included, go to the outlier branch.  Every artefact is bit-exact,
    including s on the dead channels.  Then an all-zero batch through a plan
    whose statistics are all zero but one weight column: every code is the
    zero code and the output is zero."""
    M, K, N = 300, 512, 192
    X, W = _heavy(M, K, N, 4242)
    X[:, [3, 40, 41, 200]] = 0
    W[:, [17, 40, 333]] = 0
    for k in ((24, K - 3) if layout == "1x32" else (24,)):
        o = _oracle(X, W, 0.6, k, layout)
        assert all(o["act_max"][j] == 0 for j in (3, 40, 200)) and all(o["w_max"][j] == 0 for j in (17, 40, 333))
        assert (3 in o["O"]) == (k == K - 3)
        g = run_pipeline(X, W, 0.6, k, layout)
        _compare(g, o, layout)
    Z = np.zeros((40, 96), np.uint16)
    WZ = np.zeros((64, 96), np.uint16)
    WZ[:, 5] = synth.f32_to_bf16_bits(np.full(64, 0.25, np.float32))
    g = run_pipeline(Z, WZ, 0.5, 4, layout)
    o = _oracle(Z, WZ, 0.5, 4, layout)
    for name in ("act_max", "w_max", "s", "rcp", "O", "pos", "Wq", "Ws", "WO", "Aq", "As", "XO"):
        assert np.array_equal(np.asarray(g[name]).view(np.uint8), np.asarray(o[name]).view(np.uint8)), name
    assert not np.asarray(g["Aq"]).any() and not np.asarray(g["As"]).any()
    assert not np.abs(g["Y32"]).any() and not (np.asarray(g["Y"]) & 0x7FFF).any()


@pytest.mark.parametrize("M,K,N,k", [(48, 16416, 64, 40), (24, 32768, 32, 64), (16, 65536, 32, 128),
                                     (9, 40000, 64, 7)])
def test_large_K(M, K, N, k):
    """Input widths past 8192 and 16384 channels, where the top-k kernel holds
    17-32 and 33-64 scores per thread (its two larger instantiations), up to
    the header's limit K = 65536; the GEMM then walks 64-256 bulk stages."""
    X, W = _heavy(M, K, N, 5000 + K)
    X[:, 7] = X[:, 8]                           # a tie between two channels' maxima
    g = run_pipeline(X, W, 0.6, k)
    _compare(g, _oracle(X, W, 0.6, k))


@pytest.mark.parametrize("M,K,N,k", [(4096, 128, 8192, 0), (4096, 640, 8192, 0), (4096, 32, 8192, 0),
                                     (4096, 96, 8192, 3), (2304, 1056, 8192, 40)])
def test_many_tiles_per_workgroup(M, K, N, k):
    """More 256x256 tiles than compute units (512 or 288 tiles), so each
    workgroup walks several tiles and the copy pipeline and the scale windows
    run across tile boundaries: tiles of one half-stage (K <= 128, the copies
    two tiles ahead), a tile ending one half-stage into its second scale
    window (K = 640, k = 0), a half-filled last K-slice (K = 32, 96) and
    outlier half-stages after the bulk ones."""
    X, W = _heavy(M, K, N, 7000 + K)
    g = run_pipeline(X, W, 0.6, k)
    _compare(g, _oracle(X, W, 0.6, k))


@pytest.mark.parametrize("layout", ["1x32", "32x32", "128x1"])
def test_layouts(layout):
    X, W = _heavy(300, 512, 256, 77)
    W[5, 100] = 0.59                         # a local weight outlier inside one tile
    g = run_pipeline(X, W, 0.5, 12, layout)
    _compare(g, _oracle(X, W, 0.5, 12, layout), layout)


@pytest.mark.parametrize("M,K,N,k", [(300, 352, 96, 12), (70, 96, 64, 3)])
def test_stripes_ragged_K(M, K, N, k):
    """128x1 stripes when K is not a multiple of 128 (a short last stripe)."""
    X, W = _heavy(M, K, N, 40 + K)
    g = run_pipeline(X, W, 0.6, k, "128x1")
    _compare(g, _oracle(X, W, 0.6, k, "128x1"), "128x1")


@pytest.mark.parametrize("layout", ["1x32", "128x1"])
def test_smoothed_score(layout):
    """Eq. (4) ranking the smoothed maxima RN(a_j / s_j): a different outlier
    set than the raw score on this input (checked), bit-exact to the oracle."""
    X, W = _heavy(400, 512, 128, 91)
    W[:, 7] = synth.f32_to_bf16_bits(np.full(128, 0.55, np.float32))     # a wide weight column
    g = run_pipeline(X, W, 0.5, 16, layout, score="smoothed")
    o = _oracle(X, W, 0.5, 16, layout, score="smoothed")
    _compare(g, o, layout)
    assert not np.array_equal(o["O"], _oracle(X, W, 0.5, 16, layout)["O"])


@pytest.mark.parametrize("layout", ["1x32", "32x32", "128x1"])
@pytest.mark.parametrize("M,K,N,k,bf16", [(300, 352, 96, 6, True), (600, 800, 288, 12, False)])
def test_scale_pads_written_over_garbage(M, K, N, k, bf16, layout):
    """Ragged M, N and K (not multiples of 256, 256 and 512; K % 64 == 32, so
    the last 32-byte slice of an Aq / Wq row is half pad) and k not a
    multiple of 16: over scale buffers pre-filled with 0xFF (the E8M0 NaN
    code), payload buffers pre-filled with 0xFF and outlier buffers with bf16
    NaNs, the writers fill every pad row and pad block of the scale windows
    with code 0, every fragment-order pad of Aq / Wq (rows up to a multiple of
    32, the half slice) with zero codes and every pad of XO / WO with +0
    (checked by scale_rows, aq_rows and outlier_cols), the codes equal the
    oracle's, and the output is exact."""
    X, W = _heavy(M, K, N, 70 + K, bf16=bf16)
    Xd, Wd = dev(X), dev(W)
    act_max = mg.calibrate([Xd], K)
    w_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_weight_range(Wd, w_max)
    desc = mg.make_desc(K, N, k, 0.6, layout)
    p = mg.Plan.empty(desc)
    p.Ws.fill_(0xFF)
    p.WO.fill_(0xFF)                         # bf16 NaNs
    p.Wq.fill_(0xFF)
    mg.mg_plan_build(p, act_max, w_max, Wd)
    a = mg.Act.empty(desc, M)
    a.As.fill_(0xFF)
    a.XO.fill_(0xFF)
    a.Aq.fill_(0xFF)
    mg.mg_quantize_act(p, Xd, a)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mg.mg_dual_gemm(p, a, Y)
    mg.mg_dual_gemm(p, a, Y32)
    torch.cuda.synchronize()
    o = _oracle(X, W, 0.6, k, layout)
    assert np.array_equal(scale_rows(p.Ws, N, K), o["Ws"])
    assert np.array_equal(scale_rows(a.As, M, K), o["As"])
    assert np.array_equal(aq_rows(a.Aq, M, K), o["Aq"]) and np.array_equal(aq_rows(p.Wq, N, K), o["Wq"])
    assert np.array_equal(outlier_cols(a.XO, M, k), o["XO"]) and np.array_equal(outlier_cols(p.WO, N, k), o["WO"])
    check_output(host(Y), host(Y32), o["Y64"])


def test_smoothing_off():
    X, W = _heavy(200, 256, 128, 88)
    g = run_pipeline(X, W, 0.5, 8, smooth=False)
    o = _oracle(X, W, 0.5, 8, smooth=False)
    _compare(g, o)
    assert np.all(g["s"] == 1.0)


def test_calibration_batches_and_ties():
    """Running maxima over uneven batches; many tied scores for the top-k."""
    X, W = _heavy(999, 512, 64, 5)
    # force ties at the top: 20 channels share the largest maximum
    ch = np.arange(0, 400, 20)
    X[3, ch] = synth.f32_to_bf16_bits(np.full(ch.size, 40.0, np.float32))
    g = run_pipeline(X, W, 0.6, 9, calib_batches=7)
    _compare(g, _oracle(X, W, 0.6, 9))


def test_k_equals_K_is_bf16_gemm():
    X, W = _heavy(128, 128, 96, 9)
    g = run_pipeline(X, W, 0.5, 128, smooth=False)
    ref = bf16_to_f64(X) @ bf16_to_f64(W).T
    check_output(g["Y"], g["Y32"], ref, TOL)
    assert np.all(g["Aq"] == 0) and np.all(g["Wq"] == 0)


@pytest.mark.parametrize("k", [64, 256])
def test_division_outside_the_fast_range(k):
    """Values and scales outside the range where x * RN(1/s) with one FMA
    correction is exact take the correctly rounded division, bit for bit with
    the oracle: activation channels 2^100 larger (s > 2^20, outliers) and
    2^110 smaller, weight columns 2^100 larger (s < 2^-20), scattered entries
    scaled by 2^-128 (bf16 subnormals) and signed zeros; k = 64 and k = K put
    several outlier channels in many lanes (their further channels have their
    own path)."""
    M, K, N = 300, 256, 64
    X, W = _heavy(M, K, N, 77)
    g = np.random.default_rng(5)
    Xf, Wf = bf16_to_f64(X), bf16_to_f64(W)
    ch = g.permutation(K)
    Xf[:, ch[:6]] *= 2.0 ** 100
    Xf[:, ch[6:12]] *= 2.0 ** -110
    Wf[:, ch[12:18]] *= 2.0 ** 100
    Xf[g.random((M, K)) < 0.01] *= 2.0 ** -128
    zero = g.random((M, K)) < 0.005
    Xf[zero] = np.where(g.random(int(zero.sum())) < 0.5, 0.0, -0.0)
    X = synth.f32_to_bf16_bits(Xf.astype(np.float32))
    W = synth.f32_to_bf16_bits(Wf.astype(np.float32))
    xa = np.abs(bf16_to_f64(X))
    assert np.any((xa > 0) & (xa < 2.0 ** -126))
    o = _oracle(X, W, 0.6, k)
    assert np.any(o["s"] > 2.0 ** 20) and np.any(o["s"] < 2.0 ** -20)
    _compare(run_pipeline(X, W, 0.6, k), o)


def test_sign_symmetry_and_determinism():
    X, W = _heavy(257, 512, 128, 11)
    g1 = run_pipeline(X, W, 0.6, 16)
    g2 = run_pipeline(X, W, 0.6, 16)
    assert np.array_equal(g1["Y"], g2["Y"]) and np.array_equal(g1["Y32"], g2["Y32"])
    Xn = X ^ np.uint16(0x8000)
    gn = run_pipeline(Xn, W, 0.6, 16)
    y, yn = bf16_to_f64(g1["Y"]), bf16_to_f64(gn["Y"])
    assert np.array_equal(yn, -y)


def test_gelu_tanh():
    """Every bf16 bit pattern (plus a ragged tail): faithful bf16 rounding of the
    float64 GELU where that is at least 2^-24 in magnitude, +inf -> +inf, and
    NaN for NaN and -inf inputs (0.5 y (1 + tanh u) is -inf * 0 there)."""
    y = np.arange(65536 + 5, dtype=np.uint32).astype(np.uint16)
    yd = dev(y)
    out = torch.empty_like(yd)
    mg.mg_gelu_tanh_bf16(yd, out)
    torch.cuda.synchronize()
    with np.errstate(over="ignore", invalid="ignore"):
        h = bf16_to_f64(host(out))
        yf = bf16_to_f64(y)
        ref = layer.gelu_tanh(yf)
    fin = np.isfinite(yf)
    assert_faithful_bf16(h[fin], ref[fin])
    assert np.all(h[yf == np.inf] == np.inf)
    assert np.all(np.isnan(h[np.isnan(yf) | (yf == -np.inf)]))


@pytest.mark.parametrize("M,K,k", [(300, 512, 12), (77, 96, 5), (1000, 1024, 0)])
def test_gelu_quantize_fused(M, K, k):
    """GELU + quantize in one pass equals the GELU kernel followed by the
    quantizer, bit for bit, and both equal the oracle's quantization of the
    GPU's h (GELU rounding is the GPU's own: the oracle consumes its h)."""
    g = np.random.default_rng(M + K)
    y = (g.standard_normal((M, K)) * 1.5).astype(np.float32)
    y[:, g.choice(K, max(1, K // 50), replace=False)] *= 12.0
    Y = synth.f32_to_bf16_bits(y)
    Yd = dev(Y)
    h = torch.empty_like(Yd)
    mg.mg_gelu_tanh_bf16(Yd, h)
    act_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_calib_reset(act_max)
    mg.mg_calib_act(h, act_max)
    W = synth.weights(64, K, sigma=0.01, clip=None, seed=K, bf16=True)
    p = mg.plan(act_max, dev(W), 0.5, k)
    a1, a2 = mg.Act.empty(p.desc, M), mg.Act.empty(p.desc, M)
    mg.mg_quantize_act(p, h, a1)
    mg.mg_gelu_quantize_act(p, Yd, a2)
    torch.cuda.synchronize()
    for n in ("Aq", "As", "XO"):
        assert torch.equal(getattr(a1, n).view(torch.uint8), getattr(a2, n).view(torch.uint8)), n
    oq = layer.quantize_act(host(h), host(p.s), host(p.O))
    got = dict(Aq=aq_rows(a2.Aq, M, K), As=scale_rows(a2.As, M, K), XO=outlier_cols(a2.XO, M, k))
    for n in ("Aq", "As", "XO"):
        assert np.array_equal(np.asarray(got[n]).view(np.uint8), np.asarray(oq[n]).view(np.uint8)), n


def test_empty_inputs_are_noops():
    desc = mg.make_desc(64, 32, 4, 0.5)
    p = mg.Plan.empty(desc)
    a = mg.Act.empty(desc, 0)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    act_max = torch.zeros(64, dtype=torch.float32, device="cuda")
    mg.mg_calib_act(X, act_max)
    mg.mg_quantize_act(p, X, a)
    torch.cuda.synchronize()
    assert torch.all(act_max == 0)


def test_helpers_on_a_side_stream():
    """The binding's allocating helpers run on an explicit stream (a torch
    stream, or a raw hipStream_t handle) with their temporaries allocated on
    that stream, bit for bit the default stream's results."""
    M, K, N, k = 600, 512, 256, 12
    X, W = _heavy(M, K, N, 505)
    Xd, Wd = dev(X), dev(W)
    act = mg.calibrate([Xd], K)
    ref_p = mg.plan(act, Wd, 0.6, k)
    ref_y = mg.forward(ref_p, Xd)
    W2d = dev(synth.weights(K, N, sigma=0.02, clip=0.6, seed=506, bf16=True))       # [512][256]: 256 -> 512
    act2 = mg.calibrate([torch.relu(ref_y.float()).to(torch.bfloat16)], N)
    blk = mg.ffn_block_plans(act, act2, Wd, W2d, 0.6, k, 0.5, 8)
    ref_b = mg.ffn_block_forward(blk, Xd)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    for st in (side, side.cuda_stream):
        a = mg.calibrate([Xd], K, stream=st)
        p = mg.plan(a, Wd, 0.6, k, stream=st)
        y = mg.forward(p, Xd, stream=st)
        b = mg.ffn_block_forward(blk, Xd, stream=st)
        side.synchronize()
        assert torch.equal(a, act)
        assert torch.equal(p.Wq, ref_p.Wq) and torch.equal(p.Ws, ref_p.Ws) and torch.equal(p.O, ref_p.O)
        assert torch.equal(y.view(torch.int16), ref_y.view(torch.int16))
        assert torch.equal(b.view(torch.int16), ref_b.view(torch.int16))


def test_plan_saved_and_loaded(tmp_path):
    """A plan is plain data: torch.save of Plan.state(), torch.load with
    weights_only=True and Plan.from_state() give the same forward, bit for bit."""
    M, K, N, k = 300, 544, 96, 10
    X, W = _heavy(M, K, N, 611)
    Xd, Wd = dev(X), dev(W)
    for layout in ("1x32", "32x32", "128x1"):
        p = mg.plan(mg.calibrate([Xd], K), Wd, 0.6, k, layout)
        y = mg.forward(p, Xd)
        path = tmp_path / f"plan_{layout}.pt"
        torch.save(p.state(), path)
        q = mg.Plan.from_state(torch.load(path, weights_only=True))
        assert torch.equal(mg.forward(q, Xd).view(torch.int16), y.view(torch.int16)), layout
