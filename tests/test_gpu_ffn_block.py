"""GPU parity of the full FFN block at 720p: ffn.0 (5120 -> 13824) -> GELU-tanh ->
ffn.2 (13824 -> 5120), 75600 tokens, calibrated on four batches and evaluated
on a fifth, with 1x32, 32x32 and 128x1 weight scales.

Stage-wise parity:
- ffn.0's calibration maxima equal the oracle's running maxima over the four
  batches, bit for bit;
- ffn.2's calibration maxima equal the oracle's running maxima over the
  hidden activations the GPU produced for those batches (the unquantized
  block's h; the oracle consumes the GPU's h because GELU and GEMM rounding
  may differ by an ulp);
- both plans equal the oracle's plans built from those maxima, bit for bit;
- on sampled rows of the evaluation batch: ffn.0's activation codes bit for
  bit and its output within 2e-3 (fp32) / one RNE (bf16); the GELU within one
  bf16 rounding of the float64 GELU of the GPU's ffn.0 output; ffn.2's codes
  (from the GPU's h) bit for bit and its output within 2e-3 / one RNE;
- the fused GELU + quantize pass from ffn.0's output, and the same work in
  ffn.0's GEMM epilogue (mg_dual_gemm_gelu_quant), give ffn.2's codes bit for
  bit, on every row.
The block's fidelity against the unquantized float64 block is printed, not
asserted.
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from oracle import layer
from tests.gpu_util import aq_rows, assert_faithful_bf16, bf16_to_f64, check_output, dev, host, outlier_cols, scale_rows

pytestmark = pytest.mark.gpu

CHUNK = 8192
SAMPLE = 40


def _rows(M, seed):
    g = np.random.default_rng(seed)
    tail = np.arange(max(0, (M - 1) // 256 * 256), M)
    return np.unique(np.concatenate([[0], g.choice(M, SAMPLE, replace=False), tail[-8:]]))


def _bits_equal(a, b, name):
    a, b = np.asarray(a), np.asarray(b)
    assert a.shape == b.shape, (name, a.shape, b.shape)
    if a.dtype.kind == "f":
        ok = np.array_equal(a.view(np.uint32), np.asarray(b, np.float32).view(np.uint32))
    else:
        ok = np.array_equal(a.astype(np.int64), b.astype(np.int64))
    assert ok, f"{name} differs in {int(np.sum(a != b))} places"


@pytest.fixture(scope="module")
def block():
    w0, w2, M = synth.BLOCK_FFN0, synth.BLOCK_FFN2, synth.BLOCK_M
    print(f"\n[ffn-block] generating W0, W2 and {len(synth.BLOCK_CALIB_SEEDS)} calibration batches", flush=True)
    W0, W2 = w0.make_w(), w2.make_w()
    W0d, W2d = dev(W0), dev(W2)
    o_act0 = None
    Xd = []
    for seed in synth.BLOCK_CALIB_SEEDS:
        X = w0.make_x(M=M, x_seed=seed)
        o_act0 = layer.act_max(X, o_act0)
        Xd.append(dev(X))
        del X
    o_act2 = [None]

    def on_hidden(h):
        hh = host(h)
        for r0 in range(0, hh.shape[0], CHUNK):
            o_act2[0] = layer.act_max(hh[r0:r0 + CHUNK], o_act2[0])

    act0, act2 = mg.ffn_block_stats(Xd, W0d, on_hidden=on_hidden)
    torch.cuda.synchronize()
    del Xd
    torch.cuda.empty_cache()
    return dict(W0=W0, W2=W2, W0d=W0d, W2d=W2d, act0=act0, act2=act2, o_act0=o_act0, o_act2=o_act2[0],
                X5=w0.make_x(M=M, x_seed=synth.BLOCK_EVAL_SEED))


def test_block_calibration(block):
    _bits_equal(host(block["act0"]), block["o_act0"], "act_max ffn.0")
    _bits_equal(host(block["act2"]), block["o_act2"], "act_max ffn.2 (over the GPU's h)")


@pytest.mark.parametrize("layout", ["1x32", "32x32", "128x1"])
def test_block_stagewise(block, layout):
    w0, w2 = synth.BLOCK_FFN0, synth.BLOCK_FFN2
    print(f"\n[ffn-block] layout {layout}: plans", flush=True)
    blk = mg.ffn_block_plans(block["act0"], block["act2"], block["W0d"], block["W2d"],
                             w0.alpha, w0.k, w2.alpha, w2.k, layout)
    o_p0 = layer.plan(block["o_act0"], layer.weight_range(block["W0"]), block["W0"], w0.alpha, w0.k, layout)
    o_p2 = layer.plan(block["o_act2"], layer.weight_range(block["W2"]), block["W2"], w2.alpha, w2.k, layout)
    for tag, p, op in (("ffn.0", blk.plan0, o_p0), ("ffn.2", blk.plan2, o_p2)):
        g = {n: host(t) for n, t in p.tensors().items()}
        g["Wq"] = aq_rows(p.Wq, p.desc.N, p.desc.K)
        g["Ws"] = scale_rows(p.Ws, p.desc.N, p.desc.K)
        g["WO"] = outlier_cols(p.WO, p.desc.N, p.desc.k)
        for name in ("s", "rcp", "O", "pos", "Wq", "Ws", "WO") + (("Wst",) if layout != "1x32" else ()):
            _bits_equal(g[name], op[name], f"{tag} {name}")

    print(f"[ffn-block] layout {layout}: evaluation batch", flush=True)
    X5 = block["X5"]
    M = X5.shape[0]
    X5d = dev(X5)
    a0 = mg.Act.empty(blk.plan0.desc, M)
    mg.mg_quantize_act(blk.plan0, X5d, a0)
    Y0 = torch.empty((M, w0.N), dtype=torch.bfloat16, device="cuda")
    mg.mg_dual_gemm(blk.plan0, a0, Y0)
    rows = _rows(M, 11)
    ridx = torch.from_numpy(rows).cuda()
    Y0_32 = torch.empty((M, w0.N), dtype=torch.float32, device="cuda")
    mg.mg_dual_gemm(blk.plan0, a0, Y0_32)
    g0 = dict(Aq=aq_rows(a0.Aq, M, w0.K)[rows], As=scale_rows(a0.As, M, w0.K)[rows],
              XO=outlier_cols(a0.XO, M, w0.k)[rows], Y=host(Y0[ridx]),
              Y32=host(Y0_32[ridx]))
    del Y0_32
    h = torch.empty_like(Y0)
    mg.mg_gelu_tanh_bf16(Y0, h)
    a2 = mg.Act.empty(blk.plan2.desc, M)
    mg.mg_quantize_act(blk.plan2, h, a2)
    af = mg.Act.empty(blk.plan2.desc, M)          # GELU + quantize in one pass, from ffn.0's output
    mg.mg_gelu_quantize_act(blk.plan2, Y0, af)
    for n in ("Aq", "As", "XO"):
        assert torch.equal(getattr(af, n).view(torch.uint8), getattr(a2, n).view(torch.uint8)), f"fused {n}"
    # GELU + quantize in ffn.0's GEMM epilogue (ffn.0's output never written)
    for t in (af.Aq, af.As, af.XO):
        t.view(torch.uint8).fill_(0x5A)
    mg.mg_dual_gemm_gelu_quant(blk.plan0, a0, blk.plan2, af)
    for n in ("Aq", "As", "XO"):
        assert torch.equal(getattr(af, n).view(torch.uint8), getattr(a2, n).view(torch.uint8)), f"epilogue {n}"
    del af, Y0, a0
    Y2 = torch.empty((M, w2.N), dtype=torch.bfloat16, device="cuda")
    mg.mg_dual_gemm(blk.plan2, a2, Y2)
    Y2_32 = torch.empty((M, w2.N), dtype=torch.float32, device="cuda")
    mg.mg_dual_gemm(blk.plan2, a2, Y2_32)
    torch.cuda.synchronize()
    hr = host(h[ridx])
    g2 = dict(Aq=aq_rows(a2.Aq, M, w2.K)[rows], As=scale_rows(a2.As, M, w2.K)[rows],
              XO=outlier_cols(a2.XO, M, w2.k)[rows], Y=host(Y2[ridx]),
              Y32=host(Y2_32[ridx]))
    del a2, Y2, Y2_32, h, X5d
    torch.cuda.empty_cache()

    # ffn.0 on the sampled rows
    oq0 = layer.quantize_act(X5[rows], o_p0["s"], o_p0["O"])
    for name in ("Aq", "As", "XO"):
        _bits_equal(g0[name], oq0[name], f"ffn.0 {name}")
    Y64_0 = layer.dual_gemm_f64(oq0["Aq"], oq0["As"], o_p0["Wq"], o_p0["Ws"], oq0["XO"], o_p0["WO"])
    e0 = check_output(g0["Y"], g0["Y32"], Y64_0)
    # GELU of the GPU's ffn.0 output
    ref_h = layer.gelu_tanh(bf16_to_f64(g0["Y"]))
    assert_faithful_bf16(bf16_to_f64(hr), ref_h)
    # ffn.2 from the GPU's h
    oq2 = layer.quantize_act(hr, o_p2["s"], o_p2["O"])
    for name in ("Aq", "As", "XO"):
        _bits_equal(g2[name], oq2[name], f"ffn.2 {name}")
    Y64_2 = layer.dual_gemm_f64(oq2["Aq"], oq2["As"], o_p2["Wq"], o_p2["Ws"], oq2["XO"], o_p2["WO"])
    e2 = check_output(g2["Y"], g2["Y32"], Y64_2)

    # fidelity of the block against the unquantized float64 block (reported)
    ref = layer.gelu_tanh(layer.reference_f64(X5[rows], block["W0"])) @ layer.as_f32(block["W2"]).astype(np.float64).T
    fid = layer.rel_fro(bf16_to_f64(g2["Y"]), ref)
    print(f"[ffn-block] {layout}: ffn.0 err {e0:.2e}, ffn.2 err {e2:.2e}, "
          f"block rel-Frobenius vs float64 {fid:.4f} on {rows.size} rows", flush=True)
