"""GELU and the next projection's activation quantize inside the dual GEMM's
epilogue (mg_dual_gemm_gelu_quant; "W4A4 Quantization for Inference on
Wan2.2-I2V-A14B", the integration paragraph: the FFN's second projection
quantizes the GELU-gated hidden activations).

The fused call must write, bit for bit and including every pad byte, what the
two-step path writes: mg_dual_gemm (bf16 output) followed by
mg_gelu_quantize_act -- which the FFN-block tests check stage-wise against the
oracle.  Both workspaces start filled with a garbage byte, so a byte that one
path leaves unwritten shows up.  Shapes cover ragged M (pad rows of the last
32-row and 256-row groups), N not a multiple of 256 or 512 (tiles and scale
windows that end inside the next layer's K), k2 = 0, one outlier, and many
outliers per lane (the lanes' further outlier channels), and the three weight
layouts; the 720p FFN block at full size is in tests/test_gpu_ffn_block.py.
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu


def _bf16(x: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16_bits(x.astype(np.float32))


def _inputs(M, K0, N0, N2, seed):
    g = np.random.default_rng(seed)
    X = g.normal(0.0, 0.5, (M, K0)).astype(np.float32)
    X[:, g.choice(K0, max(1, K0 // 50), replace=False)] *= 20.0
    W0 = g.normal(0.0, 0.06, (N0, K0)).astype(np.float32)
    W2 = g.normal(0.0, 0.04, (N2, N0)).astype(np.float32)
    return _bf16(X), _bf16(W0), _bf16(W2)


def _garbage(act: mg.Act) -> None:
    for t in (act.Aq, act.As, act.XO):
        t.view(torch.uint8).fill_(0x5A)


@pytest.mark.parametrize("M,K0,N0,N2,k0,k2,layout", [
    (300, 512, 352, 96, 8, 5, "1x32"),
    (777, 256, 800, 64, 0, 64, "32x32"),
    (64, 1024, 512, 128, 16, 0, "1x32"),
    (513, 256, 1056, 32, 4, 300, "128x1"),
    (1, 128, 32, 32, 1, 1, "1x32"),
    (2000, 640, 2304, 160, 12, 40, "1x32"),
])
def test_epilogue_equals_two_step(M, K0, N0, N2, k0, k2, layout):
    print(f"\n[fused-epilogue] M={M} K0={K0} N0={N0} N2={N2} k0={k0} k2={k2} {layout}", flush=True)
    X, W0, W2 = _inputs(M, K0, N0, N2, 1000 + M)
    Xd, W0d, W2d = dev(X), dev(W0), dev(W2)
    act0, act2 = mg.ffn_block_stats([Xd], W0d)
    blk = mg.ffn_block_plans(act0, act2, W0d, W2d, 0.6, k0, 0.5, k2, layout)
    a0 = mg.Act.empty(blk.plan0.desc, M)
    mg.mg_quantize_act(blk.plan0, Xd, a0)
    # two steps: ffn.0's bf16 output, then GELU + quantize in one pass
    Y0 = torch.empty((M, N0), dtype=torch.bfloat16, device="cuda")
    mg.mg_dual_gemm(blk.plan0, a0, Y0)
    ref = mg.Act.empty(blk.plan2.desc, M)
    _garbage(ref)
    mg.mg_gelu_quantize_act(blk.plan2, Y0, ref)
    # the GEMM epilogue
    fused = mg.Act.empty(blk.plan2.desc, M)
    _garbage(fused)
    mg.mg_dual_gemm_gelu_quant(blk.plan0, a0, blk.plan2, fused)
    torch.cuda.synchronize()
    for name in ("Aq", "As", "XO"):
        a = getattr(fused, name).view(torch.uint8)
        b = getattr(ref, name).view(torch.uint8)
        if not torch.equal(a, b):
            bad = int((a != b).sum())
            raise AssertionError(f"{name}: {bad} of {a.numel()} bytes differ")
    # and the block's output through either path
    y_two = mg.ffn_block_forward(blk, Xd)
    y_epi = mg.ffn_block_forward(blk, Xd, epilogue=True)
    assert torch.equal(y_two.view(torch.int16), y_epi.view(torch.int16))


def test_rejects_mismatched_widths():
    X, W0, W2 = _inputs(64, 256, 256, 64, 5)
    Xd, W0d = dev(X), dev(W0)
    p0 = mg.plan(mg.calibrate([Xd], 256), W0d, 0.6, 4)
    W2b = dev(_bf16(np.ones((64, 512), np.float32)))
    p2 = mg.plan(torch.ones(512, device="cuda"), W2b, 0.5, 4)        # K = 512 != N0 = 256
    a0 = mg.Act.empty(p0.desc, 64)
    a2 = mg.Act.empty(p2.desc, 64)
    with pytest.raises(ValueError):
        mg.mg_dual_gemm_gelu_quant(p0, a0, p2, a2)
