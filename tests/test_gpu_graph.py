"""HIP graph capture of the hot path.

Every entry point launches kernels on the caller's stream only: resets are
fill kernels (no memset nodes), nothing is allocated and nothing
synchronizes, so a whole step can be captured once and replayed.  Each test
captures on torch's capture stream after an eager warm-up (which also sets
the GEMM's one-time kernel attribute), then replays several times with
different inputs copied into the captured input buffer, eager work that
overwrites every output, and a synchronization between replays; every
replay must equal a separate eager run on the same input, bit for bit.
"""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from tests.gpu_util import dev

pytestmark = pytest.mark.gpu

REPLAYS = 6


def _bits(t: torch.Tensor) -> torch.Tensor:
    return t.detach().contiguous().view(torch.uint8).clone()


def _same(got: dict, want: dict, tag: str) -> None:
    for name, w in want.items():
        assert torch.equal(got[name], w), f"{tag}: {name} differs"


class _StepBuffers:
    """Outputs of one calibrate -> plan -> quantize -> dual GEMM step."""

    def __init__(self, desc, M, K, N):
        self.act_max = torch.empty(K, dtype=torch.float32, device="cuda")
        self.w_max = torch.empty(K, dtype=torch.float32, device="cuda")
        self.plan = mg.Plan.empty(desc)
        self.act = mg.Act.empty(desc, M)
        self.Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def tensors(self) -> dict:
        t = dict(act_max=self.act_max, w_max=self.w_max, Aq=self.act.Aq, As=self.act.As, XO=self.act.XO, Y=self.Y)
        t.update({n: v for n, v in self.plan.tensors().items() if v is not None and v.numel()})
        return t

    def snapshot(self) -> dict:
        return {n: _bits(v) for n, v in self.tensors().items()}

    def scribble(self) -> None:
        for v in self.tensors().values():
            v.view(torch.uint8).fill_(0xA5)


def _step(X, W, b: _StepBuffers) -> None:
    mg.mg_calib_reset(b.act_max)
    mg.mg_calib_act(X, b.act_max)
    mg.mg_weight_range(W, b.w_max)
    mg.mg_plan_build(b.plan, b.act_max, b.w_max, W)
    mg.mg_quantize_act(b.plan, X, b.act)
    mg.mg_dual_gemm(b.plan, b.act, b.Y)


def _capture(fn) -> torch.cuda.CUDAGraph:
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                   # warm-up on a side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_step_graph_replays_match_eager():
    M, K, N, k = 1000, 1024, 512, 40
    Xs = [synth.heavy_tail_act(M, K, sigma=0.25, frac=0.02, mult=25.0, ch_seed=70 + r, x_seed=80 + r, bf16=True)
          for r in range(3)]
    Wd = dev(synth.weights(N, K, sigma=0.02, clip=0.6, seed=90, bf16=True))
    desc = mg.make_desc(K, N, k, 0.6)
    print(f"\n[graph] step M={M} K={K} N={N} k={k}: eager references", flush=True)
    want = []
    for X in Xs:
        b = _StepBuffers(desc, M, K, N)
        _step(dev(X), Wd, b)
        torch.cuda.synchronize()
        want.append(b.snapshot())
    Xd = dev(Xs[0]).clone()
    b = _StepBuffers(desc, M, K, N)
    g = _capture(lambda: _step(Xd, Wd, b))
    print("[graph] step captured; replaying", flush=True)
    for rep in range(REPLAYS):
        r = rep % 3
        Xd.copy_(dev(Xs[r]))
        b.scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(b.snapshot(), want[r], f"replay {rep} (input {r})")


@pytest.mark.parametrize("epilogue", [False, True])
def test_ffn_block_forward_graph_replays_match_eager(epilogue):
    """quantize -> GEMM (ffn.0) -> fused GELU + quantize -> GEMM (ffn.2) with
    plans built beforehand, captured as one graph; with epilogue=True the GELU
    and ffn.2's quantize run in ffn.0's GEMM epilogue (which reads its
    arguments from the kernel-argument segment once per tile: a graph's kernel
    node carries its own copy of that segment)."""
    M, K0, N0, N2, k0, k2 = 600, 512, 1024, 384, 16, 32
    Xs = [synth.heavy_tail_act(M, K0, sigma=0.25, frac=0.02, mult=25.0, ch_seed=170 + r, x_seed=180 + r, bf16=True)
          for r in range(3)]
    W0 = dev(synth.weights(N0, K0, sigma=0.02, clip=0.6, seed=190, bf16=True))
    W2 = dev(synth.weights(N2, N0, sigma=0.01, clip=None, seed=191, bf16=True))
    # plans from the first batch and the unquantized block's hidden activations
    X0 = dev(Xs[0])
    act0 = mg.calibrate([X0], K0)
    ref0 = mg.reference_plan(W0)
    aref = mg.Act.empty(ref0.desc, M)
    y = torch.empty((M, N0), dtype=torch.bfloat16, device="cuda")
    mg.mg_forward(ref0, X0, aref, y)
    h = torch.empty_like(y)
    mg.mg_gelu_tanh_bf16(y, h)
    act2 = mg.calibrate([h], N0)
    p0 = mg.plan(act0, W0, 0.6, k0)
    p2 = mg.plan(act2, W2, 0.5, k2)
    torch.cuda.synchronize()

    class Bufs:
        def __init__(self):
            self.a0 = mg.Act.empty(p0.desc, M)
            self.y0 = torch.empty((M, N0), dtype=torch.bfloat16, device="cuda")
            self.a2 = mg.Act.empty(p2.desc, M)
            self.y2 = torch.empty((M, N2), dtype=torch.bfloat16, device="cuda")

        def tensors(self):
            t = dict(Aq0=self.a0.Aq, As0=self.a0.As, XO0=self.a0.XO, Y0=self.y0,
                     Aq2=self.a2.Aq, As2=self.a2.As, XO2=self.a2.XO, Y2=self.y2)
            if epilogue:
                del t["Y0"]                   # not written in the epilogue form
            return t

    def fwd(X, bb):
        mg.mg_quantize_act(p0, X, bb.a0)
        if epilogue:
            mg.mg_dual_gemm_gelu_quant(p0, bb.a0, p2, bb.a2)
        else:
            mg.mg_dual_gemm(p0, bb.a0, bb.y0)
            mg.mg_gelu_quantize_act(p2, bb.y0, bb.a2)
        mg.mg_dual_gemm(p2, bb.a2, bb.y2)

    print(f"\n[graph] FFN block M={M} {K0}->{N0}->{N2} epilogue={epilogue}: eager references", flush=True)
    want = []
    for X in Xs:
        bb = Bufs()
        fwd(dev(X), bb)
        torch.cuda.synchronize()
        want.append({n: _bits(v) for n, v in bb.tensors().items()})
    Xd = dev(Xs[0]).clone()
    bb = Bufs()
    g = _capture(lambda: fwd(Xd, bb))
    print("[graph] FFN block captured; replaying", flush=True)
    for rep in range(REPLAYS):
        r = rep % 3
        Xd.copy_(dev(Xs[r]))
        for v in bb.tensors().values():
            v.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same({n: _bits(v) for n, v in bb.tensors().items()}, want[r], f"replay {rep} (input {r})")
