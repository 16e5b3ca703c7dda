"""mg_forward_noalloc (the forward pass with the library's own per-GPU
workspace, for callers that cannot allocate) against mg_forward with a
caller workspace: bit-identical outputs on two calls in a row, the second with
fewer rows (and K), so the shared array holds the first call's contents."""
import numpy as np
import pytest
import torch

import mixed_gemm_amd as mg
import synth
from tests.gpu_util import dev, host

pytestmark = pytest.mark.gpu


def _layer(M, K, N, k, seed, alpha=0.6):
    X = synth.heavy_tail_act(M, K, sigma=0.25, frac=0.02, mult=25.0, ch_seed=seed, x_seed=seed + 1, bf16=True)
    W = synth.weights(N, K, sigma=0.02, clip=0.6, seed=seed + 2, bf16=True)
    Xd, Wd = dev(X), dev(W)
    p = mg.plan(mg.calibrate([Xd], K), Wd, alpha, k)
    return p, Xd


@pytest.mark.parametrize("y_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_forward_twice(y_dtype):
    print("\n[noalloc] two calls: 9000x5120x1024 k=64, then 700x1536x512 k=13", flush=True)
    cases = [(9000, 5120, 1024, 64, 11), (700, 1536, 512, 13, 12)]
    for M, K, N, k, seed in cases:
        p, Xd = _layer(M, K, N, k, seed)
        Y_ref = torch.empty((M, N), dtype=y_dtype, device="cuda")
        a = mg.Act.empty(p.desc, M)
        mg.mg_forward(p, Xd, a, Y_ref)
        Y = torch.full((M, N), float("nan"), dtype=y_dtype, device="cuda")
        mg.mg_forward_noalloc(p, Xd, Y)
        torch.cuda.synchronize()
        ref, got = host(Y_ref), host(Y)
        assert np.array_equal(ref.view(np.uint8), got.view(np.uint8)), (M, K, N, k)
        print(f"[noalloc] M={M} K={K} N={N} k={k}: identical", flush=True)


def test_noalloc_rejects_oversized_workspace():
    p, Xd = _layer(64, 5120, 256, 64, 21)
    M = 24000                                   # 24000 rows at K = 5120, k = 64 exceed 64 MiB
    X = torch.zeros((M, 5120), dtype=torch.bfloat16, device="cuda")
    Y = torch.empty((M, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.MGError, match="limit"):
        mg.mg_forward_noalloc(p, X, Y)
    # the largest M that fits still runs and matches mg_forward
    M = 23000
    X = dev(synth.heavy_tail_act(M, 5120, sigma=0.25, frac=0.02, mult=25.0, ch_seed=21, x_seed=23, bf16=True))
    Y = torch.empty((M, 256), dtype=torch.bfloat16, device="cuda")
    Y_ref = torch.empty_like(Y)
    mg.mg_forward_noalloc(p, X, Y)
    mg.mg_forward(p, X, mg.Act.empty(p.desc, M), Y_ref)
    torch.cuda.synchronize()
    assert torch.equal(Y.view(torch.int16), Y_ref.view(torch.int16))
