"""Seeded synthetic inputs for the dual-branch W4A4 linear layer.

This module is shared by the CPU oracle and the HIP path and holds none of the
method's arithmetic: it only draws activations X and weights W with the shapes,
magnitudes and heavy-tailed channel structure of the Wan2.2-A14B FFN inputs
described in "W4A4 Quantization for Inference on Wan2.2-I2V-A14B" (arXiv
2606.29337, the Fig. 2 statistics of high_noise_model.block_00.ffn.0: a few
input channels with column maxima far above the rest, smooth weights).

The real calibration prompts and model weights are not available; these
generators stand in for them.

Conventions
-----------
* Every generator is ``numpy.random.Generator(numpy.random.PCG64(seed))``.
* Normals are drawn with ``standard_normal(..., dtype=float32)`` in row chunks
  from one generator, in row-major order, so a chunked draw equals a whole draw.
* bf16 tensors are returned as ``uint16`` bit patterns, rounded from float32 to
  nearest-even on the bit pattern (inputs here are always finite).
* X is ``[M][K]`` (tokens x input channels); W is ``[N][K]`` (nn.Linear layout).
"""
from __future__ import annotations

import dataclasses
from typing import Iterator

import numpy as np

CHUNK_ROWS = 4096


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    u = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (u >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def pick_channels(K: int, frac: float, seed: int) -> np.ndarray:
    """Sorted, distinct heavy-tail channel indices: round(frac*K) of K, drawn
    without replacement from a dedicated seed shared by every batch of a layer."""
    n = int(round(frac * K))
    return np.sort(rng(seed).choice(K, size=n, replace=False)).astype(np.int64)


def _normal_rows(g: np.random.Generator, M: int, K: int) -> Iterator[tuple[int, np.ndarray]]:
    for r0 in range(0, M, CHUNK_ROWS):
        r1 = min(M, r0 + CHUNK_ROWS)
        yield r0, g.standard_normal((r1 - r0, K), dtype=np.float32)


def gelu_tanh_input_f32(z: np.ndarray) -> np.ndarray:
    """Input recipe of the hidden activations that feed a down-projection: the
    tanh form of GELU of a pre-activation z, 0.5 z (1 + tanh(0.7978845608 (z +
    0.044715 z^3))), evaluated in float32 with numpy.  This draws the inputs
    only; no result is ever compared with it (the layer's own GELU step is
    checked against the oracle, in float64)."""
    z = z.astype(np.float32)
    c = np.float32(0.7978845608)
    u = c * (z + np.float32(0.044715) * z * z * z)
    return (np.float32(0.5) * z * (np.float32(1.0) + np.tanh(u))).astype(np.float32)


def heavy_tail_act(M: int, K: int, *, sigma: float, frac: float, mult: float,
                   ch_seed: int, x_seed: int, bf16: bool) -> np.ndarray:
    """N(0, sigma^2) activations with round(frac*K) channels multiplied by ``mult``."""
    ch = pick_channels(K, frac, ch_seed)
    g = rng(x_seed)
    out = np.empty((M, K), dtype=np.uint16 if bf16 else np.float32)
    for r0, z in _normal_rows(g, M, K):
        z *= np.float32(sigma)
        z[:, ch] *= np.float32(mult)
        out[r0:r0 + z.shape[0]] = f32_to_bf16_bits(z) if bf16 else z
    return out


def drifting_channels(K: int, steps: int, *, frac: float, drift: float, seed: int) -> list[np.ndarray]:
    """Heavy-channel sets for a sequence of batches: round(frac*K) channels at
    the first step; from one step to the next, round(drift * n) of them are
    replaced by channels outside the set (the rest persist)."""
    g = rng(seed)
    n = int(round(frac * K))
    cur = g.choice(K, size=n, replace=False)
    sets = [np.sort(cur).astype(np.int64)]
    for _ in range(1, steps):
        m = int(round(drift * n))
        keep = g.choice(n, size=n - m, replace=False)
        outside = np.setdiff1d(np.arange(K), cur)
        cur = np.concatenate([cur[keep], g.choice(outside, size=m, replace=False)])
        sets.append(np.sort(cur).astype(np.int64))
    return sets


def drifting_act(M: int, K: int, steps: int, *, sigma: float, frac: float, mult: float, drift: float,
                 ch_seed: int, x_seed: int) -> list[np.ndarray]:
    """bf16 batches like heavy_tail_act whose heavy channels follow
    drifting_channels (a denoising-step sequence with persistent, slowly
    moving outlier channels)."""
    out = []
    for t, ch in enumerate(drifting_channels(K, steps, frac=frac, drift=drift, seed=ch_seed)):
        g = rng(x_seed + t)
        X = np.empty((M, K), dtype=np.uint16)
        for r0, z in _normal_rows(g, M, K):
            z *= np.float32(sigma)
            z[:, ch] *= np.float32(mult)
            X[r0:r0 + z.shape[0]] = f32_to_bf16_bits(z)
        out.append(X)
    return out


def gelu_act(M: int, K: int, *, frac: float, mult: float, ch_seed: int, x_seed: int) -> np.ndarray:
    """bf16 hidden activations of a GELU-gated FFN: gelu_tanh_input_f32 of an
    N(0,1) pre-activation with round(frac*K) channels x mult."""
    ch = pick_channels(K, frac, ch_seed)
    g = rng(x_seed)
    out = np.empty((M, K), dtype=np.uint16)
    for r0, z in _normal_rows(g, M, K):
        z[:, ch] *= np.float32(mult)
        out[r0:r0 + z.shape[0]] = f32_to_bf16_bits(gelu_tanh_input_f32(z))
    return out


def weights(N: int, K: int, *, sigma: float, clip: float | None, seed: int, bf16: bool) -> np.ndarray:
    g = rng(seed)
    out = np.empty((N, K), dtype=np.uint16 if bf16 else np.float32)
    for r0, z in _normal_rows(g, N, K):
        z *= np.float32(sigma)
        if clip is not None:
            np.clip(z, -clip, clip, out=z)
        out[r0:r0 + z.shape[0]] = f32_to_bf16_bits(z) if bf16 else z
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One dual-branch linear layer workload."""
    name: str
    M: int
    K: int
    N: int
    k: int
    alpha: float
    dtype: str            # "f32" or "bf16" (activations and weights)
    act: str              # "heavy" or "gelu"
    act_sigma: float
    act_frac: float
    act_mult: float
    w_sigma: float
    w_clip: float | None
    ch_seed: int
    x_seed: int
    w_seed: int

    def make_x(self, M: int | None = None, x_seed: int | None = None) -> np.ndarray:
        M = self.M if M is None else M
        xs = self.x_seed if x_seed is None else x_seed
        if self.act == "gelu":
            return gelu_act(M, self.K, frac=self.act_frac, mult=self.act_mult,
                            ch_seed=self.ch_seed, x_seed=xs)
        return heavy_tail_act(M, self.K, sigma=self.act_sigma, frac=self.act_frac,
                              mult=self.act_mult, ch_seed=self.ch_seed, x_seed=xs,
                              bf16=self.dtype == "bf16")

    def make_w(self) -> np.ndarray:
        return weights(self.N, self.K, sigma=self.w_sigma, clip=self.w_clip,
                       seed=self.w_seed, bf16=self.dtype == "bf16")

    def flops(self, M: int | None = None) -> float:
        return 2.0 * (self.M if M is None else M) * self.K * self.N


# Tiny layer: 256 tokens x 512 -> 1024, fp32, 2% of channels x25.
TINY = Workload("tiny_256x512x1024", 256, 512, 1024, 8, 0.5, "f32", "heavy",
                0.25, 0.02, 25.0, 0.05, 0.6, 101, 102, 103)
# Wan2.2-A14B FFN up-projection at 480p (21x30x52 tokens), 5120 -> 13824.
FFN0_480P = Workload("ffn0_480p_32760x5120x13824", 32760, 5120, 13824, 64, 0.6, "bf16", "heavy",
                     0.25, 0.02, 25.0, 0.02, 0.6, 201, 202, 203)
# FFN down-projection at 480p, 13824 -> 5120: GELU-tanh hidden activations with 1% channels x20.
FFN2_480P = Workload("ffn2_480p_32760x13824x5120", 32760, 13824, 5120, 128, 0.5, "bf16", "gelu",
                     1.0, 0.01, 20.0, 0.01, None, 301, 302, 303)
# FFN up-projection at 720p (21x45x80 tokens).
FFN0_720P = Workload("ffn0_720p_75600x5120x13824", 75600, 5120, 13824, 64, 0.6, "bf16", "heavy",
                     0.25, 0.02, 25.0, 0.02, 0.6, 201, 402, 203)

# The (k, alpha) sweep run on the 720p up-projection.
SWEEP_K = (0, 32, 64, 128)
SWEEP_ALPHA = (0.5, 0.6, 0.7)

# Full FFN block at 720p: ffn.0 -> GELU-tanh -> ffn.2.  Calibration batches use
# x seeds 501..504, the evaluation batch seed 505.
BLOCK_M = 75600
BLOCK_CALIB_SEEDS = (501, 502, 503, 504)
BLOCK_EVAL_SEED = 505
BLOCK_FFN0 = dataclasses.replace(FFN0_720P, name="block_ffn0_720p", x_seed=BLOCK_EVAL_SEED)
BLOCK_FFN2 = dataclasses.replace(FFN2_480P, name="block_ffn2_720p", M=BLOCK_M)

ALL = {w.name: w for w in (TINY, FFN0_480P, FFN2_480P, FFN0_720P)}
