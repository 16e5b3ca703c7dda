"""MXFP4 (E2M1 elements, E8M0 block scales) encode/decode -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The pages ("W4A4 Quantization for Inference on Wan2.2-I2V-A14B", block-packing
paragraph after Eq. (5)) say only that 4-bit payloads are stored with
per-block exponents, in 32x32 tiles or K-major stripes, for the HiF4/MXFP4
formats.  HiF4 is never defined, so the oracle implements MXFP4:

* element grid (E2M1 magnitudes) {0, 0.5, 1, 1.5, 2, 3, 4, 6}, code = index;
* block scale X = 2^(c - 127) with the E8M0 code c = floor(log2 amax) - 2 + 127,
  clamped below at 0 (amax = 0 or tiny blocks give c = 0);
* element code = nearest grid value to |v| / X, ties to the even code,
  values beyond 6 saturate to 6; sign bit copied from v (so -0 -> 0x8);
* two elements per byte, the even K index in the low nibble.

Arrays of bf16 values are uint16 bit patterns throughout the oracle.
"""
from __future__ import annotations

import numpy as np

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
# Midpoints between neighbouring grid values.
MIDS = (GRID[1:] + GRID[:-1]) / 2.0
BLOCK = 32


def e8m0_from_amax(amax: np.ndarray) -> np.ndarray:
    """E8M0 scale code of a block from its f32 absolute maximum.

    floor(log2 amax) for a normal f32 is its unbiased exponent E - 127, so the
    biased code floor(log2 amax) - 2 + 127 is E - 2; subnormal or zero amax
    (E = 0) and E < 2 clamp to code 0 (2^-127)."""
    a = np.ascontiguousarray(amax, dtype=np.float32)
    E = ((a.view(np.uint32) >> np.uint32(23)) & np.uint32(0xFF)).astype(np.int64)
    return np.maximum(E - 2, 0).astype(np.uint8)


def e2m1_code(r: np.ndarray) -> np.ndarray:
    """Magnitude code (0..7) of r >= 0 (float64, already divided by the scale).

    The code is the number of midpoints strictly below r; exactly on a
    midpoint (a tie) the even code of the two neighbours wins, i.e. the upper
    neighbour when its code is even.  Anything above the last midpoint (5)
    maps to code 7 (6.0): saturation."""
    r = np.asarray(r, dtype=np.float64)
    i = np.searchsorted(MIDS, r, side="left")          # #{mid < r}
    on_mid = np.zeros(r.shape, dtype=bool)
    inside = i < MIDS.size
    on_mid[inside] = MIDS[i[inside]] == r[inside]
    upper_even = (i + 1) % 2 == 0
    return (i + (on_mid & upper_even)).astype(np.uint8)


def encode_with_scale(v: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Nibbles (sign<<3 | code) of f32 values v under per-element E8M0 codes c."""
    v = np.asarray(v, dtype=np.float32)
    r = np.ldexp(np.abs(v).astype(np.float64), 127 - c.astype(np.int64))   # exact
    sign = np.signbit(v).astype(np.uint8)
    return (sign << 3) | e2m1_code(r)


def decode_nibbles(nib: np.ndarray, c: np.ndarray) -> np.ndarray:
    """Exact float64 values of nibbles under per-element E8M0 codes c."""
    nib = np.asarray(nib, dtype=np.uint8)
    mag = GRID[nib & 7]
    val = np.ldexp(mag, c.astype(np.int64) - 127)
    return np.where(nib & 8, -val, val)


def pack_nibbles(nib: np.ndarray) -> np.ndarray:
    """[R][K] nibbles -> [R][K/2] bytes, even index in the low nibble."""
    nib = np.asarray(nib, dtype=np.uint8)
    return (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(b: np.ndarray) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint8)
    out = np.empty(b.shape[:-1] + (b.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = b & 0xF
    out[..., 1::2] = b >> 4
    return out


def block_amax_rows(v: np.ndarray) -> np.ndarray:
    """[R][K] f32 -> [R][K/32] f32 absolute maxima of consecutive 32-blocks."""
    R, K = v.shape
    assert K % BLOCK == 0
    return np.abs(v).reshape(R, K // BLOCK, BLOCK).max(axis=2)


def encode_rows(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """1x32 blocks along K.  [R][K] f32 -> (packed [R][K/2] u8, scales [R][K/32] u8)."""
    v = np.asarray(v, dtype=np.float32)
    c = e8m0_from_amax(block_amax_rows(v))
    nib = encode_with_scale(v, np.repeat(c, BLOCK, axis=1))
    return pack_nibbles(nib), c


def encode_tiles(v: np.ndarray) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """32x32 tiles (32 rows x 32 K).  [R][K] f32 ->
    (packed [R][K/2] u8, per-row scales [R][K/32] u8 = tile scale broadcast
    over the tile's rows, compact tile scales [R/32][K/32] u8)."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    assert R % BLOCK == 0 and K % BLOCK == 0
    tamax = np.abs(v).reshape(R // BLOCK, BLOCK, K // BLOCK, BLOCK).max(axis=(1, 3))
    ct = e8m0_from_amax(tamax)
    c_rows = np.repeat(ct, BLOCK, axis=0)
    nib = encode_with_scale(v, np.repeat(c_rows, BLOCK, axis=1))
    return pack_nibbles(nib), c_rows, ct


def encode_stripes(v: np.ndarray, width: int = 128) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """K-major stripes of `width` consecutive K of one row (the 128x1 layout;
    the last stripe of a row may be shorter).  [R][K] f32 -> (packed [R][K/2]
    u8, per-block scales [R][K/32] u8 = the stripe's code on each of its
    32-blocks, compact stripe scales [R][ceil(K/width)] u8)."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    assert K % BLOCK == 0 and width % BLOCK == 0
    ns = -(-K // width)
    pad = ns * width - K
    a = np.abs(np.pad(v, ((0, 0), (0, pad)))).reshape(R, ns, width).max(axis=2)
    cs = e8m0_from_amax(a)
    c_blocks = np.repeat(cs, width // BLOCK, axis=1)[:, :K // BLOCK]
    nib = encode_with_scale(v, np.repeat(c_blocks, BLOCK, axis=1))
    return pack_nibbles(nib), c_blocks, cs


def decode_rows(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(packed [R][K/2], scales [R][K/32]) -> exact float64 [R][K]."""
    nib = unpack_nibbles(packed)
    return decode_nibbles(nib, np.repeat(np.asarray(scales), BLOCK, axis=1))
