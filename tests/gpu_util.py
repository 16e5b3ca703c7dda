"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device and
running the library's entry points stage by stage."""
from __future__ import annotations

import numpy as np
import torch

import mixed_gemm_amd as mg


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def scale_rows(x, rows: int, K: int) -> np.ndarray:
    """[rows][K/32] E8M0 codes of a scale array (As, Ws) stored in scale
    windows: the code of (row r, block b) at byte ((r // 256) * nwin + b // 16)
    * 4096 + (r % 256) * 16 + 8 * (b % 2) + (b % 16) // 2, nwin = ceil(K /
    512) (inside a window row the even blocks first, then the odd ones).
    Asserts that the bytes the writers fill around the matrix (blocks past
    K/32, rows up to the end of the last 256-row group) hold code 0."""
    a = np.ascontiguousarray(host(x) if isinstance(x, torch.Tensor) else np.asarray(x)).reshape(-1)
    nwin, nb = -(-K // 512), K // 32
    assert a.dtype == np.uint8 and a.size % (nwin * 4096) == 0, (a.dtype, a.size)
    groups = a.size // (nwin * 4096)
    assert groups * 256 >= rows, (groups, rows)
    # [group][window][row][odd][block // 2] -> [group][row][window][block // 2][odd]
    full = a.reshape(groups, nwin, 256, 2, 8).transpose(0, 2, 1, 4, 3).reshape(groups * 256, nwin * 16)
    written = full[: -(-rows // 256) * 256].copy()
    written[:rows, :nb] = 0
    assert not written.any(), "scale pad bytes must hold code 0"
    return np.ascontiguousarray(full[:rows, :nb])


def frag_rows(x, rows: int, row_bytes: int) -> np.ndarray:
    """[rows][row_bytes] bytes of an operand stored in fragment order (Aq, Wq:
    row_bytes = K/2; XO, WO: row_bytes = 2k): 32-row x 32-byte blocks of 1 KB,
    block (r // 32, b // 32) at ((r // 32) * ns + b // 32) * 1024 with ns =
    2 * ceil(row_bytes / 64), byte b of row r at 16 * (r % 32 + 32 * ((b //
    16) % 2)) + b % 16 inside it.  Asserts that the pads (rows up to the next
    multiple of 32, bytes up to ns * 32) hold 0."""
    a = np.ascontiguousarray(host(x) if isinstance(x, torch.Tensor) else np.asarray(x)).reshape(-1).view(np.uint8)
    ns = 2 * -(-row_bytes // 64)
    groups = -(-rows // 32)
    assert a.size == groups * ns * 1024, (a.size, groups, ns)
    # [group][slice][half][row % 32][16] -> [group][row % 32][slice][half][16]
    full = a.reshape(groups, ns, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(groups * 32, ns * 32)
    pad = full.copy()
    pad[:rows, :row_bytes] = 0
    assert not pad.any(), "fragment-order pad bytes must hold 0"
    return np.ascontiguousarray(full[:rows, :row_bytes])


def outlier_cols(x, rows: int, k: int) -> np.ndarray:
    """The [rows][k] bf16 bit patterns of XO or WO (fragment order, rows of
    2k bytes), asserting that the pads hold +0."""
    return frag_rows(x, rows, 2 * k).view(np.uint16)


def aq_rows(x, rows: int, K: int) -> np.ndarray:
    """The [rows][K/2] packed nibbles of Aq or Wq (fragment order)."""
    return frag_rows(x, rows, K // 2)


def run_pipeline(X: np.ndarray, W: np.ndarray, alpha: float, k: int, layout: str = "1x32",
                 smooth: bool = True, calib_batches: int = 1, score: str = "max") -> dict:
    """calibrate (optionally in several batches) -> weight ranges -> plan -> quantize -> GEMM,
    each through its own entry point; returns every artefact on the host."""
    Xd, Wd = dev(X), dev(W)
    M, K = X.shape
    N = W.shape[0]
    act_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_calib_reset(act_max)
    for part in np.array_split(np.arange(M), calib_batches):
        if part.size:
            mg.mg_calib_act(Xd[part[0]:part[-1] + 1], act_max)
    w_max = torch.empty(K, dtype=torch.float32, device="cuda")
    mg.mg_weight_range(Wd, w_max)
    desc = mg.make_desc(K, N, k, alpha, layout, smooth, score)
    p = mg.Plan.empty(desc)
    mg.mg_plan_build(p, act_max, w_max, Wd)
    a = mg.Act.empty(desc, M)
    mg.mg_quantize_act(p, Xd, a)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    mg.mg_dual_gemm(p, a, Y)
    Y32 = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mg.mg_dual_gemm(p, a, Y32)
    torch.cuda.synchronize()
    out = dict(act_max=host(act_max), w_max=host(w_max), Y=host(Y), Y32=host(Y32))
    out.update({n: host(t) for n, t in p.tensors().items()})
    out["Wq"] = aq_rows(p.Wq, N, K)
    out["Ws"] = scale_rows(p.Ws, N, K)
    out["WO"] = outlier_cols(p.WO, N, k)
    out.update(Aq=aq_rows(a.Aq, M, K), As=scale_rows(a.As, M, K), XO=outlier_cols(a.XO, M, k))
    return out


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def assert_faithful_bf16(h: np.ndarray, ref: np.ndarray, floor: float = 2.0 ** -24) -> None:
    """h (float64 values of bf16 results) is a faithful bf16 rounding of the
    float64 values ref -- less than one bf16 ulp away, so one of the two bf16
    neighbours -- wherever |ref| >= floor; below it |h| <= floor."""
    h, ref = np.asarray(h, np.float64), np.asarray(ref, np.float64)
    big = np.abs(ref) >= floor
    m = np.maximum(np.abs(ref), np.abs(h))
    ulp = np.exp2(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 7)
    bad = big & ~(np.abs(h - ref) < ulp)
    assert not bad.any(), f"{int(bad.sum())} results not faithful, e.g. {h[bad][:4]} vs {ref[bad][:4]}"
    small = ~big & (np.abs(h) > floor)
    assert not small.any(), f"{int(small.sum())} tiny results above {floor}: {h[small][:4]}"


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_output(Y_bf16: np.ndarray, Y32: np.ndarray, Y64: np.ndarray, tol: float = 2e-3) -> float:
    """The GEMM's fp32 result against the unrounded float64 oracle:
    max|Y32 - Y64| / max|Y64| <= tol; the bf16 output is exactly the fp32
    result rounded to nearest-even; and every bf16 element is within one bf16
    rounding (2^-8 relative) of the oracle plus the fp32 error."""
    err = float(np.abs(Y32.astype(np.float64) - Y64).max() / np.abs(Y64).max())
    assert err <= tol, err
    assert np.array_equal(Y_bf16, f32_to_bf16_bits(Y32))
    yb = bf16_to_f64(Y_bf16)
    assert np.all(np.abs(yb - Y64) <= 2.0 ** -8 * np.abs(Y64) + 2 * err * np.abs(Y64).max() + 1e-30)
    return err
