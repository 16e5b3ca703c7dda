"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, answers size queries with the closed-form byte counts, and rejects
bad arguments on the host (no GPU call is reached by these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mixed_gemm_amd as mg
from tests.gpu_util import frag_rows, scale_rows

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "mixed_gemm.h")
FAKE = 1 << 20          # aligned, never dereferenced: every call below fails validation first


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(mg_\w+)\s*\(", text, re.M)))


def test_every_export_has_a_ctypes_signature():
    """Without argtypes ctypes would pass device pointers as 32-bit ints."""
    L = mg.lib()
    for n in mg.EXPORTS:
        assert getattr(L, n).argtypes is not None, n
    for n in ("mg_quantize_act", "mg_gelu_quantize_act", "mg_dual_gemm", "mg_forward", "mg_calib_act"):
        assert ctypes.c_void_p in getattr(L, n).argtypes, n


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 15
    L = mg.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(mg.EXPORTS)
    assert mg.mg_version() >= 100


def test_plan_and_act_sizes():
    d = mg.make_desc(5120, 13824, 64, 0.6, "1x32")
    b = mg.mg_plan_bytes(d)
    # Wq, WO in fragment order: 32-row x 32-byte blocks of 1 KB
    assert b == [4 * 5120, 4 * 5120, 4 * 64, 4 * 5120, 432 * 80 * 1024, 13824 * 160, 0, 432 * 4 * 1024]
    d2 = mg.make_desc(512, 1024, 8, 0.5, "32x32")
    assert mg.mg_plan_bytes(d2)[6] == 32 * 16
    # scales in 256-row x 16-block windows of 4 KB: 128 row groups x 10 windows
    assert mg.mg_act_bytes(d, 32760) == [1024 * 80 * 1024, 128 * 10 * 4096, 1024 * 4 * 1024]
    d4 = mg.make_desc(352, 96, 3, 0.5, "1x32")               # 176-byte rows: 6 slices; 6-byte XO rows: 2
    assert mg.mg_act_bytes(d4, 33) == [2 * 6 * 1024, 1 * 1 * 4096, 2 * 2 * 1024]
    assert mg.mg_plan_bytes(d4)[4] == 3 * 6 * 1024 and mg.mg_plan_bytes(d4)[7] == 3 * 2 * 1024
    d5 = mg.make_desc(480, 96, 40, 0.5, "1x32")              # 240-byte rows: 8 slices (7 padded to 8); XO 80: 4
    assert mg.mg_act_bytes(d5, 64) == [2 * 8 * 1024, 1 * 1 * 4096, 2 * 4 * 1024]
    assert mg.mg_act_bytes(d, 0) == [0, 0, 0]
    d3 = mg.make_desc(352, 96, 3, 0.5, "1x32")               # K % 512 != 0: one window per group
    assert mg.mg_plan_bytes(d3)[5] == 1 * 1 * 4096
    assert mg.mg_act_bytes(d3, 300)[1] == 2 * 1 * 4096


@pytest.mark.parametrize("rows,K", [(300, 352), (256, 512), (1, 32), (513, 1568)])
def test_scale_window_layout(rows, K):
    """The tests' reader of the stored scale order against the header's byte
    formula applied code by code, and the buffer size against mg_act_bytes."""
    rng = np.random.default_rng(rows + K)
    nb, nwin = K // 32, -(-K // 512)
    codes = rng.integers(1, 255, size=(rows, nb), dtype=np.uint8)
    buf = np.zeros(-(-rows // 256) * nwin * 4096, dtype=np.uint8)
    for r in range(rows):
        for b in range(nb):
            buf[((r // 256) * nwin + b // 16) * 4096 + (r % 256) * 16 + 8 * (b % 2) + (b % 16) // 2] = codes[r, b]
    assert buf.size == mg.mg_act_bytes(mg.make_desc(K, 32, 0, 0.5, "1x32"), rows)[1]
    assert buf.size == int(np.prod(mg.scale_shape(rows, K)))
    assert np.array_equal(scale_rows(buf, rows, K), codes)
    if buf.size > rows * nb:                                  # a non-zero pad byte is caught
        pad = np.flatnonzero(buf == 0)[0]
        buf[pad] = 7
        with pytest.raises(AssertionError):
            scale_rows(buf, rows, K)


@pytest.mark.parametrize("rows,row_bytes", [(33, 176), (32, 64), (1, 16), (70, 6), (64, 2560)])
def test_fragment_order_layout(rows, row_bytes):
    """The tests' reader of the fragment order against the header's byte
    formula applied byte by byte, and the buffer size against frag_shape."""
    rng = np.random.default_rng(rows * 7 + row_bytes)
    data = rng.integers(1, 255, size=(rows, row_bytes), dtype=np.uint8)
    ns = 2 * -(-row_bytes // 64)
    buf = np.zeros(-(-rows // 32) * ns * 1024, dtype=np.uint8)
    for r in range(rows):
        for b in range(row_bytes):
            buf[((r // 32) * ns + b // 32) * 1024 + 16 * (r % 32 + 32 * ((b // 16) % 2)) + b % 16] = data[r, b]
    assert buf.size == int(np.prod(mg.frag_shape(rows, row_bytes)))
    assert np.array_equal(frag_rows(buf, rows, row_bytes), data)
    if buf.size > data.size:                                  # a non-zero pad byte is caught
        buf[np.flatnonzero(buf == 0)[0]] = 9
        with pytest.raises(AssertionError):
            frag_rows(buf, rows, row_bytes)


@pytest.mark.parametrize("K,N,k,alpha,layout,smooth,code", [
    (100, 64, 4, 0.5, 0, 1, -2),      # K % 32
    (0, 64, 0, 0.5, 0, 1, -2),        # K == 0
    (64, 48, 4, 0.5, 0, 1, -2),       # N % 32
    (64, 64, 65, 0.5, 0, 1, -2),      # k > K
    (64, 64, -1, 0.5, 0, 1, -2),      # k < 0
    (64, 64, 4, 0.0, 0, 1, -1),       # alpha
    (64, 64, 4, 1.0, 0, 1, -1),       # alpha
    (64, 64, 4, 0.5, 3, 1, -1),       # layout
    (64, 64, 4, 0.5, 0, 3, -1),       # smooth flag
    (131072, 64, 4, 0.5, 0, 1, -5),   # K beyond the limit
])
def test_desc_validation(K, N, k, alpha, layout, smooth, code):
    d = mg.mg_plan_desc(K, N, k, layout, smooth, 0, alpha)
    out = (ctypes.c_size_t * 8)()
    assert mg.lib().mg_plan_bytes(ctypes.byref(d), out) == code
    assert mg.lib().mg_last_error()


def test_score_and_stripe_layout_sizes():
    out = (ctypes.c_size_t * 8)()
    d = mg.mg_plan_desc(64, 64, 4, 0, 1, 2, 0.5)                  # score 2 does not exist
    assert mg.lib().mg_plan_bytes(ctypes.byref(d), out) == -1
    d = mg.make_desc(352, 64, 4, 0.5, "128x1", score="smoothed")  # stripes 128, 128, 96
    assert mg.mg_plan_bytes(d)[6] == 64 * 3
    p = mg.mg_plan(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    assert mg.lib().mg_fold_pack(ctypes.byref(p), FAKE, 1, None) == -1     # Wst required


def test_alpha_ignored_without_smoothing():
    d = mg.make_desc(64, 64, 4, 0.0, "1x32", smooth=False)
    assert mg.mg_plan_bytes(d)[0] == 256


def _plan(K=64, N=64, k=4, **over):
    d = mg.make_desc(K, N, k, 0.5)
    p = mg.mg_plan(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, FAKE)
    for n, v in over.items():
        setattr(p, n, v)
    return p


def test_pointer_validation():
    L = mg.lib()
    # null and misaligned pointers
    assert L.mg_calib_act(None, 1, 8, 64, FAKE, None) == -1
    assert L.mg_calib_act(FAKE + 2, 1, 8, 64, FAKE, None) == -4
    assert L.mg_calib_act(FAKE, 7, 8, 64, FAKE, None) == -3
    assert L.mg_calib_act(FAKE, 1, -1, 64, FAKE, None) == -2
    assert L.mg_calib_act(FAKE, 1, 8, 60, FAKE, None) == -2
    assert L.mg_weight_range(FAKE, 1, 0, 64, FAKE, None) == -2
    assert L.mg_calib_reset(None, 64, None) == -1
    p = _plan(s=None)
    assert L.mg_smooth_scales(ctypes.byref(p), FAKE, FAKE, None) == -1
    p = _plan(Wq=FAKE + 8)
    assert L.mg_fold_pack(ctypes.byref(p), FAKE, 1, None) == -4
    p = _plan(WO=None)
    assert L.mg_fold_pack(ctypes.byref(p), FAKE, 1, None) == -1
    p = _plan()
    a = mg.mg_act(FAKE, FAKE, None)                 # XO missing while k > 0
    assert L.mg_quantize_act(ctypes.byref(p), FAKE, 1, 16, ctypes.byref(a), None) == -1
    assert L.mg_dual_gemm(ctypes.byref(p), ctypes.byref(a), 16, FAKE, 1, None) == -1
    a = mg.mg_act(FAKE, FAKE, FAKE)
    assert L.mg_forward(ctypes.byref(p), FAKE, 1, 16, ctypes.byref(a), None, 1, None) == -1
    assert L.mg_dual_gemm(ctypes.byref(p), ctypes.byref(a), 16, FAKE, 9, None) == -3
    assert L.mg_quantize_act(ctypes.byref(p), FAKE, 5, 16, ctypes.byref(a), None) == -3
    assert L.mg_gelu_tanh_bf16(FAKE, FAKE, -5, None) == -2
    assert L.mg_gelu_tanh_bf16(None, FAKE, 5, None) == -1
    assert b"null" in L.mg_last_error()
    # k == 0 allows null O / WO / XO: validation passes and only the GPU work would remain,
    # so check it through a descriptor-level query instead
    d = mg.make_desc(64, 64, 0, 0.5)
    assert mg.mg_act_bytes(d, 5)[2] == 0


def test_tile_layout_needs_wst():
    L = mg.lib()
    d = mg.make_desc(64, 64, 4, 0.5, "32x32")
    p = mg.mg_plan(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE)
    assert L.mg_fold_pack(ctypes.byref(p), FAKE, 1, None) == -1


def test_percentile_state_validation():
    L = mg.lib()
    st = mg.mg_pct(FAKE, FAKE, 64, 0)
    assert L.mg_pct_select(ctypes.byref(st), 0, 0.0, None, None) == -1        # q must lie in (0, 1]
    assert L.mg_pct_select(ctypes.byref(st), 0, 1.5, None, None) == -1
    assert L.mg_pct_select(ctypes.byref(st), 0, float("nan"), None, None) == -1
    assert L.mg_pct_select(ctypes.byref(st), 1, 0.5, None, None) == -1        # pass 1 writes score
    assert L.mg_pct_select(ctypes.byref(st), 2, 0.5, FAKE, None) == -1        # pass 0 or 1
    assert L.mg_pct_count(ctypes.byref(st), 3, FAKE, 8, None) == -1
    assert L.mg_pct_count(ctypes.byref(st), 0, FAKE, -1, None) == -2
    assert L.mg_pct_count(ctypes.byref(st), 0, None, 8, None) == -1
    assert L.mg_pct_count(ctypes.byref(st), 0, FAKE + 4, 8, None) == -4
    assert L.mg_pct_count(ctypes.byref(st), 0, None, 0, None) == 0            # M == 0: no-op
    assert L.mg_pct_count(ctypes.byref(st), 0, FAKE, 65535 * 65535 + 1, None) == -5   # 16-bit counters
    assert L.mg_pct_reset(ctypes.byref(mg.mg_pct(FAKE, FAKE, 60, 0)), None) == -2
    assert L.mg_pct_reset(ctypes.byref(mg.mg_pct(None, FAKE, 64, 0)), None) == -1
    assert L.mg_pct_reset(ctypes.byref(mg.mg_pct(FAKE, FAKE, 64, 1)), None) == -1
    assert L.mg_pct_reset(None, None) == -1


def test_missing_library_and_host_tensors_fail_loudly(tmp_path):
    """No fallback: without the built library every entry point raises, and a
    host tensor is refused before any library call."""
    import torch
    saved_lib, saved_path = mg._lib, mg.LIB_PATH
    try:
        mg._lib = None
        mg.LIB_PATH = str(tmp_path / "libmissing.so")
        with pytest.raises(RuntimeError, match="not built"):
            mg.lib()
        with pytest.raises(RuntimeError, match="not built"):
            mg.mg_version()
        with pytest.raises(RuntimeError, match="not built"):
            mg.mg_calib_reset(torch.zeros(32))
    finally:
        mg._lib, mg.LIB_PATH = saved_lib, saved_path
    with pytest.raises(ValueError, match="device tensor"):
        mg.mg_calib_reset(torch.zeros(32))


def test_plan_state_round_trip(tmp_path):
    """Plan.state() survives torch.save / torch.load(weights_only=True), and
    from_state() rejects buffers of the wrong size (host tensors: no GPU)."""
    import torch
    for layout in ("1x32", "32x32", "128x1"):
        d = mg.make_desc(544, 96, 10, 0.6, layout, True, "smoothed")
        p = mg.Plan.empty(d, device="cpu")
        for i, t in enumerate(p.tensors().values()):
            t.view(torch.uint8).view(-1).copy_(torch.arange(t.numel() * t.element_size()) % 251)
        torch.save(p.state(), tmp_path / "p.pt")
        q = mg.Plan.from_state(torch.load(tmp_path / "p.pt", weights_only=True), device="cpu")
        assert [getattr(q.desc, f) for f, _ in mg.mg_plan_desc._fields_] == \
               [getattr(d, f) for f, _ in mg.mg_plan_desc._fields_]
        for n, t in p.tensors().items():
            assert torch.equal(t, getattr(q, n)), n
        bad = p.state()
        bad["tensors"]["Ws"] = bad["tensors"]["Ws"].reshape(-1)[:16]
        with pytest.raises(ValueError):
            mg.Plan.from_state(bad, device="cpu")


def test_binding_checks_shapes_before_any_launch():
    """Every binding entry point compares its tensors with the plan descriptor
    before taking a pointer: a mismatched X, Y, W, act or statistic raises
    ValueError (host tensors here, so no GPU call could be reached)."""
    import torch
    d = mg.make_desc(64, 96, 4, 0.5)
    p = mg.Plan.empty(d, device="cpu")
    a = mg.Act.empty(d, 8, device="cpu")
    X = torch.zeros((8, 64), dtype=torch.bfloat16)
    Y = torch.zeros((8, 96), dtype=torch.bfloat16)
    W = torch.zeros((96, 64), dtype=torch.bfloat16)
    v64, v32 = torch.zeros(64), torch.zeros(32)
    cases = [
        lambda: mg.mg_quantize_act(p, torch.zeros((8, 32), dtype=torch.bfloat16), a),      # K mismatch
        lambda: mg.mg_quantize_act(p, torch.zeros((9, 64), dtype=torch.bfloat16), a),      # act.M != M
        lambda: mg.mg_quantize_act(p, torch.zeros(64, dtype=torch.bfloat16), a),           # not 2-D
        lambda: mg.mg_quantize_act(p, X, mg.Act.empty(mg.make_desc(64, 96, 40, 0.5), 8, device="cpu")),
        lambda: mg.mg_quantize_act_stats(p, X, a, v32),                                     # stats of K
        lambda: mg.mg_dual_gemm(p, a, torch.zeros((8, 64), dtype=torch.bfloat16)),         # Y not [M][N]
        lambda: mg.mg_dual_gemm(p, a, torch.zeros((8, 96), dtype=torch.float64)),          # Y dtype
        lambda: mg.mg_dual_gemm(p, mg.Act.empty(mg.make_desc(128, 96, 4, 0.5), 8, device="cpu"), Y),
        lambda: mg.mg_forward(p, X, a, torch.zeros((7, 96), dtype=torch.bfloat16)),
        lambda: mg.mg_forward(p, torch.zeros((8, 64), dtype=torch.bfloat16), mg.Act.empty(d, 4, device="cpu"), Y),
        lambda: mg.mg_gelu_quantize_act(p, torch.zeros((8, 96), dtype=torch.bfloat16), a),
        lambda: mg.mg_gelu_quantize_act(p, torch.zeros((8, 64), dtype=torch.float32), a),
        lambda: mg.mg_fold_pack(p, torch.zeros((64, 96), dtype=torch.bfloat16)),           # W transposed
        lambda: mg.mg_plan_build(p, v64, v64, torch.zeros((96, 32), dtype=torch.bfloat16)),
        lambda: mg.mg_plan_build(p, v32, v64, W),
        lambda: mg.mg_smooth_scales(p, v64, v32),
        lambda: mg.mg_outlier_set(p, v32),
        lambda: mg.mg_calib_act(X, v32),
        lambda: mg.mg_calib_act(X, torch.zeros(64, dtype=torch.float64)),
        lambda: mg.mg_weight_range(W, v32),
        lambda: mg.mg_gelu_tanh_bf16(Y, torch.zeros((8, 95), dtype=torch.bfloat16)),
        lambda: mg.mg_gelu_tanh_bf16(Y, torch.zeros((8, 96), dtype=torch.float32)),
        lambda: mg.Plan(d, *[t for t in list(p.tensors().values())[:-1]], torch.zeros((96, 4), dtype=torch.bfloat16)),
        lambda: mg.mg_pct_select(mg.PctState(64, device="cpu"), 1, 0.5, v32),
    ]
    for i, f in enumerate(cases):
        with pytest.raises(ValueError):
            f()
            pytest.fail(f"case {i} was not rejected")
    # the well-formed calls get past the shape checks and stop only at the
    # host-tensor check of the pointer marshalling
    for f in (lambda: mg.mg_quantize_act(p, X, a), lambda: mg.mg_dual_gemm(p, a, Y),
              lambda: mg.mg_forward(p, X, a, Y), lambda: mg.mg_plan_build(p, v64, v64, W),
              lambda: mg.mg_calib_act(X, v64)):
        with pytest.raises(ValueError, match="device tensor"):
            f()


def test_forward_validates_both_steps_before_launching():
    """mg_forward and mg_forward_noalloc check every argument of both steps
    (including the GEMM's 3 GiB operand limit) before any launch: on this
    GPU-less host an accepted call would fail with a HIP error instead."""
    L = mg.lib()
    p = _plan(K=5120, N=256, k=64)
    a = mg.mg_act(FAKE, FAKE, FAKE)
    big = (3 << 30) // 2560 + 1                    # Aq of this many rows passes 3 GiB
    assert L.mg_forward(ctypes.byref(p), FAKE, 1, big, ctypes.byref(a), FAKE, 1, None) == -5
    assert L.mg_forward(ctypes.byref(p), FAKE, 1, 8, ctypes.byref(a), FAKE, 9, None) == -3
    assert L.mg_forward(ctypes.byref(p), FAKE, 1, 0, None, None, 1, None) == 0          # M == 0: no-op
    # the no-allocation variant: the same checks, then its 64 MiB workspace limit
    assert L.mg_forward_noalloc(None, FAKE, 1, 8, FAKE, 1, None) == -1
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 1, -1, FAKE, 1, None) == -2
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 7, 8, FAKE, 1, None) == -3
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 1, 8, None, 1, None) == -1
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE + 4, 1, 8, FAKE, 1, None) == -4
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 1, 0, FAKE, 1, None) == 0
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 1, 24000, FAKE, 1, None) == -5
    assert b"limit" in L.mg_last_error()
    assert L.mg_forward_noalloc(ctypes.byref(p), FAKE, 1, big, FAKE, 1, None) == -5


def test_gemm_gelu_quant_validates_before_launching():
    """mg_dual_gemm_gelu_quant checks both plans, both workspaces, the chained
    widths (the next layer's K = this layer's N) and both layers' operand
    limits before any launch (an accepted call would fail with a HIP error on
    this GPU-less host)."""
    L = mg.lib()
    p0 = _plan(K=5120, N=256, k=64)
    p2 = _plan(K=256, N=128, k=8)
    bad = _plan(K=512, N=128, k=8)
    a = mg.mg_act(FAKE, FAKE, FAKE)
    call = lambda q0, a0, M, q2, a2: L.mg_dual_gemm_gelu_quant(q0, a0, M, q2, a2, None)
    r = ctypes.byref
    assert call(None, r(a), 8, r(p2), r(a), ) == -1
    assert call(r(p0), r(a), 8, None, r(a)) == -1
    assert call(r(p0), r(a), 8, r(bad), r(a)) == -2
    assert b"equal" in L.mg_last_error()
    assert call(r(p0), r(a), -1, r(p2), r(a)) == -2
    assert call(r(p0), r(a), 0, r(p2), r(a)) == 0                    # M == 0: no-op
    assert call(r(p0), None, 8, r(p2), r(a)) == -1
    assert call(r(p0), r(a), 8, r(p2), None) == -1
    assert call(r(p0), r(a), 8, r(p2), r(mg.mg_act(FAKE, None, FAKE))) == -1
    big = (3 << 30) // 2560 + 1
    assert call(r(p0), r(a), big, r(p2), r(a)) == -5
