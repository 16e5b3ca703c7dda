"""Python binding of libmixed_gemm (the smoothed, outlier-split, dual-branch
W4A4 linear layer of "W4A4 Quantization for Inference on Wan2.2-I2V-A14B" on
MI355X / gfx950).

Argument marshalling only: every function below has the name of the C entry
point it calls (``include/mixed_gemm.h``), takes torch tensors for the device
buffers, and passes their data pointers and torch's current HIP stream.  Every
step of the layer runs in the library's HIP kernels; there is no fallback.
If the library is not built this module raises on first use.

bf16 data travels in ``torch.bfloat16`` (or 16-bit integer) tensors.
"""
from __future__ import annotations

import ctypes
import functools
import inspect
import os
from dataclasses import dataclass

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
# MIXED_GEMM_LIB may name another build of the library (for example the
# 4-wave GEMM variant, `python -m mixed_gemm_amd.build --gemm-waves 4`)
LIB_PATH = os.environ.get("MIXED_GEMM_LIB") or os.path.join(HERE, "libmixed_gemm.so")

MG_F32, MG_BF16 = 0, 1
MG_W_1X32, MG_W_32X32, MG_W_128X1 = 0, 1, 2
LAYOUTS = {"1x32": MG_W_1X32, "32x32": MG_W_32X32, "128x1": MG_W_128X1}
MG_SCORE_MAX, MG_SCORE_SMOOTHED = 0, 1
SCORES = {"max": MG_SCORE_MAX, "smoothed": MG_SCORE_SMOOTHED}

STATUS = {0: "MG_OK", -1: "MG_ERR_ARG", -2: "MG_ERR_SHAPE", -3: "MG_ERR_DTYPE", -4: "MG_ERR_ALIGN",
          -5: "MG_ERR_UNSUPPORTED", -6: "MG_ERR_HIP"}


class MGError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


class mg_plan_desc(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int32), ("N", ctypes.c_int32), ("k", ctypes.c_int32),
                ("layout", ctypes.c_int32), ("smooth", ctypes.c_int32), ("score", ctypes.c_int32),
                ("alpha", ctypes.c_double)]


class mg_plan(ctypes.Structure):
    _fields_ = [("d", mg_plan_desc), ("s", ctypes.c_void_p), ("rcp", ctypes.c_void_p),
                ("O", ctypes.c_void_p), ("pos", ctypes.c_void_p), ("Wq", ctypes.c_void_p),
                ("Ws", ctypes.c_void_p), ("Wst", ctypes.c_void_p), ("WO", ctypes.c_void_p)]


class mg_act(ctypes.Structure):
    _fields_ = [("Aq", ctypes.c_void_p), ("As", ctypes.c_void_p), ("XO", ctypes.c_void_p)]


class mg_pct(ctypes.Structure):
    _fields_ = [("hist", ctypes.c_void_p), ("sel", ctypes.c_void_p), ("K", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


EXPORTS = ("mg_version", "mg_last_error", "mg_plan_bytes", "mg_act_bytes", "mg_calib_reset",
           "mg_calib_act", "mg_weight_range", "mg_smooth_scales", "mg_outlier_set", "mg_fold_pack",
           "mg_plan_build", "mg_quantize_act", "mg_dual_gemm", "mg_forward", "mg_gelu_tanh_bf16",
           "mg_gelu_quantize_act", "mg_pct_reset", "mg_pct_count", "mg_pct_select", "mg_quantize_act_stats",
           "mg_forward_noalloc", "mg_dual_gemm_gelu_quant")

_lib = None


def lib() -> ctypes.CDLL:
    """Load libmixed_gemm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -m mixed_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        P = ctypes.POINTER
        sig = {
            "mg_version": ([], ctypes.c_int),
            "mg_last_error": ([], ctypes.c_char_p),
            "mg_plan_bytes": ([P(mg_plan_desc), P(sz)], ctypes.c_int),
            "mg_act_bytes": ([P(mg_plan_desc), i64, P(sz)], ctypes.c_int),
            "mg_calib_reset": ([vp, i32, vp], ctypes.c_int),
            "mg_calib_act": ([vp, i32, i64, i32, vp, vp], ctypes.c_int),
            "mg_weight_range": ([vp, i32, i32, i32, vp, vp], ctypes.c_int),
            "mg_smooth_scales": ([P(mg_plan), vp, vp, vp], ctypes.c_int),
            "mg_outlier_set": ([P(mg_plan), vp, vp], ctypes.c_int),
            "mg_fold_pack": ([P(mg_plan), vp, i32, vp], ctypes.c_int),
            "mg_plan_build": ([P(mg_plan), vp, vp, vp, i32, vp], ctypes.c_int),
            "mg_quantize_act": ([P(mg_plan), vp, i32, i64, P(mg_act), vp], ctypes.c_int),
            "mg_dual_gemm": ([P(mg_plan), P(mg_act), i64, vp, i32, vp], ctypes.c_int),
            "mg_forward": ([P(mg_plan), vp, i32, i64, P(mg_act), vp, i32, vp], ctypes.c_int),
            "mg_forward_noalloc": ([P(mg_plan), vp, i32, i64, vp, i32, vp], ctypes.c_int),
            "mg_gelu_tanh_bf16": ([vp, vp, i64, vp], ctypes.c_int),
            "mg_gelu_quantize_act": ([P(mg_plan), vp, i64, P(mg_act), vp], ctypes.c_int),
            "mg_dual_gemm_gelu_quant": ([P(mg_plan), P(mg_act), i64, P(mg_plan), P(mg_act), vp], ctypes.c_int),
            "mg_quantize_act_stats": ([P(mg_plan), vp, i32, i64, P(mg_act), vp, vp], ctypes.c_int),
            "mg_pct_reset": ([P(mg_pct), vp], ctypes.c_int),
            "mg_pct_count": ([P(mg_pct), i32, vp, i64, vp], ctypes.c_int),
            "mg_pct_select": ([P(mg_pct), i32, ctypes.c_double, vp, vp], ctypes.c_int),
        }
        missing = set(EXPORTS) - set(sig)
        if missing:                       # an undeclared signature would truncate 64-bit pointers
            raise RuntimeError(f"no ctypes signature for {sorted(missing)}")
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def _check(code: int) -> None:
    if code != 0:
        raise MGError(code, lib().mg_last_error().decode())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _on_stream(fn):
    """Run a helper that allocates temporaries with torch's current stream set
    to its `stream` argument (a torch stream or a raw hipStream_t handle), so
    the caching allocator ties them to the stream whose kernels use them: a
    block freed on another stream could be handed out again while those
    kernels still read it."""
    sig = inspect.signature(fn)

    @functools.wraps(fn)
    def wrap(*args, **kwargs):
        stream = sig.bind(*args, **kwargs).arguments.get("stream")
        if stream is None:
            return fn(*args, **kwargs)
        if not isinstance(stream, torch.cuda.Stream):
            stream = torch.cuda.ExternalStream(int(stream))
        with torch.cuda.stream(stream):
            return fn(*args, **kwargs)
    return wrap


def _ptr(t: torch.Tensor | None) -> int | None:
    if t is None or t.numel() == 0:
        return None
    if not t.is_cuda:
        raise ValueError("device tensor expected")
    if not t.is_contiguous():
        raise ValueError("contiguous tensor expected")
    return t.data_ptr()


def _dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MG_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return MG_BF16
    raise ValueError(f"unsupported dtype {t.dtype}")


# The C ABI receives bare pointers and cannot know buffer sizes, so the binding
# checks every shape against the plan descriptor before anything is launched
# (a mismatched buffer would make a kernel read or write past its allocation).

def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _is_bf16(t: torch.Tensor) -> bool:
    return t.dtype in (torch.bfloat16, torch.int16, torch.uint16)


def _matrix(X: torch.Tensor, name: str, cols: int | None = None) -> tuple[int, int]:
    _need(X.dim() == 2, f"{name} must be 2-D, got shape {tuple(X.shape)}")
    if cols is not None:
        _need(X.shape[1] == cols, f"{name} must have {cols} columns, got shape {tuple(X.shape)}")
    return int(X.shape[0]), int(X.shape[1])


def _vec(t: torch.Tensor, n: int, name: str) -> None:
    _need(t is not None and t.numel() == n and t.dtype == torch.float32,
          f"{name} must be a float32 tensor of {n} elements")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check_act(desc, act: "Act", M: int | None = None) -> None:
    _need(isinstance(act, Act), "act must be an Act")
    if M is not None:
        _need(act.M == M, f"act holds {act.M} rows, the input has {M}")
    want = mg_act_bytes(desc, act.M)
    got = [_nbytes(act.Aq), _nbytes(act.As), _nbytes(act.XO)]
    _need(got == want, f"act buffers {got} bytes do not match the plan's sizes {want} for M={act.M}")
    _need(tuple(act.Aq.shape) == frag_shape(act.M, desc.K // 2), f"act.Aq must have shape {frag_shape(act.M, desc.K // 2)}")


def _check_y(desc, Y: torch.Tensor, M: int) -> None:
    _need(Y.dim() == 2 and tuple(Y.shape) == (M, desc.N), f"Y must be [{M}][{desc.N}], got {tuple(Y.shape)}")
    _need(Y.dtype == torch.float32 or _is_bf16(Y), f"Y must be bf16 or float32, got {Y.dtype}")


# ----------------------------------------------------------------------------- plan / workspace

def make_desc(K: int, N: int, k: int, alpha: float = 0.5, layout: str | int = "1x32",
              smooth: bool = True, score: str | int = "max") -> mg_plan_desc:
    lay = LAYOUTS[layout] if isinstance(layout, str) else int(layout)
    sc = SCORES[score] if isinstance(score, str) else int(score)
    return mg_plan_desc(int(K), int(N), int(k), lay, int(bool(smooth)), sc, float(alpha))


def mg_plan_bytes(desc: mg_plan_desc) -> list[int]:
    out = (ctypes.c_size_t * 8)()
    _check(lib().mg_plan_bytes(ctypes.byref(desc), out))
    return list(out)


def mg_act_bytes(desc: mg_plan_desc, M: int) -> list[int]:
    out = (ctypes.c_size_t * 3)()
    _check(lib().mg_act_bytes(ctypes.byref(desc), int(M), out))
    return list(out)


def frag_shape(rows: int, row_bytes: int) -> tuple:
    """Shape of an operand stored in fragment order (Aq, Wq: row_bytes = K/2;
    XO, WO: row_bytes = 2k), as bytes: [ceil(rows/32)][2 ceil(row_bytes/64)][1024]
    (the C header's fragment order: 1 KB blocks of 32 rows x 32 bytes, an even
    number of 32-byte slices per row)."""
    return (-(-rows // 32), 2 * -(-row_bytes // 64), 1024)


def scale_shape(rows: int, K: int) -> tuple:
    """Shape of a scale array (As, Ws) for `rows` rows in its stored order:
    [ceil(rows/256)][ceil(K/512)][256 rows][16 blocks] (the C header's scale
    windows)."""
    return (-(-rows // 256), -(-K // 512), 256, 16)


@dataclass
class Plan:
    """Device buffers of one layer's plan (allocated with torch from mg_plan_bytes)."""
    desc: mg_plan_desc
    s: torch.Tensor
    rcp: torch.Tensor
    O: torch.Tensor
    pos: torch.Tensor
    Wq: torch.Tensor
    Ws: torch.Tensor
    Wst: torch.Tensor
    WO: torch.Tensor

    def __post_init__(self):
        got = [_nbytes(t) for t in self.tensors().values()]
        want = mg_plan_bytes(self.desc)
        _need(got == want, f"plan buffer sizes {got} differ from mg_plan_bytes {want}")
        _need(self.Wq.dtype == torch.uint8 and tuple(self.Wq.shape) == frag_shape(self.desc.N, self.desc.K // 2),
              "plan.Wq must be uint8 of frag_shape(N, K/2)")

    @staticmethod
    def empty(desc: mg_plan_desc, device="cuda") -> "Plan":
        K, N, k = desc.K, desc.N, desc.k
        e = lambda n, dt: torch.empty(n, dtype=dt, device=device)
        wst = {MG_W_32X32: (N // 32, K // 32), MG_W_128X1: (N, (K + 127) // 128)}.get(desc.layout, 0)
        p = Plan(desc, e(K, torch.float32), e(K, torch.float32), e(k, torch.int32), e(K, torch.int32),
                 e(frag_shape(N, K // 2), torch.uint8), e(scale_shape(N, K), torch.uint8), e(wst, torch.uint8),
                 e(frag_shape(N, 2 * k), torch.uint8))
        return p

    def c(self) -> mg_plan:
        return mg_plan(self.desc, _ptr(self.s), _ptr(self.rcp), _ptr(self.O), _ptr(self.pos), _ptr(self.Wq),
                       _ptr(self.Ws), _ptr(self.Wst), _ptr(self.WO))

    def tensors(self) -> dict:
        return dict(s=self.s, rcp=self.rcp, O=self.O, pos=self.pos, Wq=self.Wq, Ws=self.Ws, Wst=self.Wst,
                    WO=self.WO)

    def state(self) -> dict:
        """The plan as plain data (descriptor fields and tensors) for torch.save;
        a plan holds no other state."""
        d = {f: getattr(self.desc, f) for f, _ in mg_plan_desc._fields_}
        return {"desc": d, "tensors": self.tensors()}

    @staticmethod
    def from_state(state: dict, device="cuda") -> "Plan":
        """A plan from state() (e.g. after torch.load(..., weights_only=True)),
        its buffers checked against mg_plan_bytes."""
        desc = mg_plan_desc(**state["desc"])
        return Plan(desc, **{n: t.to(device) for n, t in state["tensors"].items()})


@dataclass
class Act:
    """Per-forward activation workspace (Aq, As, XO) for M rows."""
    M: int
    Aq: torch.Tensor
    As: torch.Tensor
    XO: torch.Tensor

    @staticmethod
    def empty(desc: mg_plan_desc, M: int, device="cuda") -> "Act":
        K, k = desc.K, desc.k
        a = Act(M, torch.empty(frag_shape(M, K // 2), dtype=torch.uint8, device=device),
                torch.empty(scale_shape(M, K), dtype=torch.uint8, device=device),
                torch.empty(frag_shape(M, 2 * k), dtype=torch.uint8, device=device))
        _check_act(desc, a)
        return a

    def c(self) -> mg_act:
        return mg_act(_ptr(self.Aq), _ptr(self.As), _ptr(self.XO))


# ----------------------------------------------------------------------------- entry points

def mg_version() -> int:
    return lib().mg_version()


def mg_calib_reset(act_max: torch.Tensor, stream=None) -> None:
    _need(act_max.dtype == torch.float32, "act_max must be float32")
    _check(lib().mg_calib_reset(_ptr(act_max), act_max.numel(), _stream(stream)))


def mg_calib_act(X: torch.Tensor, act_max: torch.Tensor, stream=None) -> None:
    M, K = _matrix(X, "X")
    _vec(act_max, K, "act_max")
    _check(lib().mg_calib_act(_ptr(X), _dtype(X), M, K, _ptr(act_max), _stream(stream)))


def mg_weight_range(W: torch.Tensor, w_max: torch.Tensor, stream=None) -> None:
    N, K = _matrix(W, "W")
    _vec(w_max, K, "w_max")
    _check(lib().mg_weight_range(_ptr(W), _dtype(W), N, K, _ptr(w_max), _stream(stream)))


def mg_smooth_scales(plan: Plan, act_max, w_max, stream=None) -> None:
    if plan.desc.smooth:
        _vec(act_max, plan.desc.K, "act_max")
        _vec(w_max, plan.desc.K, "w_max")
    p = plan.c()
    _check(lib().mg_smooth_scales(ctypes.byref(p), _ptr(act_max), _ptr(w_max), _stream(stream)))


def mg_outlier_set(plan: Plan, act_max, stream=None) -> None:
    _vec(act_max, plan.desc.K, "score")
    p = plan.c()
    _check(lib().mg_outlier_set(ctypes.byref(p), _ptr(act_max), _stream(stream)))


def mg_fold_pack(plan: Plan, W: torch.Tensor, stream=None) -> None:
    _need(tuple(W.shape) == (plan.desc.N, plan.desc.K), f"W must be [{plan.desc.N}][{plan.desc.K}]")
    p = plan.c()
    _check(lib().mg_fold_pack(ctypes.byref(p), _ptr(W), _dtype(W), _stream(stream)))


def mg_plan_build(plan: Plan, act_max, w_max, W: torch.Tensor, stream=None) -> None:
    _vec(act_max, plan.desc.K, "act_max")
    if plan.desc.smooth:
        _vec(w_max, plan.desc.K, "w_max")
    _need(tuple(W.shape) == (plan.desc.N, plan.desc.K), f"W must be [{plan.desc.N}][{plan.desc.K}]")
    p = plan.c()
    _check(lib().mg_plan_build(ctypes.byref(p), _ptr(act_max), _ptr(w_max), _ptr(W), _dtype(W),
                               _stream(stream)))


def mg_quantize_act(plan: Plan, X: torch.Tensor, act: Act, stream=None) -> None:
    M, _ = _matrix(X, "X", plan.desc.K)
    _check_act(plan.desc, act, M)
    p, a = plan.c(), act.c()
    _check(lib().mg_quantize_act(ctypes.byref(p), _ptr(X), _dtype(X), X.shape[0], ctypes.byref(a),
                                 _stream(stream)))


def mg_dual_gemm(plan: Plan, act: Act, Y: torch.Tensor, stream=None) -> None:
    _check_act(plan.desc, act)
    _check_y(plan.desc, Y, act.M)
    p, a = plan.c(), act.c()
    _check(lib().mg_dual_gemm(ctypes.byref(p), ctypes.byref(a), act.M, _ptr(Y), _dtype(Y), _stream(stream)))


def mg_forward(plan: Plan, X: torch.Tensor, act: Act, Y: torch.Tensor, stream=None) -> None:
    M, _ = _matrix(X, "X", plan.desc.K)
    _check_act(plan.desc, act, M)
    _check_y(plan.desc, Y, M)
    p, a = plan.c(), act.c()
    _check(lib().mg_forward(ctypes.byref(p), _ptr(X), _dtype(X), X.shape[0], ctypes.byref(a), _ptr(Y),
                            _dtype(Y), _stream(stream)))


def mg_forward_noalloc(plan: Plan, X: torch.Tensor, Y: torch.Tensor, stream=None) -> None:
    """mg_forward with the library's own per-GPU workspace (no Act; see the
    header for the size limit and the sharing rule)."""
    M, _ = _matrix(X, "X", plan.desc.K)
    _check_y(plan.desc, Y, M)
    p = plan.c()
    _check(lib().mg_forward_noalloc(ctypes.byref(p), _ptr(X), _dtype(X), M, _ptr(Y), _dtype(Y), _stream(stream)))


def mg_gelu_tanh_bf16(inp: torch.Tensor, out: torch.Tensor, stream=None) -> None:
    _need(_is_bf16(inp) and _is_bf16(out), "bf16 input and output expected")
    _need(out.numel() == inp.numel(), f"out holds {out.numel()} values, in {inp.numel()}")
    _check(lib().mg_gelu_tanh_bf16(_ptr(inp), _ptr(out), inp.numel(), _stream(stream)))


def mg_quantize_act_stats(plan: Plan, X: torch.Tensor, act: Act, act_max: torch.Tensor, stream=None) -> None:
    M, _ = _matrix(X, "X", plan.desc.K)
    _check_act(plan.desc, act, M)
    _vec(act_max, plan.desc.K, "act_max")
    p, a = plan.c(), act.c()
    _check(lib().mg_quantize_act_stats(ctypes.byref(p), _ptr(X), _dtype(X), X.shape[0], ctypes.byref(a),
                                       _ptr(act_max), _stream(stream)))


def mg_gelu_quantize_act(plan: Plan, Y: torch.Tensor, act: Act, stream=None) -> None:
    _need(_is_bf16(Y), "bf16 input expected")
    M, _ = _matrix(Y, "Y", plan.desc.K)
    _check_act(plan.desc, act, M)
    p, a = plan.c(), act.c()
    _check(lib().mg_gelu_quantize_act(ctypes.byref(p), _ptr(Y), Y.shape[0], ctypes.byref(a), _stream(stream)))


def mg_dual_gemm_gelu_quant(plan0: Plan, act0: Act, plan2: Plan, act2: Act, stream=None) -> None:
    """plan0's dual GEMM whose epilogue applies GELU to the bf16 output and
    quantizes it for plan2 into act2 (the output itself is never written)."""
    _need(plan2.desc.K == plan0.desc.N, f"plan2's K={plan2.desc.K} must equal plan0's N={plan0.desc.N}")
    _check_act(plan0.desc, act0)
    _check_act(plan2.desc, act2, act0.M)
    p0, a0, p2, a2 = plan0.c(), act0.c(), plan2.c(), act2.c()
    _check(lib().mg_dual_gemm_gelu_quant(ctypes.byref(p0), ctypes.byref(a0), act0.M, ctypes.byref(p2),
                                         ctypes.byref(a2), _stream(stream)))


class PctState:
    """Device state of one percentile calibration run: hist [K][256] u32
    counts (stored as int32) and sel [K][2] (selected high byte, rank)."""

    def __init__(self, K: int, device="cuda"):
        self.K = K
        self.hist = torch.empty((K, 256), dtype=torch.int32, device=device)
        self.sel = torch.empty((K, 2), dtype=torch.int32, device=device)

    def c(self) -> mg_pct:
        return mg_pct(_ptr(self.hist), _ptr(self.sel), self.K, 0)


def mg_pct_reset(st: PctState, stream=None) -> None:
    c = st.c()
    _check(lib().mg_pct_reset(ctypes.byref(c), _stream(stream)))


def mg_pct_count(st: PctState, pass_: int, X: torch.Tensor, stream=None) -> None:
    if X.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError("bf16 input expected")
    if X.dim() != 2 or X.shape[1] != st.K:
        raise ValueError(f"X must be [M][{st.K}]")
    c = st.c()
    _check(lib().mg_pct_count(ctypes.byref(c), pass_, _ptr(X), X.shape[0], _stream(stream)))


def mg_pct_select(st: PctState, pass_: int, q: float, score: torch.Tensor | None = None, stream=None) -> None:
    if score is not None:
        _vec(score, st.K, "score")
    c = st.c()
    _check(lib().mg_pct_select(ctypes.byref(c), pass_, float(q), _ptr(score), _stream(stream)))


# ----------------------------------------------------------------------------- convenience

@_on_stream
def percentile(batches, K: int, q: float, device="cuda", stream=None) -> torch.Tensor:
    """Per-channel nearest-rank q-quantile of |x| over all rows of the given
    [M][K] bf16 device tensors (two passes over the batches)."""
    batches = list(batches)
    st = PctState(K, device)
    score = torch.empty(K, dtype=torch.float32, device=device)
    mg_pct_reset(st, stream)
    for X in batches:
        mg_pct_count(st, 0, X, stream)
    mg_pct_select(st, 0, q, None, stream)
    for X in batches:
        mg_pct_count(st, 1, X, stream)
    mg_pct_select(st, 1, q, score, stream)
    return score


@_on_stream
def calibrate(batches, K: int, device="cuda", stream=None) -> torch.Tensor:
    """Running per-channel activation maxima over an iterable of [M][K] device tensors."""
    act_max = torch.empty(K, dtype=torch.float32, device=device)
    mg_calib_reset(act_max, stream)
    for X in batches:
        mg_calib_act(X, act_max, stream)
    return act_max


@_on_stream
def plan(act_max: torch.Tensor, W: torch.Tensor, alpha: float, k: int, layout: str = "1x32",
         smooth: bool = True, stream=None, score: str = "max", rank: torch.Tensor | None = None) -> Plan:
    """calibrated maxima + weights -> a built plan (weight ranges, Eq. (2), Eq. (4), fold + pack).
    Eq. (4) ranks act_max, or the per-channel statistic ``rank`` when given (e.g. percentile())."""
    N, K = W.shape
    desc = make_desc(K, N, k, alpha, layout, smooth, score)
    p = Plan.empty(desc, W.device)
    w_max = torch.empty(K, dtype=torch.float32, device=W.device)
    mg_weight_range(W, w_max, stream)
    if rank is None:
        mg_plan_build(p, act_max, w_max, W, stream)
    else:
        mg_smooth_scales(p, act_max, w_max, stream)
        mg_outlier_set(p, rank, stream)
        mg_fold_pack(p, W, stream)
    return p


@_on_stream
def forward(p: Plan, X: torch.Tensor, act: Act | None = None, Y: torch.Tensor | None = None,
            stream=None) -> torch.Tensor:
    M = X.shape[0]
    if act is None or act.M != M:
        act = Act.empty(p.desc, M, X.device)
    if Y is None:
        Y = torch.empty((M, p.desc.N), dtype=torch.bfloat16, device=X.device)
    mg_forward(p, X, act, Y, stream)
    return Y


@_on_stream
def reference_plan(W: torch.Tensor, stream=None) -> Plan:
    """A plan that routes every channel through the bf16 branch with no
    smoothing (k = K, s = 1): forward() then computes the plain bf16 GEMM
    X W^T with fp32 accumulation -- the unquantized layer."""
    N, K = W.shape
    act_max = torch.ones(K, dtype=torch.float32, device=W.device)
    return plan(act_max, W, 0.5, K, "1x32", smooth=False, stream=stream)


class DynamicRouter:
    """Per-step outlier routing by prediction (MixQ's quantization ahead of
    detection; the pages name its port to diffusion steps as future work).

    The smoothing scales s are fixed from the offline calibration maxima, and
    the first step routes the calibrated top-k set.  Each step quantizes its
    batch with the current plan while recording the batch's per-channel
    maxima (mg_quantize_act_stats, one pass), runs the dual GEMM, and -- on a
    side stream, overlapping the GEMM -- builds the next step's plan from
    those maxima (Eq. (4) top-k, then fold and pack) into the other of two
    plan buffers.  Step t's outlier set is therefore Eq. (4) applied to the
    maxima of step t-1's batch."""

    def __init__(self, W: torch.Tensor, act_max_calib: torch.Tensor, alpha: float, k: int,
                 layout: str = "1x32", smooth: bool = True, score: str = "max"):
        N, K = W.shape
        self.W = W
        self.desc = make_desc(K, N, k, alpha, layout, smooth, score)
        self.plans = [Plan.empty(self.desc, W.device), Plan.empty(self.desc, W.device)]
        w_max = torch.empty(K, dtype=torch.float32, device=W.device)
        mg_weight_range(W, w_max)
        for p in self.plans:
            mg_smooth_scales(p, act_max_calib, w_max)
        mg_outlier_set(self.plans[0], act_max_calib)
        mg_fold_pack(self.plans[0], W)
        self.cur = 0
        self.stats = torch.empty(K, dtype=torch.float32, device=W.device)
        self.side = torch.cuda.Stream(device=W.device)
        self.ready = None                      # event: the current plan is built

    def step(self, X: torch.Tensor, act: Act | None = None, Y: torch.Tensor | None = None) -> torch.Tensor:
        main = torch.cuda.current_stream()
        M = X.shape[0]
        act = act if act is not None else Act.empty(self.desc, M, X.device)
        if Y is None:
            Y = torch.empty((M, self.desc.N), dtype=torch.bfloat16, device=X.device)
        if self.ready is not None:
            main.wait_event(self.ready)       # this step's plan, and the last read of stats
        p = self.plans[self.cur]
        mg_calib_reset(self.stats, main)
        mg_quantize_act_stats(p, X, act, self.stats, main)
        detected = torch.cuda.Event()
        detected.record(main)                  # also orders after the previous GEMM (which read the other plan)
        mg_dual_gemm(p, act, Y, main)
        nxt = self.plans[self.cur ^ 1]
        self.side.wait_event(detected)
        mg_outlier_set(nxt, self.stats, self.side)
        mg_fold_pack(nxt, self.W, self.side)
        self.ready = torch.cuda.Event()
        self.ready.record(self.side)
        self.cur ^= 1
        return Y


@dataclass
class FFNBlock:
    """ffn.0 -> GELU-tanh -> ffn.2 with one plan per projection."""
    plan0: Plan
    plan2: Plan


@_on_stream
def ffn_block_stats(calib_batches, W0: torch.Tensor, on_hidden=None, stream=None):
    """Calibration statistics of both projections of an FFN block from the
    same batches: ffn.0's from the batches themselves, ffn.2's from the
    unquantized block's hidden activations h = bf16(gelu(bf16(X W0^T))).
    `calib_batches` is an iterable of [M][K0] device tensors; `on_hidden(h)`,
    if given, sees each batch's h.  Returns (act_max0, act_max2)."""
    K0, N0 = W0.shape[1], W0.shape[0]
    act0 = torch.empty(K0, dtype=torch.float32, device=W0.device)
    act2 = torch.empty(N0, dtype=torch.float32, device=W0.device)
    mg_calib_reset(act0, stream)
    mg_calib_reset(act2, stream)
    ref0 = reference_plan(W0, stream)
    act = y = h = None
    for X in calib_batches:
        mg_calib_act(X, act0, stream)
        if act is None or act.M != X.shape[0]:
            act = Act.empty(ref0.desc, X.shape[0], X.device)
            y = torch.empty((X.shape[0], N0), dtype=torch.bfloat16, device=X.device)
            h = torch.empty_like(y)
        mg_forward(ref0, X, act, y, stream)
        mg_gelu_tanh_bf16(y, h, stream)
        mg_calib_act(h, act2, stream)
        if on_hidden is not None:
            on_hidden(h)
    return act0, act2


@_on_stream
def ffn_block_plans(act0: torch.Tensor, act2: torch.Tensor, W0: torch.Tensor, W2: torch.Tensor,
                    alpha0: float, k0: int, alpha2: float, k2: int, layout: str = "1x32",
                    stream=None) -> FFNBlock:
    return FFNBlock(plan(act0, W0, alpha0, k0, layout, stream=stream),
                    plan(act2, W2, alpha2, k2, layout, stream=stream))


@_on_stream
def ffn_block_forward(blk: FFNBlock, X: torch.Tensor, stream=None, epilogue: bool = False) -> torch.Tensor:
    """Y2 = ffn.2(gelu(ffn.0(X))): ffn.0's forward, then GELU and ffn.2's
    activation quantization in one pass (mg_gelu_quantize_act), then ffn.2's
    dual GEMM; with epilogue=True the GELU and ffn.2's quantization run inside
    ffn.0's GEMM epilogue (mg_dual_gemm_gelu_quant) and ffn.0's output is
    never written.  Both give the same bits."""
    a2 = Act.empty(blk.plan2.desc, X.shape[0], X.device)
    if epilogue:
        a0 = Act.empty(blk.plan0.desc, X.shape[0], X.device)
        mg_quantize_act(blk.plan0, X, a0, stream)
        mg_dual_gemm_gelu_quant(blk.plan0, a0, blk.plan2, a2, stream)
        del a0
    else:
        y0 = forward(blk.plan0, X, stream=stream)
        mg_gelu_quantize_act(blk.plan2, y0, a2, stream)
        del y0
    y2 = torch.empty((X.shape[0], blk.plan2.desc.N), dtype=torch.bfloat16, device=X.device)
    mg_dual_gemm(blk.plan2, a2, y2, stream)
    return y2
