"""The C ABI used from C: tests/c/abi_demo.c (built by mixed_gemm_amd/build.py
as an executable and as libabi_demo.so) calibrates on two batches, builds the
weight ranges and the plan, and runs the forward (bf16 and fp32 outputs),
every call made from C through include/mixed_gemm.h with the HIP runtime for
memory; it writes every input and artefact to a file.  Here its entry point
runs in this process, and the file is checked against the oracle: bit for
bit for the statistics, plan and codes, the output within 2e-3 (fp32) and one
RNE (bf16)."""
import ctypes
import os

import numpy as np
import pytest

from oracle import layer
from tests.gpu_util import aq_rows, check_output, outlier_cols, scale_rows

pytestmark = pytest.mark.gpu

SO = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "libabi_demo.so")


def _read(path):
    blobs = {}
    with open(path, "rb") as f:
        while True:
            tag = f.read(16)
            if not tag:
                break
            n = int.from_bytes(f.read(8), "little")
            blobs[tag.rstrip(b"\0").decode()] = f.read(n)
    return blobs


def test_c_program_matches_oracle(tmp_path):
    assert os.path.exists(SO), "tests/c/libabi_demo.so is not built (python -m mixed_gemm_amd.build)"
    demo = ctypes.CDLL(SO)
    demo.abi_demo_run.argtypes = [ctypes.c_char_p]
    demo.abi_demo_run.restype = ctypes.c_int
    out = tmp_path / "abi.bin"
    print("\n[c-abi] abi_demo_run", flush=True)
    assert demo.abi_demo_run(str(out).encode()) == 0
    b = _read(out)
    M, K, N, k = (int(v) for v in np.frombuffer(b["dims"], np.int32))

    def arr(name, dt, shape):
        return np.frombuffer(b[name], dt).reshape(shape)

    X, W = arr("X", np.uint16, (M, K)), arr("W", np.uint16, (N, K))
    a = layer.act_max(X[:100], layer.act_max(X[100:]))          # the same two batches
    w = layer.weight_range(W)
    p = layer.plan(a, w, W, 0.6, k)
    qa = layer.quantize_act(X, p["s"], p["O"])
    want = dict(act_max=a, w_max=w, s=p["s"], rcp=p["rcp"], O=p["O"], pos=p["pos"], Wq=p["Wq"], Ws=p["Ws"],
                WO=p["WO"], Aq=qa["Aq"], As=qa["As"], XO=qa["XO"])
    for name, ref in want.items():
        ref = np.ascontiguousarray(ref)
        got = np.frombuffer(b[name], np.uint8)
        if name in ("As", "Ws"):                                     # stored in scale windows
            got = scale_rows(got, M if name == "As" else N, K)
        elif name in ("Aq", "Wq"):                                   # fragment order
            got = aq_rows(got, M if name == "Aq" else N, K)
        elif name in ("XO", "WO"):                                   # fragment order, rows of 2k bytes
            got = outlier_cols(got, M if name == "XO" else N, k).view(np.uint8)
        assert got.size == ref.nbytes and np.array_equal(got.ravel(), ref.view(np.uint8).ravel()), name
    assert len(b["Wst"]) == 0
    Y64 = layer.dual_gemm_f64(qa["Aq"], qa["As"], p["Wq"], p["Ws"], qa["XO"], p["WO"])
    check_output(arr("Y", np.uint16, (M, N)), arr("Y32", np.float32, (M, N)), Y64, 2e-3)
