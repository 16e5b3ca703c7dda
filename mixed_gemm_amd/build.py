"""Build libmixed_gemm.so (HIP, gfx950) in-tree.

    python -m mixed_gemm_amd.build [--gemm-waves 4]

Compiles every ``csrc/*.hip`` with hipcc for gfx950 (one object per file, in
parallel) and links them into ``mixed_gemm_amd/libmixed_gemm.so``; then builds
``tests/c/abi_demo`` (plain C against ``include/mixed_gemm.h``, the library and
the HIP runtime), which a GPU test runs to exercise the C ABI without Python.

``--gemm-waves 4`` builds the dual GEMM with 4 waves per workgroup (one per
SIMD) instead of 8, into ``mixed_gemm_amd/libmixed_gemm_w4.so`` (objects under
``_build/w4``), for comparing the two schedules; the binding loads it when
``MIXED_GEMM_LIB`` names it.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libmixed_gemm.so")

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    # keep the compiler from emitting packed-fp32 VALU ops (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build mixed_gemm_amd)")


def _compile(src: str, obj_dir: str = OBJ, defines: tuple = ()) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *defines, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs, LIB)
    if verbose:
        print(f"built {LIB}")
    demo = build_c_demo()
    if verbose:
        print(f"built {demo}")
    return LIB


def build_c_demo() -> str:
    """tests/c/abi_demo (executable) and tests/c/libabi_demo.so (the same
    program's abi_demo_run() for in-process use): C99, host code only (no
    kernels), linked against the in-tree library (found next to it at run time
    through an $ORIGIN rpath)."""
    src = os.path.join(ROOT, "tests", "c", "abi_demo.c")
    exe = os.path.join(ROOT, "tests", "c", "abi_demo")
    so = os.path.join(ROOT, "tests", "c", "libabi_demo.so")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cc = os.environ.get("CC", "gcc")
    common = ["-std=c99", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
              "-I", os.path.join(rocm, "include"), src,
              "-L", HERE, "-lmixed_gemm", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
              "-Wl,-rpath,$ORIGIN/../../mixed_gemm_amd", "-Wl,-rpath," + os.path.join(rocm, "lib")]
    for target, extra in ((exe, []), (so, ["-DABI_DEMO_LIB", "-shared", "-fPIC"])):
        r = subprocess.run([cc, *extra, *common, "-o", target + ".tmp"], capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"C demo build failed:\n{r.stdout}\n{r.stderr}")
        os.replace(target + ".tmp", target)
    return exe


def build_gemm_waves(waves: int, verbose: bool = False) -> str:
    """The library with the dual GEMM built for `waves` waves per workgroup
    (4 or 8; 8 is the default build), as libmixed_gemm_w<waves>.so."""
    if waves not in (4, 8):
        raise ValueError("the dual GEMM is written for 4 or 8 waves per workgroup")
    obj_dir = os.path.join(OBJ, f"w{waves}")
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    defines = (f"-DMG_GEMM_WAVES={waves}",)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, obj_dir, defines), srcs))
    lib = os.path.join(HERE, f"libmixed_gemm_w{waves}.so")
    _link(objs, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    ap = argparse.ArgumentParser(description="build libmixed_gemm (gfx950) in-tree")
    ap.add_argument("--gemm-waves", type=int, default=0,
                    help="build only a variant library with this many waves per GEMM workgroup (4 or 8)")
    a = ap.parse_args()
    if a.gemm_waves:
        build_gemm_waves(a.gemm_waves, verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
