"""Host-side build and measurement helpers (CPU only): the library override
the binding honours, the build's wave-count option, and the code hash that
keys the stored GEMM traffic counters to the kernel's code."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_code_hash_ignores_comments_and_layout_only():
    b = _bench()
    src = 'int f(int a) {\n  // say "hi"\n  return a + 1; /* one */\n}\nconst char* s = "a // b";\n'
    same = 'int f(int a) { return a + 1;\n}\n/* a block\n comment */ const char* s = "a // b";'
    assert b._code_only(src) == b._code_only(same)
    assert "a // b" in b._code_only(src)                      # string literals are kept whole
    assert b._code_only(src) != b._code_only(src.replace("a + 1", "a + 2"))
    assert b._code_only("char c = '/'; // x\nint y;") == "char c = '/'; int y;"


def test_stored_traffic_matches_the_current_gemm_code():
    """The committed counter summary belongs to the GEMM code in the tree
    (otherwise the bench reports traffic as unmeasured)."""
    b = _bench()
    assert b.measured_traffic() is not None


def test_library_override_from_the_environment(tmp_path):
    lib = tmp_path / "libother.so"
    code = ("import mixed_gemm_amd as mg; print(mg.LIB_PATH)\n"
            "try:\n    mg.lib()\nexcept RuntimeError as e:\n    print('raised', 'not built' in str(e))\n")
    env = dict(os.environ, MIXED_GEMM_LIB=str(lib))
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                         check=True).stdout.split("\n")
    assert out[0] == str(lib)
    assert out[1] == "raised True"                            # a missing override fails loudly


def test_gemm_wave_option_is_checked():
    from mixed_gemm_amd import build
    with pytest.raises(ValueError):
        build.build_gemm_waves(6)
