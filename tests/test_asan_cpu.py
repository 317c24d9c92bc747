"""The host-side validation tests again, against the library built with AddressSanitizer on its
host code (lib/libattn_gqa_asan.so, loaded through ATTN_GQA_LIBRARY with the clang ASan runtime
preloaded into a fresh interpreter): every argument check, size computation and status path of
the C ABI runs under ASan. No GPU is used (every call fails validation or is a pure host query)."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
VALIDATION_TESTS = ["tests/test_api_cpu.py", "tests/test_binding_cpu.py", "tests/test_zz_no_alloc.py"]


def test_validation_tests_under_asan():
    sys.path.insert(0, ROOT)
    from attention_gqa_flash_02_amd import build

    runtime = build.asan_runtime()
    if runtime is None:
        pytest.skip("no clang AddressSanitizer runtime next to hipcc")
    if not os.path.exists(build.LIB_ASAN):
        build.build_asan()
    env = dict(os.environ, LD_PRELOAD=runtime, ATTN_GQA_LIBRARY=build.LIB_ASAN,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0")
    probe = subprocess.run([sys.executable, "-c", "from attention_gqa_flash_02_amd import _lib; print(_lib.load()._name)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert probe.returncode == 0 and probe.stdout.strip() == build.LIB_ASAN, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                        *VALIDATION_TESTS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out
