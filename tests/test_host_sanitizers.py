"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only). A host-only copy of the library (the host sources built by g++,
kernel launchers stubbed; hybrid_sliding_window_gqa_amd/build.py
build_host_sanitized) runs the host-side test files in a child process:
argument validation and workspace sizing (test_abi_cpu), window_safe_match
(test_window_safe_cpu) and the pointer-heavy prefix tree (test_prefix_tree_cpu,
test_prefix_cache_golden). Any sanitizer report aborts the child, which fails
this test. The probe entry points and the export list belong to the GPU
library only and are deselected."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
import hybrid_sliding_window_gqa_amd._lib as lib
lib.LIB_PATH = sys.argv[1]
import pytest
sys.exit(pytest.main(sys.argv[2:]))
"""


def _runtime(name):
    out = subprocess.run(["g++", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


@pytest.mark.timeout(600)
def test_host_code_is_clean_under_asan_and_ubsan():
    asan = _runtime("libasan.so")
    if asan is None:
        pytest.skip("g++ has no AddressSanitizer runtime")
    from hybrid_sliding_window_gqa_amd import build

    lib_path = build.build_host_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=asan, ASAN_OPTIONS="detect_leaks=0:detect_odr_violation=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", PYTHONPATH=ROOT)
    files = ["tests/test_abi_cpu.py", "tests/test_window_safe_cpu.py", "tests/test_prefix_tree_cpu.py",
             "tests/test_prefix_cache_golden.py"]
    res = subprocess.run([sys.executable, "-c", CHILD, lib_path, *files, "-q", "-m", "not gpu", "-p",
                          "no:cacheprovider", "-k", "not probe and not exports"],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=540)
    tail = (res.stdout + res.stderr)[-4000:]
    assert res.returncode == 0, tail
    assert "ERROR: AddressSanitizer" not in tail and "runtime error:" not in tail, tail
    assert " passed" in res.stdout, tail
