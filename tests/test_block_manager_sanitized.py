"""The C++ block manager under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/bm_fuzz.cpp drives random operation streams (add, fork, append,
free, swap out / in, batch tables) through the C API of
paged_kv_cache_309_amd/csrc/block_manager.cpp on pools of random sizes,
checking the pool accounting after every operation.  It is built here with
g++ for the host only (the manager has no device code) and must finish
without a sanitizer report.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_block_manager_clean_under_sanitizers(tmp_path):
    exe = tmp_path / "bm_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           f"-I{ROOT}/include", "-o", str(exe),
           os.path.join(ROOT, "tests", "bm_fuzz.cpp"),
           os.path.join(ROOT, "paged_kv_cache_309_amd", "csrc", "block_manager.cpp")]
    subprocess.run(cmd, check=True, capture_output=True, timeout=240)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(exe), "60"], capture_output=True, text=True, timeout=240,
                       env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout
