"""The library's host-only code (the codebook derivation) built with g++ under
the address and undefined-behaviour sanitizers and exercised over subspace
widths 2..64, both codebook readings and the invalid-argument paths.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_codebook_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "codebook_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "host", "codebook_check.cpp"),
           os.path.join(ROOT, "kv_cache_top_amd", "csrc", "pk_codebook.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "passed" in r.stdout
