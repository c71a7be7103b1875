"""The host-side C ABI code (plan, layout, header, pack / unpack) built with
g++ under AddressSanitizer and UndefinedBehaviorSanitizer and driven over
hundreds of valid and invalid shapes and parameters, with pack -> unpack round
trips and corrupted headers (CPU only; no HIP code is built here)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_code_under_asan_ubsan(tmp_path):
    exe = tmp_path / "host_checks"
    csrc = os.path.join(ROOT, "kv_cache_compression_snapkv_amd", "csrc")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "anchorkv_host.cpp"), os.path.join(ROOT, "tests", "asan", "host_checks.cpp"),
           "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
