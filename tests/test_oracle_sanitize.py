"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code, gcc): every entry point, both code widths, P = 1..16, with and without
compensation; rank mode, also through the threaded driver, must reproduce
the full simulation.  The threaded driver also runs under ThreadSanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-pthread", "-I", os.path.join(ROOT, "oracle"), os.path.join(ROOT, "oracle", "echo_oracle.c"),
           os.path.join(ROOT, "oracle", "echo_oracle_mt.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_threaded_oracle_clean_under_tsan(tmp_path):
    exe = tmp_path / "oracle_tsan"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
           "-fsanitize=thread", "-pthread", "-I", os.path.join(ROOT, "oracle"),
           os.path.join(ROOT, "oracle", "echo_oracle.c"), os.path.join(ROOT, "oracle", "echo_oracle_mt.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, TSAN_OPTIONS="halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ThreadSanitizer" not in r.stderr, r.stderr
    assert r.stdout.strip().endswith("ok")
