"""Grid sizes of every launch stay within HIP's per-dimension limit at the
largest sizes the header allows (host arithmetic only, compiled with g++;
no GPU and no launch)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_launch_shapes_within_limits(tmp_path):
    exe = str(tmp_path / "launch_shape_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-Wall", "-Werror",
                    "-I", os.path.join(ROOT, "include"),
                    "-I", os.path.join(ROOT, "error_compensated_bit_echo_amd", "csrc"),
                    os.path.join(ROOT, "tests", "launch_shape_check.cc"), "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    assert "launch shapes ok" in r.stdout
