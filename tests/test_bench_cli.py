"""The benchmark's byte accounting and command line (CPU only).

The roofline's algorithmic bytes are the method's own: per element, x
(2 B), both averages read and written (16 B), y (2 B), and the 4-bit
messages (0.5 B of code + 4 B of scale per 128 elements) -- the send
message, P-1 incoming shards and the own stage-2 chunk per own element, the
P-1 gathered chunks per other element.  Summed over a call:
B(P) = 2 + 16 + 2 + 0.53125 (3P - 2) / P per element."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("P", [1, 2, 3, 4, 8, 16])
def test_call_bytes_per_element_closed_form(P):
    n = P * 128 * 1024
    want = 2 + 16 + 2 + 0.53125 * (3 * P - 2) / P
    assert abs(bench.step_bytes(n, P) / n - want) < 1e-12


def test_headline_figures():
    n = 1 << 29
    assert abs(bench.step_bytes(n, 8) / n - 21.4609375) < 1e-12
    assert int(bench.step_bytes(n, 8)) == 11521753088          # 11.52 GB per 1 GB call
    b = bench.bytes_per_element(8)
    assert abs(b["entry"] - 18.53125) < 1e-12 and abs(b["exit"] - 2.53125) < 1e-12
    assert abs(b["reduce"] - 24.25) < 1e-12
    # 8-bit codes: one byte per element instead of half a byte
    assert abs(bench.bytes_per_element(8, bits=8)["entry"] - 19.03125) < 1e-12


def test_reduce_scatter_bytes():
    n, P = 1 << 20, 8
    C = n // P
    code = 0.53125
    want = (n - C) * (2 + 16 + code) + C * (2 + 16 + code * (P - 1) + 2)
    assert abs(bench.rs_bytes(n, P) - want) < 1e-6


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "--gpus must be 1" in r.stderr
    assert r.stdout.strip() == ""


def test_step_counts_are_checked():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "0"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "--steps" in r.stderr


def test_serving_policy_only_for_serving_workloads():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--workload", "train",
                        "--serving-policy"], capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "serving" in r.stderr
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--message-sets", "0"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2 and "--message-sets" in r.stderr


def test_committed_traffic_profile_matches_the_kernel_sources():
    """The counted HBM traffic in profiles/ was taken on the kernels as they
    stand: the bench reports roofline.traffic only while the kernel and launch
    sources hash to the value recorded with the counters."""
    import bench

    for kernel in ("entry", "reduce", "exit"):
        t = bench.traffic_from_profile(kernel, "1gb")
        assert t is not None, f"profiles/traffic.json is stale for {kernel}: retake the HBM counters"
