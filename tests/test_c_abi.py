"""libecho from plain C11 (tests/c_abi_check.c): the header compiles as C,
the library links without Python or torch, and -- on a GPU -- a C program
that owns its device memory reproduces the oracle bit for bit through the
fused, the phased and pipelined entry points, and the deferred-update
schedule with the correction array."""
import os
import shutil
import subprocess

import pytest

from error_compensated_bit_echo_amd import binding as B
from oracle import oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _build(tmp_path):
    if shutil.which("gcc") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("gcc or the HIP headers are not available")
    exe = tmp_path / "c_abi_check"
    lib_dir = os.path.dirname(B.LIB_PATH)
    orc_lib = orc._LIB_PATH
    cmd = ["gcc", "-std=c11", "-O1", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "oracle"),
           "-I", os.path.join(ROCM, "include"), os.path.join(ROOT, "tests", "c_abi_check.c"),
           "-o", str(exe), B.LIB_PATH, orc_lib, "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           f"-Wl,-rpath,{lib_dir}:{os.path.dirname(orc_lib)}:{os.path.join(ROCM, 'lib')}"]
    subprocess.run(cmd, check=True)
    return exe


def test_c_consumer_without_gpu(tmp_path):
    exe = _build(tmp_path)
    r = subprocess.run([str(exe), "cpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


@pytest.mark.gpu
def test_c_consumer_on_the_gpu(tmp_path):
    exe = _build(tmp_path)
    print("c_abi_check gpu: P=4 rank=1 n=2560, fused, phased, pipelined and deferred", flush=True)
    r = subprocess.run([str(exe), "gpu"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
