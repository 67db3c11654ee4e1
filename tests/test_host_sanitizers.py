"""The host side of the C ABI under AddressSanitizer and
UndefinedBehaviorSanitizer: tests/host/abi_sweep.cpp drives every entry point
over a grid of valid and invalid arguments and plans, with the kernel
launches replaced by counting stand-ins (tests/host/stub_launch.cpp).  Host
compiler only; no GPU code is built or run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rmsnorm_row_normalisation_amd", "csrc")
HOST = os.path.join(ROOT, "tests", "host")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.isdir(ROCM_INCLUDE),
                    reason="needs g++ and the HIP host headers")
def test_abi_sweep_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_sweep"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{ROCM_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           os.path.join(CSRC, "ks_api.cpp"), os.path.join(HOST, "stub_launch.cpp"), os.path.join(HOST, "abi_sweep.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600,
                         env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1",
                              "UBSAN_OPTIONS": "print_stacktrace=1"})
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "abi sweep:" in run.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_sweep_under_sanitizers(tmp_path):
    """Every oracle function over small shapes and arbitrary bit patterns, each
    buffer exactly the size the call needs."""
    exe = tmp_path / "oracle_sweep"
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", os.path.join(ROOT, "oracle", "ks_oracle.c"), os.path.join(HOST, "oracle_sweep.c"),
           "-lm", "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-3000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout[-2000:], run.stderr[-4000:])
    assert "oracle sweep:" in run.stdout
