"""Host code under the address and undefined-behaviour sanitizers (CPU only): the C ABI's
validation, dispatch and slot allocator (api.cpp against host stand-ins of the kernel
launchers, tests/sanitize/api_stub.cpp), and the fp64 C oracle on small shapes and edge
cases. Both are built with g++/gcc for the host alone; no GPU code is involved."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]


def _run(cmd, tmp_path):
    r = subprocess.run(cmd, cwd=tmp_path, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r.stdout


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not found")
def test_c_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "api_san")
    _run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
          os.path.join(ROOT, "state_space_model_ssm_amd", "csrc", "api.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "api_stub.cpp"),
          os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp"), "-o", exe], tmp_path)
    out = _run([exe], tmp_path)
    assert "api driver: ok" in out


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_san")
    _run(["gcc", "-std=gnu11", *SAN, "-ffp-contract=off", os.path.join(ROOT, "oracle", "ssm_oracle.c"),
          os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), "-o", exe, "-lm"], tmp_path)
    out = _run([exe], tmp_path)
    assert "oracle driver: ok" in out
