"""Address and undefined-behaviour sanitizer builds of the host-side C code
(CPU only): the oracle (oracle/oracle.c) and the C ABI's host code
(dense_ragged_grouped_amd/csrc/api.cpp, with its kernel launchers replaced by
stubs), each driven by a small program under tests/sanitize/ that exercises
every exported function on small, ragged, empty and invalid inputs.  A report
from either sanitizer fails the test.  Both are built with gcc / g++ (host
code only; no GPU code is built with a sanitizer)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g", "-O1"]
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def _run(exe, tmp):
    env = dict(os.environ, ASAN_OPTIONS="verify_asan_link_order=0:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="2")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, cwd=tmp, timeout=300)
    out = r.stdout + r.stderr
    assert r.returncode == 0 and "ok" in r.stdout, out[-4000:]
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    subprocess.run(["gcc", "-std=c99", *SAN, "-ffp-contract=off", "-fopenmp",
                    os.path.join(HERE, "oracle_driver.c"), os.path.join(ROOT, "oracle", "oracle.c"),
                    "-o", exe, "-lm"], check=True)
    _run(exe, tmp_path)


@pytest.mark.skipif(shutil.which("g++") is None or not os.path.exists(os.path.join(ROCM, "include", "hip")),
                    reason="needs g++ and the HIP headers")
def test_c_abi_host_code_under_sanitizers(tmp_path):
    exe = str(tmp_path / "abi_driver")
    csrc = os.path.join(ROOT, "dense_ragged_grouped_amd", "csrc")
    subprocess.run(["g++", "-std=c++17", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROCM, "include"),
                    "-I", os.path.join(ROOT, "include"), "-I", csrc,
                    os.path.join(HERE, "abi_driver.cpp"), os.path.join(csrc, "api.cpp"),
                    "-o", exe, "-L", os.path.join(ROCM, "lib"), f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
                    "-lamdhip64"], check=True)
    _run(exe, tmp_path)
