"""The host side of the C ABI (argument checks, byte accounting, launch
planning: tq_api.cpp, tq_codebook.cpp, tq_plan.cpp) built with g++ under
AddressSanitizer and UndefinedBehaviorSanitizer, linked against stand-in
launchers that touch the first and last byte of every buffer extent a kernel
would access, and driven through every entry point of include/tq.h with valid
and invalid arguments (tests/host_sanitize/driver.cpp).  No GPU and no HIP
runtime are involved: the kernels are replaced, the checks and offsets are the
library's own."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_kv_decode_tq_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
HIP_INCLUDE = "/opt/rocm/include"

SOURCES = [os.path.join(CSRC, s) for s in ("tq_api.cpp", "tq_codebook.cpp", "tq_plan.cpp")] + \
          [os.path.join(HERE, s) for s in ("stub_launch.cpp", "driver.cpp")]


def _build(tmp_path) -> str:
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir(os.path.join(HIP_INCLUDE, "hip")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "tq_host_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{HIP_INCLUDE}", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           f"-I{HERE}", *SOURCES, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower() and "cannot find" in r.stderr.lower():
        pytest.skip("the sanitizer runtimes are not installed")
    assert r.returncode == 0, r.stderr[-4000:]
    return exe


def test_host_abi_under_sanitizers(tmp_path):
    exe = _build(tmp_path)
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=23"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    log = (r.stdout + r.stderr)[-6000:]
    assert "AddressSanitizer" not in log and "runtime error" not in log, log
    assert r.returncode == 0, log
    assert "host ABI checks:" in r.stdout and "passed" in r.stdout, log
