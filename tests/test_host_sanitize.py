"""The host code of libtq (abi.cpp: argument checks, descriptors, splits,
dispatch; codebook.cpp: the Lloyd-Max builder) built with the host compiler
under AddressSanitizer and UndefinedBehaviorSanitizer, with the kernel
launchers replaced by stubs that report "no device", and driven through every
entry point (tests/host_sanitize/drive.py).  Any sanitizer report fails the
test.  No GPU is needed."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "compressed_decode_attention_append_amd", "csrc")
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer"]


def _runtime(name):
    out = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return out if os.path.isabs(out) and os.path.exists(out) else None


def test_host_code_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if not gxx or not asan or not ubsan or not os.path.exists("/opt/rocm/include/hip/hip_runtime.h"):
        pytest.skip("needs g++ with the sanitizer runtimes and the HIP headers")
    lib = str(tmp_path / "libtq_host_san.so")
    cmd = [gxx, "-std=c++17", "-shared", "-fPIC", "-g", "-O1", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC] + SAN + [
           os.path.join(CSRC, "abi.cpp"), os.path.join(CSRC, "codebook.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), "-o", lib]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-3000:]
    env = dict(os.environ, LD_PRELOAD=f"{asan}:{ubsan}", ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([sys.executable, os.path.join(HERE, "drive.py"), lib], capture_output=True, text=True,
                         env=env, timeout=600)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert "driven" in run.stdout
