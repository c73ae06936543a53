"""The C-ABI front end (api.cpp and the host-side kernel selection) built
for the host alone with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, no device code; the kernel launchers are stubs that abort if reached),
and the host ABI tests run against that build in a child process with the
sanitizer runtime preloaded. CPU only."""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_quantized_qblk_amd", "csrc")


def _asan_runtime(gxx):
    r = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_under_address_sanitizer(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the ROCm headers")
    libasan = _asan_runtime(gxx)
    if libasan is None:
        pytest.skip("no AddressSanitizer runtime for g++")
    so = str(tmp_path / "libqblk_host_asan.so")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fvisibility=hidden",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
           "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"),
           "-I", CSRC, os.path.join(CSRC, "api.cpp"), os.path.join(CSRC, "gemv_select.cpp"),
           os.path.join(ROOT, "tests", "asan", "launch_stubs.cpp"), "-o", so]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, LD_PRELOAD=libasan, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    code = ("import sys; sys.path.insert(0, %r)\n"
            "from block_quantized_qblk_amd import qblk\n"
            "qblk.LIB_PATH = %r\n"
            "import pytest\n"
            "sys.exit(pytest.main(['-q', '-p', 'no:cacheprovider', '-m', 'not gpu', "
            "'tests/test_abi_host.py']))\n") % (ROOT, so)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "passed" in r.stdout and "ERROR: AddressSanitizer" not in out, out
