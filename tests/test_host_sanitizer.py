"""Host code of libfa under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds a copy of the library (in a temporary directory) whose host code is
instrumented (``-Xarch_host`` puts each sanitizer on the host pass only; the
device code is built as usual) and runs tests/sanitize/api_driver.c against it:
descriptor validation, workspace planning, the alias and workspace checks of
every entry point and the host-only helpers, none of which makes a HIP call.
A sanitizer report or a wrong status fails the test.  CPU only (no GPU).
"""
import os
import shutil
import subprocess

import pytest

from long_context_decode_fourier_amd import build as fb_build

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "sanitize", "api_driver.c")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


@pytest.mark.skipif(not (shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")),
                    reason="hipcc not available")
def test_api_host_code_under_sanitizers(tmp_path):
    lib = str(tmp_path / "libfa.so")
    cmd = fb_build.command(lib)
    cmd = cmd[:1] + HOST_SAN + cmd[1:]
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-3000:]
    exe = str(tmp_path / "api_driver")
    link = [fb_build.hipcc(), "-O1", "-g", "-x", "c", DRIVER, "-x", "none", "-I", fb_build.INCLUDE,
            "-o", exe, lib, "-Wl,-rpath," + str(tmp_path), "-Wl,-rpath,/opt/rocm/lib",
            "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    res = subprocess.run(link, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert res.returncode == 0, res.stdout[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         env=env, timeout=120)
    assert run.returncode == 0, run.stdout[-3000:]
    assert "all checks passed" in run.stdout
    assert "runtime error" not in run.stdout and "AddressSanitizer" not in run.stdout
