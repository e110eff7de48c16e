"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

fa_api.cpp (every argument check of the boundary) is compiled for the host
with both sanitizers, linked with stand-in launchers that launch nothing
(tests/host_sanitizer/launch_stubs.cpp) and driven by a table of invalid,
empty, extreme and valid calls (tests/host_sanitizer/check_args.cpp).  Any
out-of-bounds access, signed overflow or other undefined behaviour in the
checks aborts the program; a wrong status code, or a launcher reached by an
invalid call (or missed by a valid one), fails it.  No GPU is used.
"""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HERE = os.path.join(ROOT, "tests", "host_sanitizer")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_c_abi_argument_checks_under_sanitizers(tmp_path):
    exe = str(tmp_path / "check_args")
    cmd = [HIPCC, "--offload-arch=gfx950", "-std=c++17", "-g", "-O1", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "exact_io_aware_16_amd", "csrc"),
           os.path.join(ROOT, "exact_io_aware_16_amd", "csrc", "fa_api.cpp"),
           os.path.join(HERE, "launch_stubs.cpp"), os.path.join(HERE, "check_args.cpp"), "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="halt_on_error=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert " 0 failed" in run.stdout, out[-4000:]
