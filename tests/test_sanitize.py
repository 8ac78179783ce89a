"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU:
the C ABI (argument checks, cache bookkeeping, decode planning: api.cpp and
plan.cpp) with the kernel launchers replaced by stand-ins that check the
parameters they are handed, and the fp64 oracle (swa_oracle.c), driven through
valid and invalid calls by tests/sanitize/sanitize_main.cpp.  Built with g++
and gcc only (no device code)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]


def test_host_code_under_asan_ubsan(tmp_path):
    gxx, gcc = shutil.which("g++"), shutil.which("gcc")
    if not gxx or not gcc:
        pytest.skip("needs g++ and gcc")
    inc = ["-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "sliding_window_sink_amd", "csrc")]
    oracle_o = str(tmp_path / "swa_oracle.o")
    subprocess.run([gcc, "-std=c99", *SAN, "-c", os.path.join(ROOT, "oracle", "swa_oracle.c"), "-o", oracle_o],
                   check=True, capture_output=True, text=True)
    exe = str(tmp_path / "swa_sanitize")
    srcs = [os.path.join(ROOT, "sliding_window_sink_amd", "csrc", f) for f in ("api.cpp", "plan.cpp")] + \
           [os.path.join(ROOT, "tests", "sanitize", f) for f in ("stub_launch.cpp", "sanitize_main.cpp")]
    res = subprocess.run([gxx, "-std=c++17", *SAN, *inc, *srcs, oracle_o, "-lpthread", "-lm", "-o", exe],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert run.returncode == 0 and "sanitize ok" in run.stdout, (run.stdout[-2000:], run.stderr[-4000:])
