"""The host-side argument checks (fa_validate.h) built by an ordinary C++
compiler with AddressSanitizer and UndefinedBehaviorSanitizer, and run on
directed cases and a fuzz of extreme sizes and strides. No GPU, no HIP
runtime: the checks touch neither."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_validation_under_sanitizers(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no g++")
    exe = tmp_path / "validate_check"
    flags = ["-std=c++17", "-O1", "-g", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include",
             "-I" + os.path.join(ROOT, "include"), "-fno-sanitize-recover=all",
             "-fsanitize=address,undefined"]
    r = subprocess.run([gxx, *flags, "-o", str(exe),
                        os.path.join(ROOT, "tests", "host", "validate_check.cpp")],
                       capture_output=True, text=True)
    if r.returncode != 0 and "asan" in (r.stderr or "").lower():
        pytest.skip("sanitizer runtime not available: " + r.stderr[-300:])
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    print(r.stdout)
    assert r.returncode == 0 and r.stdout.strip().endswith("OK"), r.stdout + r.stderr
