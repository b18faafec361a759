"""Host sanitizer leg: the C ABI's argument validation (csrc/validate.h,
pure integer host code) built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer and driven through every LTXA_E_* path by
tests/host/validate_check.cpp.  No GPU and no HIP are involved."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "validate_check.cpp")
GXX = shutil.which("g++")


def _build(tmp_path, name, extra=()):
    exe = str(tmp_path / name)
    cmd = [GXX, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Werror", *extra,
           "-I" + os.path.join(ROOT, "include"),
           "-I" + os.path.join(ROOT, "video_dit_sequence_amd", "csrc"), SRC, "-o", exe]
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    return exe


def _run(exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    return subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)


@pytest.mark.skipif(GXX is None, reason="g++ is not installed")
def test_validation_under_asan_ubsan(tmp_path):
    res = _run(_build(tmp_path, "validate_check"))
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr


@pytest.mark.skipif(GXX is None, reason="g++ is not installed")
def test_sanitizer_catches_a_short_host_array(tmp_path):
    # The same driver with a planted caller mistake (two max_pos values for a
    # three-axis call) must be stopped by AddressSanitizer: the leg is live.
    res = _run(_build(tmp_path, "validate_check_planted", ["-DLTXA_CHECK_PLANT_SHORT_ARRAY"]))
    assert res.returncode != 0
    assert "heap-buffer-overflow" in res.stderr
