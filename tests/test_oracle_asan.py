"""The C oracle (candidate build, loss and gradients) built with AddressSanitizer and
UndefinedBehaviorSanitizer on the CPU and driven through its branches by
tests/asan_oracle_main.c: the fallback, a wrapping window, P = V, P = 0, the asserted
conditions, labels out of range, and the loss and gradient helpers."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def test_oracle_under_address_sanitizer(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "asan_oracle")
    build = subprocess.run([gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer",
                            "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                            "-Wall", "-Wextra", "-o", exe, os.path.join(HERE, "asan_oracle_main.c"),
                            "-lm"], capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("no sanitizer runtime: " + build.stderr[-200:])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0 and run.stdout.strip() == "ok", run.stdout + run.stderr
