"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code, gcc): a C driver calls every oracle entry point on exact-size heap
buffers over ragged, one-step and empty shapes; any out-of-bounds access, leak
or undefined behaviour fails the run."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "asan_oracle")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-pthread",
           os.path.join(ROOT, "oracle", "ssd_oracle.c"), os.path.join(ROOT, "tests", "asan_oracle_driver.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr and "cannot find" in build.stderr:
        pytest.skip("sanitizer runtime libraries are not installed")
    assert build.returncode == 0, build.stderr
    # verify_asan_link_order=0: a library the environment preloads may come
    # before the ASan runtime; the driver itself is fully instrumented
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "oracle sanitizer run ok" in run.stdout
