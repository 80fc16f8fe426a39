"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven over small problems of every kind by
oracle/sanitize_main.c: no out-of-bounds access, leak or undefined
behaviour in the checker itself."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    src = [os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(ROOT, "oracle", "sanitize_main.c")]
    build = subprocess.run(["gcc", "-std=c99", "-g", "-O1", "-fsanitize=address,undefined",
                            "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-Wall", "-Wno-unknown-pragmas",
                            "-o", exe, *src, "-lm"], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr
