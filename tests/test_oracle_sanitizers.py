"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (host
gcc, no GPU code) and driven through every routine on small shapes, each buffer
allocated at exactly its layout's size (tests/oracle_sanitize_driver.c): no
out-of-bounds access, leak or undefined operation."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "tq_oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-lm", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip().endswith("ok"), r.stdout + r.stderr
