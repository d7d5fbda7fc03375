"""The C oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host only) and driven over small ragged shapes by tests/sanitize/
oracle_driver.c: no out-of-bounds access, use after free, leak or
undefined behaviour, and the recurrences agree with the direct definition."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_address_and_ub_sanitizers(tmp_path):
    exe = tmp_path / "oracle_driver"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "attn_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"),
           "-o", str(exe), "-lm", "-lpthread"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all cases passed" in r.stdout
