"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

tests/oracle_sanitize_driver.c calls every entry point of oracle/oracle.c on
small seeded problems, edge cases (empty rows, block sizes 1 / 4 / 16, slots
of -1, the last slot, no-op copies) and bad arguments; built together with
oracle.c with both sanitizers, any out-of-bounds access, use of freed memory,
leak, signed overflow or other undefined behaviour ends the run with a
report and a nonzero status.  The driver also checks results that hold by
construction (paged == contiguous, blockwise == plain, swap and FP8 codec
round trips)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c99", "-g", "-O1", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-o", str(exe), os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           os.path.join(ROOT, "oracle", "oracle.c"), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
