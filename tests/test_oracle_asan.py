"""The oracle under AddressSanitizer, LeakSanitizer and UBSan (CPU only).

Builds the oracle sources and the multi-threaded driver together with
tests/oracle_asan_driver.c into one sanitized executable and runs it: the
one-thread and threaded encode and decode on small seeded inputs (both table
formats, ragged token counts) and the rejection of corrupt blobs must run
clean, with no out-of-bounds access, leak or undefined behaviour reported.
"""

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_runs_clean_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_asan")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=undefined", "-ffp-contract=off", "-pthread", "-I", ORACLE, "-o", exe,
           os.path.join(HERE, "oracle_asan_driver.c"), os.path.join(ORACLE, "cachegen_oracle.c"),
           os.path.join(ORACLE, "cachegen_oracle_mt.c"), "-lm"]
    subprocess.run(cmd, check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "Sanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert "ok" in r.stdout
