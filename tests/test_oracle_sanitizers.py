"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_driver.c calls every entry point of oracle/q8ref.c on
small and edge-case inputs (zero and subnormal blocks, ragged row counts,
row pitches, flat KV rows, partial attention blocks) with buffers of exactly
the sizes the entry points' contracts state.  Built with gcc (host code only;
the OpenMP pragmas are left out so that the sanitizers see one thread), any
out-of-bounds access, leak or undefined operation fails the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-Wno-unknown-pragmas",
           os.path.join(HERE, "oracle_sanitize_driver.c"), os.path.join(ROOT, "oracle", "q8ref.c"),
           "-lm", "-o", exe]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.startswith("ok"), r.stdout[-2000:] + r.stderr[-4000:]
    assert "runtime error" not in r.stderr, r.stderr[-4000:]
