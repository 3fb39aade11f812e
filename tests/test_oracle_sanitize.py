"""The C oracle built with gcc's AddressSanitizer and
UndefinedBehaviorSanitizer and driven through its index-heavy cases (packed,
empty and one-token documents, unequal head sizes, ragged chunk snapshots,
every prologue flag, null optional pointers, rejected arguments, two OpenMP
threads) by ``tests/oracle_sanitize_main.c``: no out-of-bounds access,
leak or undefined behaviour may be reported, and the scalar hand-computed
trajectory must still come out.  CPU only."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    exe = tmp_path / "oracle_sanitize"
    cmd = ["gcc", "-std=c11", "-g", "-O1", "-fno-omit-frame-pointer", "-fopenmp",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "tests", "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "kda_oracle.c"),
           "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: the environment may preload a library ahead
    # of the sanitizer runtime, which is harmless for these checks
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ORACLE_SANITIZE_PASS" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
