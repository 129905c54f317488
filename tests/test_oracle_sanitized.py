"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer.

`oracle/sanitize_driver.c` calls every exported oracle function (codecs,
compression of every key format, scores, selections, token sets, attention,
the threaded per-query pipeline, and rejected arguments); here it is compiled
together with `oracle/qsa_oracle.c` under both sanitizers, with recovery off,
and run.  Any out-of-bounds access, leak or undefined operation fails the run.

CPU only (host code; gcc).
"""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ORACLE = os.path.join(os.path.dirname(HERE), "oracle")


def _sanitizers_available(tmp):
    probe = os.path.join(tmp, "probe.c")
    with open(probe, "w") as f:
        f.write("int main(void){return 0;}\n")
    r = subprocess.run(["gcc", "-fsanitize=address,undefined", probe, "-o", os.path.join(tmp, "probe")],
                       capture_output=True, text=True)
    return r.returncode == 0


def test_oracle_under_asan_and_ubsan():
    tmp = tempfile.mkdtemp(prefix="qsa_oracle_san_")
    try:
        if not _sanitizers_available(tmp):
            pytest.skip("gcc here has no AddressSanitizer / UndefinedBehaviorSanitizer runtime")
        exe = os.path.join(tmp, "oracle_san")
        cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off", "-fno-fast-math",
               "-fopenmp", "-std=c99", "-Wall", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
               os.path.join(ORACLE, "qsa_oracle.c"), os.path.join(ORACLE, "sanitize_driver.c"),
               "-o", exe, "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:halt_on_error=1:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="4")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, f"sanitized oracle failed:\n{r.stdout}\n{r.stderr[-4000:]}"
        assert "ok" in r.stdout
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
